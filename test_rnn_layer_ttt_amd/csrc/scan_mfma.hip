// Matrix-core chunk scan of the TTT-Linear recurrence for d = 64 (gfx950).
//
// Recurrence: "Edifice.Recurrent.TTT", "Equations (TTT-Linear)"; exact
// LayerNorm gradient: "Error Correction in Trained TTT Layers", abstract;
// chunk-start gradients: "PonderTTT", "Technical Architecture" (dual form).
//
// The sequence is cut into tiles of 16 tokens.  With W_c the weight at the
// start of a tile, E_s = eta_s delta_s and k_s.k_t the key Gram matrix, the
// per-token recurrence is, exactly,
//
//   z_t = W_c k_t - sum_{s<t in tile} eta_s (k_s.k_t) delta_s      (gradient point)
//   o_t = W_c q_t - sum_{s<=t in tile} eta_s (k_s.q_t) delta_s     (= W_t q_t)
//   W_{c+1} = W_c - sum_s eta_s delta_s k_s^T
//
// so every d x d product is a dense tile contraction (K W_c^T, Q W_c^T, K K^T,
// K Q^T, the output correction and the rank-16 update) and runs on MFMA; the
// only serial part left is, per token, the d-vector correction, the LayerNorm
// statistics and delta (one wave, 64 lanes = 64 rows, DPP + permlane
// reductions).  The dual form drops the in-tile correction of z_t (tile =
// chunk = 16), which makes the 16 tokens of a tile independent.
//
// Precision: W is kept in fp32 as MFMA accumulators.  With bf16 inputs every
// product runs as bf16 MFMA with fp32 accumulation; the fp32 operands (W,
// delta, the eta-scaled Gram entries) are split into bf16 hi + lo parts, so
// only the lo*lo term (~2^-17 relative) is dropped.  With fp32 inputs the
// products run as fp32 MFMA (16x16x4).
//
// Work split: 4 waves; wave w owns rows 16w..16w+15 of W (as W^T tiles in the
// 16x16 accumulator layout: lane l holds W[16w + l%16][16jt + 4(l/16) + r]).
// Wave 0 also runs the serial part.  Per tile: (A) all waves form their
// 16-column slices of K W^T and Q W^T; (B) the serial LayerNorm pass; (C) all
// waves apply the output correction, gate, store, and update their W rows.
#include "scan_common.h"

#include <type_traits>

namespace ttt {
namespace {

constexpr int D = 64;
constexpr int BT = 16;      // tokens per tile
constexpr int NT = 256;     // 4 waves
constexpr int KPAD = 68;    // padded fp32 row (floats) of K/Q tiles in LDS
constexpr int ZPAD = 20;    // padded row (floats) of the per-feature z / delta tiles

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float fast_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ unsigned short bf16_bits(float x) {
  const __bf16 b = static_cast<__bf16>(x);
  return __builtin_bit_cast(unsigned short, b);
}
__device__ __forceinline__ float bf16_val(unsigned short b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// x = hi + lo with hi, lo bf16 (round to nearest even each)
__device__ __forceinline__ void split_bf16(float x, unsigned short& hi, unsigned short& lo) {
  hi = bf16_bits(x);
  lo = bf16_bits(x - bf16_val(hi));
}

__device__ __forceinline__ f32x4 mfma_k32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_k16(const i16x4& a, const i16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_k4(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// LDS layout of one staged tile
// ---------------------------------------------------------------------------
// bf16 inputs: K and Q rows in the operand layout of the 16x16x32 MFMA
// (lane l = t + 16G holds, in slot e, column j = 32ks + 16(e/4) + 4G + e%4 of
// row t), K^T in the A layout of the 16x16x16 MFMA (lane l = j%16 + 16G of
// column tile jt holds rows s = 4G + e of column j), v transposed to
// feature-major rows for the serial pass, and the raw gate logits.
struct TileBf16 {
  uint16_t KA[2][64][8];
  uint16_t QA[2][64][8];
  uint16_t KT[4][64][4];
  uint16_t Vt[D][24];      // v[t][i] at Vt[i][t] (rows padded to 48 bytes)
  uint16_t Gl[BT][D];
  float ETA[BT];           // sigmoid(eta_logit)/d, 0 for tokens past the end
};
// fp32 inputs: K and Q rows (padded against bank conflicts), v transposed.
struct TileF32 {
  float K[BT][KPAD];
  float Q[BT][KPAD];
  float Vt[D][ZPAD];
  float Gl[BT][D];
  float ETA[BT];
};

// Tiles per staged batch: 32 KB of input per batch for either element type,
// so that one batch in flight per CU covers the HBM latency.
template <bool BF16>
struct Cfg {
  static constexpr int kTiles = BF16 ? 4 : 2;
  static constexpr int kTokens = kTiles * BT;
  static constexpr int kVE = BF16 ? 8 : 4;                    // elements per 16-byte vector
  static constexpr int kVecPerArr = kTokens * D / kVE;         // 16-byte vectors per array
  static constexpr int kPerThread = 4 * kVecPerArr / NT;       // q, k, v, gate
};

template <bool BF16>
struct Smem {
  using Tile = typename std::conditional<BF16, TileBf16, TileF32>::type;
  Tile tile[2][Cfg<BF16>::kTiles];
  float Zt[D][ZPAD];  // z_t (gradient points) of the tile, by feature i (padded rows)
  float Dt[D][ZPAD];  // delta_t of the tile, by feature i (padded rows)
  float Cc[BT][BT];   // eta_s (k_s . k_t)
  float O[Cfg<BF16>::kTokens][KPAD];   // gated outputs of the batch, written back at its end
};

template <bool BF16>
struct Prefetch {
  uint4 v[Cfg<BF16>::kPerThread];
  uint32_t eta;   // raw bits (bf16 in the low half, or fp32)
};

// Issue the global loads of one batch (tokens t0 .. t0 + kTokens - 1).  The
// array loop is unrolled, so each load's base pointer is a kernel argument and
// the loads issue as global loads (counted by vmcnt only, not lgkmcnt).
template <bool BF16>
__device__ __forceinline__ void load_batch(Prefetch<BF16>& p, const void* const src[4],
                                           const void* etap, int64_t bhT, int64_t t0, int64_t T,
                                           int tid) {
  using In = typename std::conditional<BF16, uint16_t, float>::type;
  using C = Cfg<BF16>;
  constexpr int kPerArr = C::kPerThread / 4;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const In* base = static_cast<const In*>(src[a]) + (bhT + t0) * D;
#pragma unroll
    for (int r = 0; r < kPerArr; ++r) {
      const int vid = tid + r * NT;
      const int t = (vid * C::kVE) / D;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (t0 + t < T) x = *reinterpret_cast<const uint4*>(base + vid * C::kVE);
      p.v[a * kPerArr + r] = x;
    }
  }
  p.eta = 0u;
  if (tid < C::kTokens && t0 + tid < T) {
    const In* e = static_cast<const In*>(etap) + bhT + t0 + tid;
    if constexpr (BF16)
      p.eta = *e;
    else
      p.eta = __float_as_uint(*e);
  }
}

// Write a loaded batch into its LDS tiles, in the layouts above.
template <bool BF16>
__device__ __forceinline__ void store_batch(const Prefetch<BF16>& p,
                                            typename Smem<BF16>::Tile* tiles, int64_t t0,
                                            int64_t T, int tid) {
  using C = Cfg<BF16>;
  constexpr int kPerArr = C::kPerThread / 4;
#pragma unroll
  for (int r = 0; r < C::kPerThread; ++r) {
    const int a = r / kPerArr;              // q, k, v, gate
    const int vid = tid + (r % kPerArr) * NT;
    const int tb = (vid * C::kVE) / D;      // token within the batch
    const int t = tb % BT;                  // token within its tile
    const int j0 = (vid * C::kVE) % D;
    auto& tl = tiles[tb / BT];
    const uint4 x = p.v[r];
    if constexpr (BF16) {
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
      if (a <= 1) {
        // rows of q (a=0) or k (a=1) into the 16x16x32 operand layout
        uint16_t(*dst)[64][8] = (a == 0) ? tl.QA : tl.KA;
        const int ks = j0 / 32, hh = (j0 % 32) / 16, g = (j0 % 16) / 4;
        *reinterpret_cast<uint2*>(&dst[ks][t + 16 * g][4 * hh]) = make_uint2(w[0], w[1]);
        *reinterpret_cast<uint2*>(&dst[ks][t + 16 * (g + 1)][4 * hh]) = make_uint2(w[2], w[3]);
      }
      if (a == 1 || a == 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = j0 + e;
          const uint16_t bits = (e & 1) ? static_cast<uint16_t>(w[e / 2] >> 16)
                                        : static_cast<uint16_t>(w[e / 2] & 0xFFFFu);
          if (a == 1)
            tl.KT[j / 16][(j % 16) + 16 * (t / 4)][t % 4] = bits;
          else
            tl.Vt[j][t] = bits;
        }
      }
      if (a == 3) *reinterpret_cast<uint4*>(&tl.Gl[t][j0]) = x;
    } else {
      const float4 f = make_float4(__uint_as_float(x.x), __uint_as_float(x.y),
                                   __uint_as_float(x.z), __uint_as_float(x.w));
      if (a == 0) *reinterpret_cast<float4*>(&tl.Q[t][j0]) = f;
      if (a == 1) *reinterpret_cast<float4*>(&tl.K[t][j0]) = f;
      if (a == 2) {
        tl.Vt[j0][t] = f.x;
        tl.Vt[j0 + 1][t] = f.y;
        tl.Vt[j0 + 2][t] = f.z;
        tl.Vt[j0 + 3][t] = f.w;
      }
      if (a == 3) *reinterpret_cast<float4*>(&tl.Gl[t][j0]) = f;
    }
  }
  if (tid < C::kTokens) {
    const float x = BF16 ? __uint_as_float(p.eta << 16) : __uint_as_float(p.eta);
    tiles[tid / BT].ETA[tid % BT] = (t0 + tid < T) ? fast_sigmoid(x) * (1.0f / D) : 0.0f;
  }
}

// Step K of a sum over the 64 lanes of a wave: an inclusive scan inside each
// 16-lane row (row_shr 1, 2, 4, 8; out-of-row sources add zero), then
// row_bcast:15 and row_bcast:31.  After the six steps lane 63 holds the total
// (rows 1 and 3 pick up the rows below them, then rows 2 and 3 pick up lane
// 31); the other lanes hold partial sums that are never read.
template <int K>
__device__ __forceinline__ float red_step(float x) {
  constexpr int kCtrl[6] = {0x111, 0x112, 0x114, 0x118, 0x142, 0x143};
  return x + __int_as_float(
                 __builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl[K], 0xF, 0xF, true));
}
__device__ __forceinline__ float lane63(float x) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// Two independent wave sums, interleaved step by step; wave-uniform results.
__device__ __forceinline__ void wave_total2(float& a, float& b) {
  a = red_step<0>(a); b = red_step<0>(b);
  a = red_step<1>(a); b = red_step<1>(b);
  a = red_step<2>(a); b = red_step<2>(b);
  a = red_step<3>(a); b = red_step<3>(b);
  a = red_step<4>(a); b = red_step<4>(b);
  a = red_step<5>(a); b = red_step<5>(b);
  a = lane63(a);
  b = lane63(b);
}

// delta for one token from z (lane = feature i) and the wave sums s1 = sum z,
// s2 = sum z^2; bv = beta_i - v_t[i].  mu = s1/d, d*var = s2 - s1*mu.
template <int LN>
__device__ __forceinline__ float delta_from_sums(float z, float s1, float s2, float bv, float gam,
                                                 float eps) {
  const float mu = s1 * (1.0f / D);
  const float dvar = fmaf(-s1, mu, s2);
  const float rs = __builtin_amdgcn_rsqf(fmaxf(fmaf(dvar, 1.0f / D, eps), eps));
  const float zc = z - mu;
  if constexpr (LN == kLnST) {
    return fmaf(gam * rs, zc, bv);
  } else {
    const float xh = zc * rs;
    const float g = gam * fmaf(gam, xh, bv);
    float sg = g, sgx = g * xh;
    wave_total2(sg, sgx);
    return rs * (g - sg * (1.0f / D) - xh * (sgx * (1.0f / D)));
  }
}

// delta for one token from z (lane = feature i); bv = beta_i - v_t[i].
template <int LN>
__device__ __forceinline__ float token_delta(float z, float v, float bv, float gam, float eps) {
  if constexpr (LN == kLnNone) {
    return z - v;
  } else {
    float s1 = z, s2 = z * z;
    wave_total2(s1, s2);
    return delta_from_sums<LN>(z, s1, s2, bv, gam, eps);
  }
}

// The serial pass over one tile (lane = feature i).  zr[t] = (W_c k_t)_i on
// entry; cc points at eta_s (k_s . k_t) in LDS.  Token s's delta is applied to
// row s+1 at once; its updates of rows s+2.. are spread over the reduction
// steps of token s+1, where they fill the DPP wait states.
template <int LN>
__device__ __forceinline__ void serial_tile(float (&zr)[BT], const float (&bv)[BT],
                                            const float (&vv)[BT], const float (*cc)[BT],
                                            float gam, float eps, float (&dr)[BT]) {
  float cprev[BT];
  float dprev = 0.0f;
#pragma unroll
  for (int s = 0; s < BT; ++s) {
    float crow[BT];
#pragma unroll
    for (int q4 = (s + 1) / 4; q4 < BT / 4; ++q4) {
      const float4 x = *reinterpret_cast<const float4*>(&cc[s][4 * q4]);
      crow[4 * q4] = x.x; crow[4 * q4 + 1] = x.y; crow[4 * q4 + 2] = x.z; crow[4 * q4 + 3] = x.w;
    }
    const float z = zr[s];
    // deferred rows s+1 .. BT-1 of the previous token, split into six slices
    constexpr int kSlots = 6;
    const int n = BT - 1 - s;
    auto fill = [&](int k) {
      if (s == 0) return;
#pragma unroll
      for (int t = s + 1 + (k * n) / kSlots; t < s + 1 + ((k + 1) * n) / kSlots; ++t)
        zr[t] = fmaf(-cprev[t], dprev, zr[t]);
    };
    float dl;
    if constexpr (LN == kLnNone) {
#pragma unroll
      for (int k = 0; k < kSlots; ++k) fill(k);
      dl = z - vv[s];
    } else {
      float a = z, b = z * z;
      a = red_step<0>(a); b = red_step<0>(b); fill(0);
      a = red_step<1>(a); b = red_step<1>(b); fill(1);
      a = red_step<2>(a); b = red_step<2>(b); fill(2);
      a = red_step<3>(a); b = red_step<3>(b); fill(3);
      a = red_step<4>(a); b = red_step<4>(b); fill(4);
      a = red_step<5>(a); b = red_step<5>(b); fill(5);
      dl = delta_from_sums<LN>(z, lane63(a), lane63(b), bv[s], gam, eps);
    }
    dr[s] = dl;
    if (s + 1 < BT) zr[s + 1] = fmaf(-crow[s + 1], dl, zr[s + 1]);
#pragma unroll
    for (int t = s + 2; t < BT; ++t) cprev[t] = crow[t];
    dprev = dl;
  }
}

template <bool BF16>
__device__ __forceinline__ void read_v16(const typename Smem<BF16>::Tile& tl, int lane, float* v) {
  if constexpr (BF16) {
    const uint4 a = *reinterpret_cast<const uint4*>(&tl.Vt[lane][0]);
    const uint4 b = *reinterpret_cast<const uint4*>(&tl.Vt[lane][8]);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 x = *reinterpret_cast<const float4*>(&tl.Vt[lane][4 * q4]);
      v[4 * q4] = x.x; v[4 * q4 + 1] = x.y; v[4 * q4 + 2] = x.z; v[4 * q4 + 3] = x.w;
    }
  }
}

template <bool BF16>
__device__ __forceinline__ float gate_logit(const typename Smem<BF16>::Tile& tl, int t, int i) {
  if constexpr (BF16)
    return __uint_as_float(static_cast<uint32_t>(tl.Gl[t][i]) << 16);
  else
    return tl.Gl[t][i];
}

template <bool BF16, int LN, bool DUAL>
__global__ void __launch_bounds__(NT)
scan_mfma_kernel(const void* __restrict__ qp, const void* __restrict__ kp,
                 const void* __restrict__ vp, const void* __restrict__ etap,
                 const void* __restrict__ gatep, const float* __restrict__ W0,
                 const float* __restrict__ gamma, const float* __restrict__ beta,
                 float* __restrict__ out, float* __restrict__ W_final, int H, int64_t T,
                 float eps) {
  using C = Cfg<BF16>;
  __shared__ Smem<BF16> sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int G = lane >> 4;
  const int64_t bh = blockIdx.x;
  const int h = static_cast<int>(bh % H);
  const int64_t bhT = bh * T;
  const void* const src[4] = {qp, kp, vp, gatep};
  const int irow = 16 * wave + l16;   // the W row (feature i) this lane's accumulators hold

  // W^T tiles: Wt[jt][r] = W[irow][16 jt + 4G + r]
  f32x4 Wt[4];
  {
    const float* w = W0 + bh * D * D + irow * D + 4 * G;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      const float4 x = *reinterpret_cast<const float4*>(w + 16 * jt);
      Wt[jt] = f32x4{x.x, x.y, x.z, x.w};
    }
  }
  float gam = 1.0f, bet = 0.0f;   // LayerNorm affine of feature `lane` (serial part)
  if constexpr (LN != kLnNone) {
    gam = gamma[h * D + lane];
    bet = beta[h * D + lane];
  }

  const int64_t ntiles = (T + BT - 1) / BT;
  const int64_t nbatches = (T + C::kTokens - 1) / C::kTokens;
  // Pipeline: LDS holds the current batch and (from the end of the previous
  // batch) the next one; the registers of `pf` hold the batch after that, in
  // flight.  All global loads are issued right after a batch boundary, next to
  // the output stores, so the single wait per batch (before store_batch) finds
  // them a whole batch old.
  // W0, gamma and beta have landed before the first input load is issued, so
  // no use of them inside the loop waits on an in-flight batch.
  __builtin_amdgcn_s_waitcnt(0);
  Prefetch<BF16> pf;
  if (nbatches > 0) {
    load_batch<BF16>(pf, src, etap, bhT, 0, T, tid);
    store_batch<BF16>(pf, sm.tile[0], 0, T, tid);
  }
  if (nbatches > 1) load_batch<BF16>(pf, src, etap, bhT, C::kTokens, T, tid);
  __syncthreads();

  for (int64_t b = 0; b < nbatches; ++b) {
    const int64_t tb0 = b * C::kTokens;
    const int ntb = static_cast<int>(min<int64_t>(C::kTiles, ntiles - b * C::kTiles));
    for (int ct = 0; ct < ntb; ++ct) {
      const int64_t t0 = tb0 + ct * BT;
      const auto& tl = sm.tile[b & 1][ct];

      // ---------------- (A) Z = K W^T, U = Q W^T, Gram matrices ----------------
      f32x4 Z = {0, 0, 0, 0}, U = {0, 0, 0, 0}, KQ = {0, 0, 0, 0}, KK = {0, 0, 0, 0};
      if constexpr (BF16) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8 bh_, bl_;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            unsigned short hi, lo;
            split_bf16(Wt[2 * ks + e / 4][e % 4], hi, lo);
            bh_[e] = __builtin_bit_cast(__bf16, hi);
            bl_[e] = __builtin_bit_cast(__bf16, lo);
          }
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&tl.KA[ks][lane][0]);
          const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&tl.QA[ks][lane][0]);
          Z = mfma_k32(ka, bh_, Z);
          U = mfma_k32(qa, bh_, U);
          Z = mfma_k32(ka, bl_, Z);
          U = mfma_k32(qa, bl_, U);
          KQ = mfma_k32(ka, qa, KQ);
          if (!DUAL && wave == 0) KK = mfma_k32(ka, ka, KK);
        }
      } else {
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          const float4 ka = *reinterpret_cast<const float4*>(&tl.K[l16][16 * jt + 4 * G]);
          const float4 qa = *reinterpret_cast<const float4*>(&tl.Q[l16][16 * jt + 4 * G]);
          const float kv[4] = {ka.x, ka.y, ka.z, ka.w};
          const float qv[4] = {qa.x, qa.y, qa.z, qa.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            Z = mfma_k4(kv[r], Wt[jt][r], Z);
            U = mfma_k4(qv[r], Wt[jt][r], U);
            KQ = mfma_k4(kv[r], qv[r], KQ);
            if (!DUAL && wave == 0) KK = mfma_k4(kv[r], kv[r], KK);
          }
        }
      }
      // Z[t = 4G + r][i = irow] -> Zt[i][t]
      *reinterpret_cast<float4*>(&sm.Zt[irow][4 * G]) = make_float4(Z[0], Z[1], Z[2], Z[3]);
      // KQ[s = 4G + r][t = l16] -> eta_s-scaled, causal (s <= t): operand M[t][s]
      const float4 eta4 = *reinterpret_cast<const float4*>(&tl.ETA[4 * G]);   // eta_{4G+r}
      const float etav[4] = {eta4.x, eta4.y, eta4.z, eta4.w};
      float M[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) M[r] = (4 * G + r <= l16) ? etav[r] * KQ[r] : 0.0f;
      if (!DUAL && wave == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.Cc[4 * G + r][l16] = etav[r] * KK[r];
      }
      __syncthreads();

      // ---------------- (B) serial LayerNorm pass -> delta ----------------
      if constexpr (!DUAL) {
        if (wave == 0) {
          float zr[BT], dr[BT], vv[BT];
#pragma unroll
          for (int q4 = 0; q4 < BT / 4; ++q4) {
            const float4 x = *reinterpret_cast<const float4*>(&sm.Zt[lane][4 * q4]);
            zr[4 * q4] = x.x; zr[4 * q4 + 1] = x.y; zr[4 * q4 + 2] = x.z; zr[4 * q4 + 3] = x.w;
          }
          read_v16<BF16>(tl, lane, vv);
          float bv[BT];
#pragma unroll
          for (int t = 0; t < BT; ++t) bv[t] = bet - vv[t];
          serial_tile<LN>(zr, bv, vv, sm.Cc, gam, eps, dr);
#pragma unroll
          for (int q4 = 0; q4 < BT / 4; ++q4)
            *reinterpret_cast<float4*>(&sm.Dt[lane][4 * q4]) =
                make_float4(dr[4 * q4], dr[4 * q4 + 1], dr[4 * q4 + 2], dr[4 * q4 + 3]);
        }
      } else {
        // dual form: the 16 tokens are independent; wave w takes tokens 4w..4w+3
        const float4 x = *reinterpret_cast<const float4*>(&sm.Zt[lane][4 * wave]);
        float vv[BT];
        read_v16<BF16>(tl, lane, vv);
        const float zz[4] = {x.x, x.y, x.z, x.w};
        float dd[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float v = vv[4 * wave + u];
          dd[u] = token_delta<LN>(zz[u], v, bet - v, gam, eps);
        }
        *reinterpret_cast<float4*>(&sm.Dt[lane][4 * wave]) =
            make_float4(dd[0], dd[1], dd[2], dd[3]);
      }
      __syncthreads();

      // ---------------- (C) outputs and the W update ----------------
      const float4 dv4 = *reinterpret_cast<const float4*>(&sm.Dt[irow][4 * G]);
      const float dv[4] = {dv4.x, dv4.y, dv4.z, dv4.w};   // delta[s = 4G + e][irow]
      float ev[4];                                          // eta_s delta[s][irow]
#pragma unroll
      for (int e = 0; e < 4; ++e) ev[e] = etav[e] * dv[e];
      if constexpr (BF16) {
        i16x4 mh, ml, dh, dlo, eh, el;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          unsigned short a, bb;
          split_bf16(-M[e], a, bb);
          mh[e] = static_cast<short>(a);
          ml[e] = static_cast<short>(bb);
          split_bf16(dv[e], a, bb);
          dh[e] = static_cast<short>(a);
          dlo[e] = static_cast<short>(bb);
          split_bf16(-ev[e], a, bb);
          eh[e] = static_cast<short>(a);
          el[e] = static_cast<short>(bb);
        }
        U = mfma_k16(mh, dh, U);
        U = mfma_k16(mh, dlo, U);
        U = mfma_k16(ml, dh, U);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          const i16x4 kt = *reinterpret_cast<const i16x4*>(&tl.KT[jt][lane][0]);
          Wt[jt] = mfma_k16(kt, eh, Wt[jt]);
          Wt[jt] = mfma_k16(kt, el, Wt[jt]);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) U = mfma_k4(-M[q], dv[q], U);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            Wt[jt] = mfma_k4(tl.K[4 * G + q][16 * jt + l16], -ev[q], Wt[jt]);
        }
      }
      // gate and stage: U[t = 4G + r][irow]
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * G + r;
        sm.O[ct * BT + t][irow] = U[r] * fast_sigmoid(gate_logit<BF16>(tl, t, irow));
      }
    }
    if (b + 1 < nbatches) store_batch<BF16>(pf, sm.tile[(b + 1) & 1], tb0 + C::kTokens, T, tid);
    __syncthreads();
    if (b + 2 < nbatches) load_batch<BF16>(pf, src, etap, bhT, tb0 + 2 * C::kTokens, T, tid);
    // write the batch's outputs back as 16-byte stores (rows past T skipped)
    {
      const int rows = static_cast<int>(min<int64_t>(C::kTokens, T - tb0));
      float* dst = out + (bhT + tb0) * D;
      for (int i = tid; i < rows * (D / 4); i += NT) {
        const int t = i / (D / 4), c4 = i % (D / 4);
        *reinterpret_cast<float4*>(dst + t * D + 4 * c4) =
            *reinterpret_cast<const float4*>(&sm.O[t][4 * c4]);
      }
    }
  }

  if (W_final != nullptr) {
    float* w = W_final + bh * D * D + irow * D + 4 * G;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
      *reinterpret_cast<float4*>(w + 16 * jt) = make_float4(Wt[jt][0], Wt[jt][1], Wt[jt][2], Wt[jt][3]);
  }
}

template <bool BF16, int LN, bool DUAL>
hipError_t launch_one(const ScanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((scan_mfma_kernel<BF16, LN, DUAL>), dim3(static_cast<unsigned>(a.B * a.H)),
                     dim3(NT), 0, s, a.q, a.k, a.v, a.eta_logit, a.gate_logit, a.W0, a.gamma,
                     a.beta, a.out, a.W_final, static_cast<int>(a.H), a.T, a.eps);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_ln(const ScanArgs& a, hipStream_t s) {
  if (a.dual) {
    switch (a.ln) {
      case kLnST: return launch_one<BF16, kLnST, true>(a, s);
      case kLnExact: return launch_one<BF16, kLnExact, true>(a, s);
      default: return launch_one<BF16, kLnNone, true>(a, s);
    }
  }
  switch (a.ln) {
    case kLnST: return launch_one<BF16, kLnST, false>(a, s);
    case kLnExact: return launch_one<BF16, kLnExact, false>(a, s);
    default: return launch_one<BF16, kLnNone, false>(a, s);
  }
}

}  // namespace

bool scan_mfma_supports(const ScanArgs& a) {
  return a.d == D && (!a.dual || a.chunk == BT);
}

hipError_t launch_scan_mfma(const ScanArgs& a, hipStream_t s) {
  if (!scan_mfma_supports(a)) return hipErrorNotSupported;
  return a.in_bf16 ? launch_ln<true>(a, s) : launch_ln<false>(a, s);
}

}  // namespace ttt
