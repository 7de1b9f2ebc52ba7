// Backward of the TTT-Linear scan for d = 64 (gfx950): the per-token scan,
// and the dual form with chunks of 16 tokens (the tiles below).
//
// Recurrence: "Edifice.Recurrent.TTT", "Equations (TTT-Linear)"; exact
// LayerNorm gradient: "Error Correction in Trained TTT Layers", abstract.  The
// gradients are those of a loss L through out and W_final: reverse-mode
// through every step of the forward.
//
// A recording forward stores delta_t and W at the start of every tile of 16
// tokens.  The tiles are walked backwards.  With W_c the weight at the start
// of tile c, E_s = eta_s delta_s, H the gradient with respect to the weight
// after the tile, dy_t = dout_t * sigmoid(g_t), and G_t the gradient with
// respect to W_t, the tile's algebra is (rows are tokens):
//
//   z_t  = W_c k_t - sum_{s<t} (k_s.k_t) E_s           (z of the forward)
//   y_t  = W_c q_t - sum_{s<=t} (q_t.k_s) E_s          (W_t q_t)
//   a_t  = G_t k_t = H k_t + sum_{t'>=t} (q_t'.k_t) dy_t' + sum_{t'>t} (k_t'.k_t) dz_t'
//   d delta_t = -eta_t a_t,  d eta_t = -delta_t . a_t,  dz_t = VJP of delta(z_t)
//   dk_t = -eta_t [H^T delta_t + sum_{t'>=t} (delta_t.dy_t') q_t' + sum_{t'>t} (delta_t.dz_t') k_t']
//          + W_c^T dz_t - sum_{s<t} eta_s (delta_s.dz_t) k_s
//   dq_t = W_c^T dy_t - sum_{s<=t} eta_s (delta_s.dy_t) k_s
//   H   <- H + sum_t dy_t q_t^T + sum_t dz_t k_t^T          (gradient before the tile)
//
// The dual form ("PonderTTT", dual-form chunk updates) takes every z of a tile
// at W_c: z_t = W_c k_t, so the two sums over dz inside the tile (in a_t and
// in dk_t) and the z correction drop out and the tokens' VJPs are independent;
// the terms that couple neighbouring tiles are unchanged.
//
// Two rewrites let the work of neighbouring tiles overlap.  (1) The part of
// a_t of tile c-1 that comes through H needs H before tile c, which is H
// after it plus tile c's rank-16 terms: K_{c-1} H^T + (K_{c-1} Q_c^T) DY_c +
// (K_{c-1} K_c^T) DZ_c; only the last term waits for tile c's chain.  (2)
// W_c = W_{c-1} - E_{c-1}^T K_{c-1}, so DZ_c W_c is formed from the one
// recorded W a period holds.
//
// One workgroup of 8 waves per (batch, head).  Period c (c = N .. 0; the
// virtual tile N has no tokens) has two phases separated by barriers:
//   A: wave 0 runs tile c's serial dz chain (lane = feature), then the Grams
//      delta_c . dz_c and dz_c . E_{c-1}; the matrix-core waves form tile
//      c-1's chain-independent products (K W^T, Q W^T, DY W, K H^T and its
//      Grams) and delta_c H for dk of tile c; waves 4 and 7 issue the loads
//      of tile c-2 and its W.
//   B: what needs the chain or the Grams: tile c-1's in-tile corrections
//      (z and its LayerNorm statistics, y -> dgate, dq, a0), tile c's
//      remaining dk terms, d eta and the H update; waves 4 and 7 store tile
//      c-2 and its W.
// Every contraction is an fp32 MFMA 16x16x4 with operands from LDS.  In a
// 64-deep contraction lane group G covers k = 16G..16G+15 (k-contiguous rows
// load as 128-bit LDS reads); in a 16-deep (token) one, k = 4G..4G+3.
#include "scan_common.h"

#include <type_traits>

namespace ttt {
namespace {

constexpr int D = 64;
constexpr int BT = 16;
constexpr int NWAVES = 8;
constexpr int NT = 64 * NWAVES;
constexpr int KP = 68;   // padded row of 64-wide matrices in LDS
constexpr int TP = 20;   // padded row of 16-wide token matrices

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float sigmoidf_(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 16-deep token contractions with bf16 operands (16x16x16 MFMA, lane group G
// holding k = 4G..4G+3, the k of mfma4's four steps): an fp32 operand is split
// into bf16 hi + lo (round to nearest each; |x - hi - lo| <= 2^-17 |x|), a
// bf16-exact one (the bf16 inputs q, k) is taken as is
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// two fp32 values to two bf16 (round to nearest even each) in one register,
// a in the low half: one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}
__device__ __forceinline__ void split4(const float (&x)[4], i16x4& hi, i16x4& lo) {
  const uint32_t h01 = pack_bf16(x[0], x[1]);
  const uint32_t h23 = pack_bf16(x[2], x[3]);
  const uint32_t l01 = pack_bf16(x[0] - __uint_as_float(h01 << 16),
                                 x[1] - __uint_as_float(h01 & 0xFFFF0000u));
  const uint32_t l23 = pack_bf16(x[2] - __uint_as_float(h23 << 16),
                                 x[3] - __uint_as_float(h23 & 0xFFFF0000u));
  hi = __builtin_bit_cast(i16x4, make_uint2(h01, h23));
  lo = __builtin_bit_cast(i16x4, make_uint2(l01, l23));
}
__device__ __forceinline__ i16x4 exact4(const float (&x)[4]) {
  i16x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = static_cast<short>(__float_as_uint(x[e]) >> 16);
  return r;
}
__device__ __forceinline__ f32x4 mfma16(const i16x4& a, const i16x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// ---- wave-wide sums (lane = feature): row scans, row broadcasts, lane 63 ----
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
#pragma clang fp contract(off)
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float rl63(float x) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
// N independent sums, interleaved step by step; wave-uniform results
template <int N>
__device__ __forceinline__ void wave_sums(float (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = dpp_add<0x111>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = dpp_add<0x112>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = dpp_add<0x114>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = dpp_add<0x118>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = dpp_add<0x142>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = dpp_add<0x143>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = rl63(x[i]);
}

// sum over the 16 lanes of a row, in every lane of it (rotations by 8, 4, 2, 1)
template <int CTRL>
__device__ __forceinline__ float ror_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x = ror_add<0x128>(x);
  x = ror_add<0x124>(x);
  x = ror_add<0x122>(x);
  return ror_add<0x121>(x);
}

// ---- LDS layout ----
struct alignas(16) TileIn {   // one tile of inputs (fp32); rows past the end are zero
  float Q[BT][KP], K[BT][KP], DY[BT][KP], De[BT][KP];
  float G2[BT][KP];           // dout sigmoid'(gate): dgate = y G2
  float ETA[BT], ELD[BT];     // eta_t, sigmoid'(eta_logit_t) / d
};
struct alignas(16) Work {     // a tile's working set around its chain
  float A[BT][KP];            // a0_t in, a_t out
  float X[BT][KP];            // xhat_t in (zero without LayerNorm), dz_t out
  float E[BT][KP];            // exact LayerNorm: e_t = gamma xhat_t + beta - v_t
  float S[BT][8];             // rs, mean g, mean g xhat, mean gamma^2 xhat, mean gamma^2 xhat^2
};
struct alignas(16) Grams {
  float KK[BT][TP], QK[BT][TP], DeDY[BT][TP];
};
struct alignas(16) BwdSmem {
  TileIn ring[3];
  float W[2][D][KP];          // recorded W at a tile start, [i][j]
  float Hm[D][KP];            // H, [i][j]
  Work wk[2];
  Grams gr[2];
  float XQ[BT][TP], XK[BT][TP], DeDZ[BT][TP], DZE[BT][TP];
  float B2[BT][KP];           // the W-side half of dk, handed to wave 3
};

// ---- MFMA operand fragments (lane group G, row or column l16) ----
// 64-deep: 16 consecutive k of a k-contiguous row
__device__ __forceinline__ void frag_row64(const float* row, int G, float (&v)[16]) {
  const float4* p = reinterpret_cast<const float4*>(row + 16 * G);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 x = p[q];
    v[4 * q] = x.x;
    v[4 * q + 1] = x.y;
    v[4 * q + 2] = x.z;
    v[4 * q + 3] = x.w;
  }
}
// 64-deep: column n of a k-major array
__device__ __forceinline__ void frag_col64(const float (*a)[KP], int n, int G, float (&v)[16]) {
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) v[ks] = a[16 * G + ks][n];
}
// 16-deep: 4 consecutive k of a k-contiguous row
__device__ __forceinline__ void frag_row16(const float* row, int G, float (&v)[4]) {
  const float4 x = *reinterpret_cast<const float4*>(row + 4 * G);
  v[0] = x.x;
  v[1] = x.y;
  v[2] = x.z;
  v[3] = x.w;
}
// 16-deep: column n of a k-major array
template <int P>
__device__ __forceinline__ void frag_col16(const float (*a)[P], int n, int G, float (&v)[4]) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) v[ks] = a[4 * G + ks][n];
}
template <int KS>
__device__ __forceinline__ f32x4 mma(const float (&a)[KS], const float (&b)[KS], f32x4 acc) {
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) acc = mfma4(a[ks], b[ks], acc);
  return acc;
}
// 16x16 Gram of two 16-row blocks of k-contiguous rows: G[m][n] = ra[m] . rb[n]
template <int P1, int P2>
__device__ __forceinline__ f32x4 gram(const float (*ra)[P1], const float (*rb)[P2], int l16,
                                      int G) {
  float a[16], b[16];
  frag_row64(ra[l16], G, a);
  frag_row64(rb[l16], G, b);
  return mma<16>(a, b, f32x4{0, 0, 0, 0});
}
// an MFMA output block: rows 4G + r, column col0 + l16
template <int P>
__device__ __forceinline__ void store_block(float (*o)[P], int col0, f32x4 v, int l16, int G) {
#pragma unroll
  for (int r = 0; r < 4; ++r) o[4 * G + r][col0 + l16] = v[r];
}

// The :mlp variant's SiLU on q and k, as the forward applies it: in fp32, and
// on the bf16-input path rounded back to bf16 (to nearest even), so that the
// backward differentiates the function the forward computed.
template <bool BF16>
__device__ __forceinline__ float silu_in(float x) {
  const float y = x * sigmoidf_(x);
  if constexpr (BF16) {
    const __bf16 b = static_cast<__bf16>(y);
    return __uint_as_float(static_cast<uint32_t>(__builtin_bit_cast(unsigned short, b)) << 16);
  } else {
    return y;
  }
}

template <bool BF16>
__device__ __forceinline__ float ld_in(const void* p, int64_t i) {
  if constexpr (BF16)
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
  else
    return static_cast<const float*>(p)[i];
}

// ---- state a wave keeps across a barrier ----
// The roles share one register array, so the kernel needs registers for the
// largest role rather than for all of them together:
//   waves 1, 5, 6: a 16x64 accumulator in [0, 16); waves 2 and 3: half of
//   DY W and dk's H-side half ([0, 8) and [16, 24); [8, 16) and [0, 8))
//   wave 1: v in [16, 32) (exact LayerNorm)
//   wave 4: a tile of inputs in flight (LoadLayout); wave 7: its W, [0, 64)
constexpr int kState = 80;
__device__ __forceinline__ f32x4 blk(const float (&st)[kState], int b) {
  return f32x4{st[4 * b], st[4 * b + 1], st[4 * b + 2], st[4 * b + 3]};
}
__device__ __forceinline__ void put(float (&st)[kState], int b, f32x4 v) {
  st[4 * b] = v[0];
  st[4 * b + 1] = v[1];
  st[4 * b + 2] = v[2];
  st[4 * b + 3] = v[3];
}

// wave 4's layout: lane -> token t = lane / 4, features 16 (lane % 4) .. +15.
// q, k, gate: 16 values (fp32) or 8 words of packed bf16; then dout, delta
// (16 fp32 each)
template <bool BF16>
struct LoadLayout {
  static constexpr int kIn = BF16 ? 8 : 16;
  static constexpr int kQ = 0, kK = kIn, kG = 2 * kIn, kDout = 3 * kIn, kDe = kDout + 16,
                       kEnd = kDe + 16;
  static_assert(kEnd <= kState, "loader state does not fit");
};

template <bool BF16>
__device__ __forceinline__ void load_in16(const void* p, int64_t base, bool in, float* dst) {
  using L = LoadLayout<BF16>;
  if constexpr (BF16) {
    const uint4* q = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + base);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 x = in ? q[i] : uint4{0, 0, 0, 0};
      dst[4 * i] = __uint_as_float(x.x);
      dst[4 * i + 1] = __uint_as_float(x.y);
      dst[4 * i + 2] = __uint_as_float(x.z);
      dst[4 * i + 3] = __uint_as_float(x.w);
    }
  } else {
    const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(p) + base);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 x = in ? q[i] : float4{0, 0, 0, 0};
      dst[4 * i] = x.x;
      dst[4 * i + 1] = x.y;
      dst[4 * i + 2] = x.z;
      dst[4 * i + 3] = x.w;
    }
  }
  (void)sizeof(L);
}
// element i of 16 loaded by load_in16
template <bool BF16>
__device__ __forceinline__ float in16(const float* src, int i) {
  if constexpr (BF16) {
    const uint32_t w = __float_as_uint(src[i >> 1]);
    return __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
  } else {
    return src[i];
  }
}

template <bool BF16>
__device__ __forceinline__ void loader_issue(float (&st)[kState], float& eta, int& n,
                                             const void* qp, const void* kp, const void* gp,
                                             const void* ep, const float* dout_p,
                                             const float* rec_delta, int64_t bhT, int64_t t0,
                                             int64_t T, int lane) {
  using L = LoadLayout<BF16>;
  n = static_cast<int>(min<int64_t>(BT, T - t0));
  const int t = lane >> 2, f0 = 16 * (lane & 3);
  const bool in = t < n;
  const int64_t base = (bhT + t0 + t) * D + f0;
  load_in16<BF16>(qp, base, in, &st[L::kQ]);
  load_in16<BF16>(kp, base, in, &st[L::kK]);
  load_in16<BF16>(gp, base, in, &st[L::kG]);
  load_in16<false>(dout_p, base, in, &st[L::kDout]);
  load_in16<false>(rec_delta, base, in, &st[L::kDe]);
  eta = lane < n ? ld_in<BF16>(ep, bhT + t0 + lane) : 0.0f;
}

template <bool BF16>
__device__ __forceinline__ void loader_store(const float (&st)[kState], float eta, int n,
                                             TileIn& tl, int lane, bool silu) {
  using L = LoadLayout<BF16>;
  const int t = lane >> 2, f0 = 16 * (lane & 3);
#pragma unroll
  for (int i = 0; i < 16; i += 4) {
    float4 q4, k4, y4, d4, g4;
    float* qv = &q4.x;
    float* kv = &k4.x;
    float* yv = &y4.x;
    float* dv = &d4.x;
    float* gv = &g4.x;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      qv[u] = in16<BF16>(&st[L::kQ], i + u);
      kv[u] = in16<BF16>(&st[L::kK], i + u);
      if (silu) {
        qv[u] = silu_in<BF16>(qv[u]);
        kv[u] = silu_in<BF16>(kv[u]);
      }
      const float sg = sigmoidf_(in16<BF16>(&st[L::kG], i + u));
      yv[u] = t < n ? st[L::kDout + i + u] * sg : 0.0f;
      gv[u] = yv[u] * (1.0f - sg);
      dv[u] = st[L::kDe + i + u];
    }
    *reinterpret_cast<float4*>(&tl.Q[t][f0 + i]) = q4;
    *reinterpret_cast<float4*>(&tl.K[t][f0 + i]) = k4;
    *reinterpret_cast<float4*>(&tl.DY[t][f0 + i]) = y4;
    *reinterpret_cast<float4*>(&tl.G2[t][f0 + i]) = g4;
    *reinterpret_cast<float4*>(&tl.De[t][f0 + i]) = d4;
  }
  if (lane < BT) {
    const float s = lane < n ? sigmoidf_(eta) : 0.0f;
    tl.ETA[lane] = s * (1.0f / D);
    tl.ELD[lane] = s * (1.0f - s) * (1.0f / D);
  }
}

// wave 7: a recorded W (64 fp32 a lane: elements 4 (lane + 64 j) .. +3)
__device__ __forceinline__ void w_issue(float (&st)[kState], const float* w_rec, int lane) {
  const float4* wp = reinterpret_cast<const float4*>(w_rec);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float4 x = wp[lane + 64 * j];
    st[4 * j] = x.x;
    st[4 * j + 1] = x.y;
    st[4 * j + 2] = x.z;
    st[4 * j + 3] = x.w;
  }
}
__device__ __forceinline__ void w_store(const float (&st)[kState], float (*W)[KP], int lane) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int e = 4 * (lane + 64 * j);
    *reinterpret_cast<float4*>(&W[e / D][e % D]) =
        make_float4(st[4 * j], st[4 * j + 1], st[4 * j + 2], st[4 * j + 3]);
  }
}

template <bool BF16, int LN, bool DUAL>
__global__ void __launch_bounds__(NT)
bwd_mfma_kernel(const void* __restrict__ qp, const void* __restrict__ kp,
                const void* __restrict__ vp, const void* __restrict__ etap,
                const void* __restrict__ gatep, const float* __restrict__ gamma,
                const float* __restrict__ beta, const float* __restrict__ dout,
                const float* __restrict__ dW_final, const float* __restrict__ rec_delta,
                const float* __restrict__ rec_W, float* __restrict__ dq, float* __restrict__ dk,
                float* __restrict__ dv, float* __restrict__ deta, float* __restrict__ dgate,
                float* __restrict__ dW0, float* __restrict__ gb_part, int H, int64_t T,
                float eps, int silu) {
  __shared__ BwdSmem sm;
  // the wave that forms B2's third column block in phase B: with bf16 inputs
  // (outside the exact LayerNorm) wave 1, whose phase B is short there, so
  // that the loader's store is the only long task of its phase; else the
  // loader (measured: each choice slower by 6-12% where it is not used)
  constexpr int kB2Wave = (BF16 && LN != kLnExact) ? 1 : 4;
  // the dual form's chain is short: its wave and the loader each take one of
  // the four DY W blocks (and its dq block) from waves 2 and 3 (bf16 inputs,
  // where the loader's state leaves slot 14 free)
  constexpr bool kSpreadDq = DUAL && BF16 && LN != kLnExact;
  static_assert(!kSpreadDq || LoadLayout<BF16>::kEnd <= 56, "slot 14 must be free");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int G = lane >> 4;
  const int64_t bh = blockIdx.x;
  const int h = static_cast<int>(bh % H);
  const int64_t bhT = bh * T;
  const int N = static_cast<int>((T + BT - 1) / BT);
  auto rows = [&](int c) { return static_cast<int>(min<int64_t>(BT, T - int64_t(c) * BT)); };
  auto wrec = [&](int c) { return (bh * N + c) * D * D; };

  // ---- prologue: H = dL/dW_final; tile N-1 and its W ----
  for (int e = tid; e < D * D; e += NT)
    sm.Hm[e / D][e % D] = dW_final != nullptr ? dW_final[bh * D * D + e] : 0.0f;
  if (N > 0) {
    const int c = N - 1, n = rows(c);
    TileIn& tl = sm.ring[c % 3];
    for (int e = tid; e < BT * D; e += NT) {
      const int t = e / D, i = e % D;
      const bool in = t < n;
      const int64_t g = (bhT + int64_t(c) * BT + t) * D + i;
      const float qv = in ? ld_in<BF16>(qp, g) : 0.0f;
      const float kv = in ? ld_in<BF16>(kp, g) : 0.0f;
      tl.Q[t][i] = silu ? silu_in<BF16>(qv) : qv;
      tl.K[t][i] = silu ? silu_in<BF16>(kv) : kv;
      const float sg = in ? sigmoidf_(ld_in<BF16>(gatep, g)) : 0.0f;
      tl.DY[t][i] = in ? dout[g] * sg : 0.0f;
      tl.G2[t][i] = tl.DY[t][i] * (1.0f - sg);
      tl.De[t][i] = in ? rec_delta[g] : 0.0f;
    }
    if (tid < BT) {
      const float s = tid < n ? sigmoidf_(ld_in<BF16>(etap, bhT + int64_t(c) * BT + tid)) : 0.0f;
      tl.ETA[tid] = s * (1.0f / D);
      tl.ELD[tid] = s * (1.0f - s) * (1.0f / D);
    }
    for (int e = tid; e < D * D; e += NT) sm.W[c & 1][e / D][e % D] = rec_W[wrec(c) + e];
  }

  // per-role constants
  float gam = 1.0f, gam0 = 1.0f;        // wave 0: gamma of feature `lane`, mean gamma^2
  float dgam = 0.0f, dbet = 0.0f;       // wave 0: this scan's dgamma, dbeta of feature `lane`
  if (wave == 0 && LN != kLnNone) {
    gam = gamma[h * D + lane];
    float s[1] = {gam * gam};
    wave_sums<1>(s);
    gam0 = s[0] * (1.0f / D);
  }
  float cg[4] = {1, 1, 1, 1}, cb[4] = {0, 0, 0, 0};   // wave 1: features 16 fb + l16
  if (wave == 1 && LN != kLnNone) {
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
      cg[fb] = gamma[h * D + 16 * fb + l16];
      cb[fb] = beta[h * D + 16 * fb + l16];
    }
  }
  float st[kState];    // the role state kept across barriers (see above)
  float ld_eta = 0.0f;
  int ld_n = 0;
  // every prologue load complete: otherwise the token guards of the chain
  // leave the gamma load pending and each token waits on the memory counter
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int c = N; c >= 0; --c) {
    const bool prep = c >= 1;       // tile c-1 exists
    const bool live = c < N;        // tile c exists
    const int cm = c - 1;
    // ============================ phase A ============================
    // dQ' = DY W of tile c-1, column block jb into state slot sl
    auto dqw1 = [&](auto jbc, auto slc) {
      constexpr int jb = decltype(jbc)::value, sl = decltype(slc)::value;
      const TileIn& tm = sm.ring[cm % 3];
      const float(*Wm)[KP] = sm.W[cm & 1];
      float a[16], bb[16];
      frag_row64(tm.DY[l16], G, a);
      frag_col64(Wm, 16 * jb + l16, G, bb);
      put(st, sl, mma<16>(a, bb, f32x4{0, 0, 0, 0}));
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I14 = std::integral_constant<int, 14>;
    if (wave == 0) {
      if (live) {
        // ---- the dz chain of tile c, t descending ----
        const TileIn& tc = sm.ring[c % 3];
        Work& w = sm.wk[c & 1];
        const float(*KK)[TP] = sm.gr[c & 1].KK;
        const int n = rows(c);
        const int64_t t0 = int64_t(c) * BT;
        float ac[BT];
#pragma unroll
        for (int t = 0; t < BT; ++t) ac[t] = w.A[t][lane];
        // a token's inputs from LDS, read one token ahead so that their
        // latency hides behind the previous token's sums
        struct Tok {
          float eta, x, e, rs, mg, mgx, g1, g2;
          float kk[BT];   // k_s . k_t, s < t
        };
        auto fetch = [&](int t, Tok& k) {
          k.eta = tc.ETA[t];
          if constexpr (LN != kLnNone) {
            k.x = w.X[t][lane];
            if constexpr (LN == kLnExact) {
              k.e = w.E[t][lane];
              const float4 s4 = *reinterpret_cast<const float4*>(&w.S[t][0]);
              k.rs = s4.x;
              k.mg = s4.y;
              k.mgx = s4.z;
              k.g1 = s4.w;
              k.g2 = w.S[t][4];
            } else {
              k.rs = w.S[t][0];
            }
          }
          if constexpr (!DUAL) {
#pragma unroll
            for (int s = 0; s < BT; ++s)
              if (s < t) k.kk[s] = KK[t][s];   // KK is symmetric: row t reads contiguously
          }
        };
        Tok cur, nxt;
        fetch(BT - 1, nxt);
#pragma unroll
        for (int t = BT - 1; t >= 0; --t) {
          cur = nxt;
          if (t > 0) fetch(t - 1, nxt);
          if (t < n) {
            const float a = ac[t];
            const float dd = -cur.eta * a;
            float dz, dvv;
            if constexpr (LN == kLnNone) {
              dz = dd;
              dvv = -dd;
            } else if constexpr (LN == kLnST) {
              const float x = cur.x, rs = cur.rs;
              const float ww = gam * dd;
              float sm2[2] = {ww, ww * x};
              wave_sums<2>(sm2);
              dz = rs * (ww - sm2[0] * (1.0f / D) - x * (sm2[1] * (1.0f / D)));
              dvv = -dd;
              dgam = fmaf(dd, x, dgam);
              dbet += dd;
            } else {
              // delta = rs (g - mean g - xhat mean(g xhat)), g = gamma e; one
              // round of five sums of dd against per-token constants
              const float x = cur.x, e = cur.e, rs = cur.rs, mg = cur.mg, mgx = cur.mgx;
              const float g1 = cur.g1, g2 = cur.g2;
              const float g = gam * e;
              const float P = g - mg - x * mgx;
              const float g2d = gam * gam * dd;
              float sm5[5] = {dd, dd * x, g2d, g2d * x, dd * P};
              wave_sums<5>(sm5);
              const float sdp = rs * sm5[0], sdpx = rs * sm5[1], drs = sm5[4];
              const float dP = rs * dd;
              const float dg = dP - sdp * (1.0f / D) - x * (sdpx * (1.0f / D));
              const float de = gam * dg;
              const float dxh = gam * de - dP * mgx - sdpx * (1.0f / D) * g;
              const float m1 = (rs * sm5[2] - gam0 * sdp - g1 * sdpx - rs * mgx * sm5[0] -
                                sdpx * mg) * (1.0f / D);
              const float m2 = (rs * sm5[3] - g1 * sdp - g2 * sdpx - rs * mgx * sm5[1] -
                                sdpx * mgx) * (1.0f / D);
              dz = rs * (dxh - m1 - x * m2) - drs * rs * rs * x * (1.0f / D);
              dvv = -de;
              dgam += fmaf(e, dg, x * de);
              dbet += de;
            }
            // the next token needs only row t-1; the other rows' updates
            // overlap its sums.  The dual form: z of every token of the tile
            // is taken at the tile's first W, so no dz flows back within it.
            if constexpr (!DUAL)
              if (t > 0) ac[t - 1] = fmaf(cur.kk[t - 1], dz, ac[t - 1]);
            w.X[t][lane] = dz;
            w.A[t][lane] = a;
            dv[(bhT + t0 + t) * D + lane] = dvv;
            if constexpr (!DUAL) {
#pragma unroll
              for (int s = 0; s + 1 < t; ++s) ac[s] = fmaf(cur.kk[s], dz, ac[s]);
            }
          }
          // keeps each token's loads one token ahead rather than all hoisted
          // (the dual form's tokens are independent: let their sums overlap)
          if constexpr (!DUAL) __builtin_amdgcn_sched_barrier(0);
        }
        // ---- Grams that need dz: DeDZ[s][t'] = delta_s . dz_t' and
        //      DZE[t][s] = eta_s (dz_t . delta_s) over tile c-1's s ----
        if constexpr (!DUAL) store_block(sm.DeDZ, 0, gram(tc.De, w.X, l16, G), l16, G);
        if (prep) {
          const TileIn& tm = sm.ring[cm % 3];
          f32x4 g2 = gram(w.X, tm.De, l16, G);
#pragma unroll
          for (int r = 0; r < 4; ++r) g2[r] *= tm.ETA[l16];
          store_block(sm.DZE, 0, g2, l16, G);
        }
      }
      if constexpr (kSpreadDq) {
        if (prep) dqw1(I1{}, I0{});
      }
    } else if (wave == 3 || wave == 2) {
      // dk's H-side half b1, column blocks j0, j0+1 (wave 3: 0-1 in state
      // slots 0-1; wave 2: 2-3 in slots 4-5), beside half of DY W each
      auto half = [&](auto s0c) {
        constexpr int s0 = decltype(s0c)::value;
        const int j0 = s0 == 0 ? 0 : 2;
        if (c + 1 < N) {
          // dk of tile c+1 = -eta b1 + B2
          const int cp = c + 1, n = rows(cp);
          const TileIn& tp = sm.ring[cp % 3];
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int t = 4 * G + r, j = 16 * (j0 + jj) + l16;
              if (t < n)
                dk[(bhT + int64_t(cp) * BT + t) * D + j] =
                    fmaf(-tp.ETA[t], st[4 * (s0 + jj) + r], sm.B2[t][j]);
            }
        }
        if (live) {
          // delta_c H, H being the gradient after tile c
          const TileIn& tc = sm.ring[c % 3];
          float a[16];
          frag_row64(tc.De[l16], G, a);
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            float bb[16];
            frag_col64(sm.Hm, 16 * (j0 + jj) + l16, G, bb);
            put(st, s0 + jj, mma<16>(a, bb, f32x4{0, 0, 0, 0}));
          }
        }
      };
      // dQ' = DY W of tile c-1, column blocks j0, j0+1 into state slots
      // j0, j0+1 (wave 2: blocks 0-1; wave 3: blocks 2-3)
      auto dqw = [&](auto j0c) {
        constexpr int j0 = decltype(j0c)::value;
        const TileIn& tm = sm.ring[cm % 3];
        const float(*Wm)[KP] = sm.W[cm & 1];
        float a[16];
        frag_row64(tm.DY[l16], G, a);
#pragma unroll
        for (int jb = j0; jb < j0 + 2; ++jb) {
          float bb[16];
          frag_col64(Wm, 16 * jb + l16, G, bb);
          put(st, jb, mma<16>(a, bb, f32x4{0, 0, 0, 0}));
        }
      };
      if (wave == 3) {
        half(std::integral_constant<int, 0>{});
        if constexpr (kSpreadDq) {
          if (prep) dqw1(I2{}, I2{});
        } else {
          if (prep) dqw(std::integral_constant<int, 2>{});
        }
      } else {
        half(std::integral_constant<int, 4>{});
        if constexpr (kSpreadDq) {
          if (prep) dqw1(I0{}, I0{});
        } else {
          if (prep) dqw(std::integral_constant<int, 0>{});
        }
      }
    } else if (wave != 4 && prep) {
      const TileIn& tm = sm.ring[cm % 3];
      const float(*Wm)[KP] = sm.W[cm & 1];
      if (wave == 1 || wave == 5 || wave == 6) {
        // Z' = K W^T (wave 1), Y' = Q W^T (wave 5), A0' = K H^T (wave 6)
        const float(*Ar)[KP] = wave == 5 ? tm.Q : tm.K;
        const float(*Br)[KP] = wave == 6 ? sm.Hm : Wm;
        float a[16];
        frag_row64(Ar[l16], G, a);
#pragma unroll
        for (int fb = 0; fb < 4; ++fb) {
          float b[16];
          frag_row64(Br[16 * fb + l16], G, b);
          put(st, fb, mma<16>(a, b, f32x4{0, 0, 0, 0}));
        }
        // fetched for phase B: v (wave 1, exact LayerNorm)
        const int nm = rows(cm);
        const int64_t t0 = int64_t(cm) * BT;
        if (wave == 1 && LN == kLnExact) {
#pragma unroll
          for (int fb = 0; fb < 4; ++fb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int t = 4 * G + r;
              st[16 + 4 * fb + r] = t < nm ? ld_in<BF16>(vp, (bhT + t0 + t) * D + 16 * fb + l16) : 0.0f;
            }
        }
      } else if (wave == 7) {
        // the W of tile c-2 in flight; Grams of tile c-1 and its cross Grams with tile c
        if (c >= 2) w_issue(st, rec_W + wrec(c - 2), lane);
        Grams& gm = sm.gr[cm & 1];
        store_block(gm.KK, 0, gram(tm.K, tm.K, l16, G), l16, G);
        store_block(gm.QK, 0, gram(tm.Q, tm.K, l16, G), l16, G);
        store_block(gm.DeDY, 0, gram(tm.De, tm.DY, l16, G), l16, G);
        if (live) {
          const TileIn& tc = sm.ring[c % 3];
          store_block(sm.XQ, 0, gram(tm.K, tc.Q, l16, G), l16, G);
          store_block(sm.XK, 0, gram(tm.K, tc.K, l16, G), l16, G);
        }
      }
    }
    if constexpr (kSpreadDq) {
      if (wave == 4 && prep) dqw1(I3{}, I14{});
    }
    if (wave == 4 && c >= 2) {
      const int u = c - 2;
      loader_issue<BF16>(st, ld_eta, ld_n, qp, kp, gatep, etap, dout, rec_delta, bhT,
                         int64_t(u) * BT, T, lane);
    }
    __syncthreads();
    // ============================ phase B ============================
    // dq of tile c-1 = DY W - sum_{s<=t} eta_s (delta_s.dy_t) k_s, column
    // blocks j0, j0+1 from DY W in state slots j0, j0+1 (wave 2: blocks 0-1,
    // wave 3: blocks 2-3)
    auto dq_blocks = [&](auto j0c) {
      constexpr int j0 = decltype(j0c)::value;
      const TileIn& tm = sm.ring[cm % 3];
      const Grams& gm = sm.gr[cm & 1];
      float a[4];
      frag_col16(gm.DeDY, l16, G, a);   // DeDY[s][t], k = s, m = t
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int s = 4 * G + ks;
        a[ks] = s <= l16 ? -tm.ETA[s] * a[ks] : 0.0f;
      }
      const int nm = rows(cm);
      const int64_t t0 = int64_t(cm) * BT;
#pragma unroll
      for (int jb = j0; jb < j0 + 2; ++jb) {
        float b[4];
        frag_col16(tm.K, 16 * jb + l16, G, b);
        const f32x4 v = mma<4>(a, b, blk(st, jb));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 4 * G + r;
          if (t < nm) dq[(bhT + t0 + t) * D + 16 * jb + l16] = v[r];
        }
      }
    };
    if (wave == 4 && c >= 2) {
      const int u = c - 2;
      loader_store<BF16>(st, ld_eta, ld_n, sm.ring[u % 3], lane, silu != 0);
    }
    // dq of tile c-1, column block jb from state slot sl (as dq_blocks)
    auto dq1 = [&](auto jbc, auto slc) {
      constexpr int jb = decltype(jbc)::value, sl = decltype(slc)::value;
      const TileIn& tm = sm.ring[cm % 3];
      const Grams& gm = sm.gr[cm & 1];
      float a[4];
      frag_col16(gm.DeDY, l16, G, a);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int s = 4 * G + ks;
        a[ks] = s <= l16 ? -tm.ETA[s] * a[ks] : 0.0f;
      }
      const int nm = rows(cm);
      const int64_t t0 = int64_t(cm) * BT;
      float b[4];
      frag_col16(tm.K, 16 * jb + l16, G, b);
      const f32x4 v = mma<4>(a, b, blk(st, sl));
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * G + r;
        if (t < nm) dq[(bhT + t0 + t) * D + 16 * jb + l16] = v[r];
      }
    };
    if constexpr (kSpreadDq) {
      if (prep && wave == 0) dq1(I1{}, I0{});
      if (prep && wave == 4) dq1(I3{}, I14{});
    }
    if (wave == 7 && c >= 2) w_store(st, sm.W[(c - 2) & 1], lane);
    if (wave == 1 && prep) {
      // z of tile c-1 and its LayerNorm statistics -> the chain's working set
      const TileIn& tm = sm.ring[cm % 3];
      const Grams& gm = sm.gr[cm & 1];
      Work& w = sm.wk[cm & 1];
      if constexpr (!DUAL) {
        // z_t = W_c k_t - sum_{s<t} eta_s (k_s . k_t) delta_s (the dual form
        // takes every z of the tile at W_c)
        float a[4];
        frag_row16(gm.KK[l16], G, a);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) a[ks] = (4 * G + ks < l16) ? a[ks] : 0.0f;
#pragma unroll
        for (int fb = 0; fb < 4; ++fb) {
          float b[4];
          frag_col16(tm.De, 16 * fb + l16, G, b);
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) b[ks] *= -tm.ETA[4 * G + ks];
          put(st, fb, mma<4>(a, b, blk(st, fb)));
        }
      }
      if constexpr (LN != kLnNone) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 4 * G + r;
          const float mu = row16_sum(st[r] + st[4 + r] + st[8 + r] + st[12 + r]) * (1.0f / D);
          float cz[4], ss = 0.0f;
#pragma unroll
          for (int fb = 0; fb < 4; ++fb) {
            cz[fb] = st[4 * fb + r] - mu;
            ss = fmaf(cz[fb], cz[fb], ss);
          }
          const float var = row16_sum(ss) * (1.0f / D);
          const float rs = __builtin_amdgcn_rsqf(var + eps);
          float xh[4];
#pragma unroll
          for (int fb = 0; fb < 4; ++fb) {
            xh[fb] = cz[fb] * rs;
            w.X[t][16 * fb + l16] = xh[fb];
          }
          if constexpr (LN == kLnExact) {
            float sg = 0.0f, sgx = 0.0f, s1 = 0.0f, s2 = 0.0f;
#pragma unroll
            for (int fb = 0; fb < 4; ++fb) {
              const float e = fmaf(cg[fb], xh[fb], cb[fb] - st[16 + 4 * fb + r]);
              w.E[t][16 * fb + l16] = e;
              const float g = cg[fb] * e, g2 = cg[fb] * cg[fb] * xh[fb];
              sg += g;
              sgx = fmaf(g, xh[fb], sgx);
              s1 += g2;
              s2 = fmaf(g2, xh[fb], s2);
            }
            sg = row16_sum(sg);
            sgx = row16_sum(sgx);
            s1 = row16_sum(s1);
            s2 = row16_sum(s2);
            if (l16 == 0) {
              *reinterpret_cast<float4*>(&w.S[t][0]) =
                  make_float4(rs, sg * (1.0f / D), sgx * (1.0f / D), s1 * (1.0f / D));
              w.S[t][4] = s2 * (1.0f / D);
            }
          } else {
            if (l16 == 0) w.S[t][0] = rs;
          }
        }
      } else {
        // no LayerNorm: the chain reads no statistics; rows past the end
        // must still hand a zero dz on
#pragma unroll
        for (int fb = 0; fb < 4; ++fb) store_block(w.X, 16 * fb, f32x4{0, 0, 0, 0}, l16, G);
      }
    } else if (wave == 5 && prep) {
      // y of tile c-1 -> dgate = y dout sigmoid'(gate)
      const TileIn& tm = sm.ring[cm % 3];
      const Grams& gm = sm.gr[cm & 1];
      float a[4];
      frag_row16(gm.QK[l16], G, a);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) a[ks] = (4 * G + ks <= l16) ? a[ks] : 0.0f;
      const int nm = rows(cm);
      const int64_t t0 = int64_t(cm) * BT;
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) {
        float b[4];
        frag_col16(tm.De, 16 * fb + l16, G, b);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) b[ks] *= -tm.ETA[4 * G + ks];
        const f32x4 y = mma<4>(a, b, blk(st, fb));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 4 * G + r;
          if (t < nm) dgate[(bhT + t0 + t) * D + 16 * fb + l16] = y[r] * tm.G2[t][16 * fb + l16];
        }
      }
    } else if (wave == 3) {
      if constexpr (kSpreadDq) {
        if (prep) dq1(I2{}, I2{});
      } else {
        if (prep) dq_blocks(std::integral_constant<int, 2>{});
      }
    } else if (wave == 2) {
      if constexpr (kSpreadDq) {
        if (prep) dq1(I0{}, I0{});
      } else {
        if (prep) dq_blocks(std::integral_constant<int, 0>{});
      }
      if (live) {
        // d eta_logit of tile c = -sigmoid'(.)/d delta_t . a_t (a Gram's diagonal)
        const TileIn& tc = sm.ring[c % 3];
        const f32x4 gd = gram(tc.De, sm.wk[c & 1].A, l16, G);
        const int n = rows(c);
        const int r = l16 - 4 * G;
        if (r >= 0 && r < 4 && l16 < n) {
          float v = gd[0];
          v = r == 1 ? gd[1] : v;
          v = r == 2 ? gd[2] : v;
          v = r == 3 ? gd[3] : v;
          deta[bhT + int64_t(c) * BT + l16] = -tc.ELD[l16] * v;
        }
      }
    } else if (wave == 6 && prep) {
      // a0 of tile c-1 = K H^T + (K_{c-1} Q_c^T) DY_c + (K_{c-1} K_c^T) DZ_c
      //                  + sum_{t'>=t} (q_t'.k_t) dy_t'
      const TileIn& tm = sm.ring[cm % 3];
      const Grams& gm = sm.gr[cm & 1];
      float au[4];
      frag_col16(gm.QK, l16, G, au);    // QK[t'][t], k = t', m = t
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) au[ks] = (4 * G + ks >= l16) ? au[ks] : 0.0f;
      float aq[4] = {0, 0, 0, 0}, ak[4] = {0, 0, 0, 0};
      if (live) {
        frag_row16(sm.XQ[l16], G, aq);
        frag_row16(sm.XK[l16], G, ak);
      }
      Work& w = sm.wk[cm & 1];
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) {
        float b[4];
        frag_col16(tm.DY, 16 * fb + l16, G, b);
        f32x4 v = mma<4>(au, b, blk(st, fb));
        if (live) {
          const TileIn& tc = sm.ring[c % 3];
          frag_col16(tc.DY, 16 * fb + l16, G, b);
          v = mma<4>(aq, b, v);
          frag_col16(sm.wk[c & 1].X, 16 * fb + l16, G, b);
          v = mma<4>(ak, b, v);
        }
        store_block(w.A, 16 * fb, v, l16, G);
      }
    }
    if ((wave == 3 || wave == 2) && live) {
      // b1 += sum_{t'>=t} (delta_t.dy_t') q_t' + sum_{t'>t} (delta_t.dz_t') k_t'
      // (the dual form: no dz term within the tile)
      const TileIn& tc = sm.ring[c % 3];
      float ay[4], az[4] = {0, 0, 0, 0};
      frag_row16(sm.gr[c & 1].DeDY[l16], G, ay);
      if constexpr (!DUAL) frag_row16(sm.DeDZ[l16], G, az);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int tp = 4 * G + ks;
        ay[ks] = tp >= l16 ? ay[ks] : 0.0f;
        az[ks] = tp > l16 ? az[ks] : 0.0f;
      }
      auto half = [&](auto s0c) {
        constexpr int s0 = decltype(s0c)::value;
        const int j0 = s0 == 0 ? 0 : 2;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int jb = j0 + jj;
          float bb[4];
          frag_col16(tc.Q, 16 * jb + l16, G, bb);
          put(st, s0 + jj, mma<4>(ay, bb, blk(st, s0 + jj)));
          if constexpr (!DUAL) {
            frag_col16(tc.K, 16 * jb + l16, G, bb);
            put(st, s0 + jj, mma<4>(az, bb, blk(st, s0 + jj)));
          }
        }
      };
      if (wave == 3)
        half(std::integral_constant<int, 0>{});
      else
        half(std::integral_constant<int, 4>{});
    }
    if ((wave == 0 || wave == kB2Wave || wave == 3) && live) {
      // B2 = DZ W_c - sum_{s<t} eta_s (delta_s.dz_t) k_s, with
      // DZ W_c = DZ W_{c-1} - (DZ E_{c-1}^T) K_{c-1} (for c = 0 the slot holds W_0);
      // the dual form has no in-tile sum
      const TileIn& tc = sm.ring[c % 3];
      const float(*Wm)[KP] = sm.W[(prep ? cm : 0) & 1];
      float a[16];
      frag_row64(sm.wk[c & 1].X[l16], G, a);
      float as[4] = {0, 0, 0, 0}, ae[4] = {0, 0, 0, 0};
      if constexpr (!DUAL) {
        frag_col16(sm.DeDZ, l16, G, as);   // DeDZ[s][t], k = s, m = t
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int s = 4 * G + ks;
          as[ks] = s < l16 ? -tc.ETA[s] * as[ks] : 0.0f;
        }
      }
      if (prep) {
        frag_row16(sm.DZE[l16], G, ae);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) ae[ks] = -ae[ks];
      }
      // column blocks: wave 0 takes 0 and 1, kB2Wave block 2, wave 3 block 3
      const int jb0 = wave == 0 ? 0 : wave == kB2Wave ? 2 : 3;
      const int njb = wave == 0 ? 2 : 1;
      for (int jj = 0; jj < njb; ++jj) {
        const int jb = jb0 + jj;
        float b[16];
        frag_col64(Wm, 16 * jb + l16, G, b);
        f32x4 v = mma<16>(a, b, f32x4{0, 0, 0, 0});
        float bk[4];
        if constexpr (!DUAL) {
          frag_col16(tc.K, 16 * jb + l16, G, bk);
          v = mma<4>(as, bk, v);
        }
        if (prep) {
          frag_col16(sm.ring[cm % 3].K, 16 * jb + l16, G, bk);
          v = mma<4>(ae, bk, v);
        }
        store_block(sm.B2, 16 * jb, v, l16, G);
      }
    }
    if (live && (wave == 7 || wave == 0 || wave == 1 || wave == 5 || wave == 6)) {
      // H += DY_c^T Q_c + DZ_c^T K_c by 16x16 blocks b = 4 ib + jb, in pairs
      // whose loads and MFMAs interleave: wave 7 takes pairs 0-2, wave 0
      // pair 3, wave 1 pairs 4-5, wave 5 pair 6, wave 6 pair 7
      const TileIn& tc = sm.ring[c % 3];
      const float(*DZ)[KP] = sm.wk[c & 1].X;
      const int p0 = wave == 7 ? 0 : wave == 0 ? 3 : wave == 1 ? 4 : wave == 5 ? 6 : 7;
      const int p1 = p0 + (wave == 7 ? 3 : wave == 1 ? 2 : 1);
      for (int pr = p0; pr < p1; ++pr) {
        const int ib = pr >> 1, jb0 = 2 * (pr & 1);
        float ay[4], az[4];
        frag_col16(tc.DY, 16 * ib + l16, G, ay);
        frag_col16(DZ, 16 * ib + l16, G, az);
        f32x4 v[2];
        float bq[2][4], bk[2][4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int r = 0; r < 4; ++r) v[u][r] = sm.Hm[16 * ib + 4 * G + r][16 * (jb0 + u) + l16];
          frag_col16(tc.Q, 16 * (jb0 + u) + l16, G, bq[u]);
          frag_col16(tc.K, 16 * (jb0 + u) + l16, G, bk[u]);
        }
        if constexpr (BF16) {
          // q and k are bf16 values: dy and dz split into hi + lo
          i16x4 yh, yl, zh, zl;
          split4(ay, yh, yl);
          split4(az, zh, zl);
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const i16x4 q16 = exact4(bq[u]), k16 = exact4(bk[u]);
            v[u] = mfma16(yh, q16, v[u]);
            v[u] = mfma16(zh, k16, v[u]);
            v[u] = mfma16(yl, q16, v[u]);
            v[u] = mfma16(zl, k16, v[u]);
          }
        } else {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int u = 0; u < 2; ++u) v[u] = mfma4(ay[ks], bq[u][ks], v[u]);
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int u = 0; u < 2; ++u) v[u] = mfma4(az[ks], bk[u][ks], v[u]);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) sm.Hm[16 * ib + 4 * G + r][16 * (jb0 + u) + l16] = v[u][r];
      }
    }
    __syncthreads();
  }
  // dk of tile 0; dW0 = H; this scan's share of dgamma, dbeta
  if ((wave == 3 || wave == 2) && N > 0) {
    auto half = [&](auto s0c) {
      constexpr int s0 = decltype(s0c)::value;
      const int j0 = s0 == 0 ? 0 : 2;
      const int n = rows(0);
      const TileIn& tp = sm.ring[0];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 4 * G + r, j = 16 * (j0 + jj) + l16;
          if (t < n)
            dk[bhT * D + t * D + j] = fmaf(-tp.ETA[t], st[4 * (s0 + jj) + r], sm.B2[t][j]);
        }
    };
    if (wave == 3)
      half(std::integral_constant<int, 0>{});
    else
      half(std::integral_constant<int, 4>{});
  }
  for (int e = tid; e < D * D; e += NT) dW0[bh * D * D + e] = sm.Hm[e / D][e % D];
  if (wave == 0 && gb_part != nullptr) {
    gb_part[(bh * 2) * D + lane] = dgam;
    gb_part[(bh * 2 + 1) * D + lane] = dbet;
  }
}

// the :mlp variant: the gradients computed for silu(q), silu(k) times
// silu'(x) = sigmoid(x) (1 + x (1 - sigmoid(x))) at the raw inputs; eight
// elements per thread (n is a multiple of d = 64; every pointer is 16-byte
// aligned), as 16-byte loads and stores
__device__ __forceinline__ float silu_grad(float x) {
  const float s = sigmoidf_(x);
  return s * fmaf(x, 1.0f - s, 1.0f);
}
template <bool BF16>
__device__ __forceinline__ void load8(const void* p, int64_t i, float (&x)[8]) {
  if constexpr (BF16) {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(u[e] << 16);
      x[2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
    }
  } else {
    const float4* f = reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    const float4 a = f[0], b = f[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}
__device__ __forceinline__ void scale8(float* g, int64_t i, const float (&x)[8]) {
  float4* p = reinterpret_cast<float4*>(g + i);
  float4 a = p[0], b = p[1];
  a.x *= silu_grad(x[0]); a.y *= silu_grad(x[1]); a.z *= silu_grad(x[2]); a.w *= silu_grad(x[3]);
  b.x *= silu_grad(x[4]); b.y *= silu_grad(x[5]); b.z *= silu_grad(x[6]); b.w *= silu_grad(x[7]);
  p[0] = a;
  p[1] = b;
}
template <bool BF16>
__global__ void silu_grad_kernel(const void* __restrict__ qp, const void* __restrict__ kp,
                                 float* __restrict__ dq, float* __restrict__ dk, int64_t n8) {
  const int64_t v = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (v >= n8) return;
  const int64_t i = 8 * v;
  float x[8];
  load8<BF16>(qp, i, x);
  scale8(dq, i, x);
  load8<BF16>(kp, i, x);
  scale8(dk, i, x);
}

// dgamma[h][i] = sum over the batch of the per-scan parts, dbeta likewise (fixed order)
__global__ void gamma_beta_sum_kernel(const float* __restrict__ gb_part, float* __restrict__ dgamma,
                                      float* __restrict__ dbeta, int64_t B, int64_t H) {
  const int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (e >= H * D) return;
  const int64_t h = e / D, i = e % D;
  float sg = 0.0f, sb = 0.0f;
  for (int64_t b = 0; b < B; ++b) {
    sg += gb_part[((b * H + h) * 2) * D + i];
    sb += gb_part[((b * H + h) * 2 + 1) * D + i];
  }
  dgamma[e] = sg;
  dbeta[e] = sb;
}

template <bool BF16, int LN, bool DUAL>
hipError_t launch_bwd(const BwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((bwd_mfma_kernel<BF16, LN, DUAL>), dim3(static_cast<unsigned>(a.B * a.H)), dim3(NT),
                     0, s, a.q, a.k, a.v, a.eta_logit, a.gate_logit, a.gamma, a.beta, a.dout,
                     a.dW_final, a.rec_delta, a.rec_W, a.dq, a.dk, a.dv, a.deta_logit,
                     a.dgate_logit, a.dW0, LN == kLnNone ? nullptr : a.gb_part,
                     static_cast<int>(a.H), a.T, a.eps, a.silu_qk ? 1 : 0);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (a.silu_qk && a.T > 0) {
    const int64_t n8 = a.B * a.H * a.T * (D / 8);
    hipLaunchKernelGGL((silu_grad_kernel<BF16>), dim3(static_cast<unsigned>((n8 + 255) / 256)),
                       dim3(256), 0, s, a.q, a.k, a.dq, a.dk, n8);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (LN == kLnNone) return hipSuccess;
  const int64_t n = a.H * D;
  hipLaunchKernelGGL(gamma_beta_sum_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                     0, s, a.gb_part, a.dgamma, a.dbeta, a.B, a.H);
  return hipGetLastError();
}

}  // namespace

template <bool BF16, bool DUAL>
hipError_t launch_ln(const BwdArgs& a, hipStream_t s) {
  switch (a.ln) {
    case kLnST: return launch_bwd<BF16, kLnST, DUAL>(a, s);
    case kLnExact: return launch_bwd<BF16, kLnExact, DUAL>(a, s);
    default: return launch_bwd<BF16, kLnNone, DUAL>(a, s);
  }
}

hipError_t launch_bwd_mfma(const BwdArgs& a, hipStream_t s) {
  // the dual form's chunks must be the tiles
  if (a.d != D || (a.dual && a.chunk != BT)) return hipErrorNotSupported;
  if (a.in_bf16) return a.dual ? launch_ln<true, true>(a, s) : launch_ln<true, false>(a, s);
  return a.dual ? launch_ln<false, true>(a, s) : launch_ln<false, false>(a, s);
}

}  // namespace ttt
