// Matrix-core chunk scan of the TTT-Linear recurrence for d = 64 (gfx950).
//
// Recurrence: "Edifice.Recurrent.TTT", "Equations (TTT-Linear)"; exact
// LayerNorm gradient: "Error Correction in Trained TTT Layers", abstract;
// chunk-start gradients: "PonderTTT", "Technical Architecture" (dual form).
//
// The sequence is cut into tiles of 16 tokens.  With W_c the weight at the
// start of tile c, E_s = eta_s delta_s and k_s.k_t the key Gram matrix, the
// per-token recurrence is, exactly,
//
//   z_t = W_c k_t - sum_{s<t in tile} eta_s (k_s.k_t) delta_s      (gradient point)
//   o_t = W_c q_t - sum_{s<=t in tile} eta_s (k_s.q_t) delta_s     (= W_t q_t)
//   W_{c+1} = W_c - sum_s eta_s delta_s k_s^T
//
// and one tile ahead, K_{c+1} W_{c+1}^T = K_{c+1} W_c^T - (K_{c+1} K_c^T) E_c.
// Every d x d product is therefore a dense tile contraction on MFMA that can
// run while the previous tile is still in its serial part; what stays serial
// is, per token, the d-vector correction of z_t, its LayerNorm statistics and
// delta_t.  The dual form drops the in-tile correction of z_t (tile = chunk =
// 16), so its 16 tokens are independent.
//
// Precision: W stays fp32 in MFMA accumulators.  With bf16 inputs every
// product runs as bf16 MFMA with fp32 accumulation and the fp32 operands (W,
// delta, the eta-scaled Gram entries) are split into bf16 hi + lo parts, so
// only the lo*lo term (~2^-17 relative) is dropped.  With fp32 inputs the
// products run as fp32 MFMA (16x16x4).
//
// Wave roles (8 waves; wave w runs on SIMD w % 4; see Roles below):
//   wave 0      serial LayerNorm pass, alone on its SIMD but for wave 4,
//               which only writes outputs back
//   waves 1,2,5,6  one 16-row slice of W each, as W^T tiles in the 16x16
//               accumulator layout (lane l holds W[16s + l%16][16jt + 4(l/16) + r]);
//               they apply the updates, form K W^T, Q W^T, the outputs and
//               the one-tile-ahead correction between serial passes
//   waves 3,7   input staging of even / odd tiles (global loads two tiles
//               ahead, LDS layouts); wave 7 also forms the coefficients
//               eta (K K^T) of the serial pass
//   dual form:  the LayerNorm of a tile's independent tokens splits over
//               waves 0 and 7, wave 4 stages the odd tiles and wave 7 writes
//               the outputs back
// The token Gram matrices K Q^T and K_{c+1} K_c^T are formed by the slices
// (bf16 inputs) or by the staging waves (fp32 inputs).
// Per tile c there are two barriers: S_c (z_c and the coefficients are in
// LDS; the serial pass of tile c starts) and G_c (delta_c is in LDS; the
// slices form z_{c+1}).
#include "scan_common.h"

#include <type_traits>

namespace ttt {
namespace {

constexpr int D = 64;
constexpr int BT = 16;      // tokens per tile
constexpr int NWAVES = 8;
constexpr int NT = 64 * NWAVES;
constexpr int RING = 4;     // staged input tiles held in LDS
constexpr int KPAD = 68;    // padded fp32 row (floats) of K/Q/output tiles in LDS
constexpr int ZPAD = 20;    // padded row (floats) of the per-feature z / delta tiles
constexpr int kSerialWave = 0;

// Wave roles.  Wave w runs on SIMD w % 4.  The serial wave shares SIMD 0 only
// with wave 4, which writes outputs back and issues no MFMAs: a wave issuing
// MFMAs on the same SIMD stretches its dependency chain by half, whatever the
// wave priorities.
// The W slices pair up on SIMDs 1 and 2, the staging waves on SIMD 3.  With
// bf16 inputs the slices form their token Gram matrices themselves; with fp32
// inputs, where a 16x16x4 MFMA costs four times the bf16 rate per flop and the
// slices' SIMDs are the busiest, the staging waves form them.
// In the dual form the LayerNorm of a tile splits over waves 0 and 7 (one on
// SIMD 0, one on SIMD 3) and the odd tiles are staged by wave 4 instead.
//
// Output write-back runs on a wave that issues no loads: the staging waves
// wait for their loads of two tiles back with vmcnt, which also counts their
// own stores still in flight.
template <bool BF16, bool DUAL>
struct Roles {
  static constexpr int kStageEven = 3;          // stages even tiles
  static constexpr int kStageOdd = DUAL ? 4 : 7;  // stages odd tiles
  static constexpr int kOutWave = DUAL ? 7 : 4;   // writes outputs back
  static constexpr int kLnHalf = 7;             // dual form: LayerNorm of tokens 8..15
  static constexpr int kCoefWave = 7;           // eta (k.k) of the serial pass
  static constexpr bool kTokInSlices = BF16;    // else: kStageEven forms M, kStageOdd X
  // W row slice owned by a wave, or -1
  __device__ static int slice_of(int wave) {
    return wave == 1 ? 0 : wave == 2 ? 1 : wave == 5 ? 2 : wave == 6 ? 3 : -1;
  }
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float fast_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// two fp32 values to two bf16 (round to nearest even each) in one register,
// a in the low half: one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}
// (a, b) = hi + lo with hi, lo bf16 pairs (round to nearest even each; the
// residual x - hi is exact in fp32)
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16(a, b);
  lo = pack_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u));
}
__device__ __forceinline__ void split4(const float (&x)[4], i16x4& hi, i16x4& lo) {
  uint32_t h01, l01, h23, l23;
  split2(x[0], x[1], h01, l01);
  split2(x[2], x[3], h23, l23);
  hi = __builtin_bit_cast(i16x4, make_uint2(h01, h23));
  lo = __builtin_bit_cast(i16x4, make_uint2(l01, l23));
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
// (a_hi + a_lo)(b_hi + b_lo) without the lo*lo term, accumulated into c
__device__ __forceinline__ f32x4 mfma_k16x3(const i16x4& ah, const i16x4& al, const i16x4& bh,
                                            const i16x4& bl, f32x4 c) {
  c = mfma_k16(ah, bh, c);
  c = mfma_k16(ah, bl, c);
  return mfma_k16(al, bh, c);
}

// ---------------------------------------------------------------------------
// LDS layouts
// ---------------------------------------------------------------------------
// bf16 inputs: K and Q rows in the operand layout of the 16x16x32 MFMA
// (lane l = t + 16G holds, in slot e, column j = 32ks + 16(e/4) + 4G + e%4 of
// row t), K^T in the A layout of the 16x16x16 MFMA (lane l = j%16 + 16G of
// column tile jt holds rows s = 4G + e of column j), v transposed to
// feature-major rows for the serial pass.
struct alignas(16) TileBf16 {
  uint16_t KA[2][64][8];
  uint16_t QA[2][64][8];
  uint16_t KT[4][64][4];   // -K^T in the A layout of the 16x16x16 MFMA
  float VB[D][ZPAD];       // beta_i - v_t[i] (v_t[i] without LayerNorm) at VB[i][t]
  float SG[BT][D];         // sigmoid(gate_logit)
  float ETA[BT];           // sigmoid(eta_logit)/d, 0 for tokens past the end
};
// fp32 inputs: K and Q rows (padded against bank conflicts), v transposed.
struct alignas(16) TileF32 {
  float K[BT][KPAD];
  float Q[BT][KPAD];
  float VB[D][ZPAD];
  float SG[BT][D];
  float ETA[BT];
};

// A operand (t = lane % 16, s = 4 (lane / 16) + e) of a 16 x 16 token matrix,
// held in registers: bf16 hi and lo parts for the 16x16x16 MFMA, or the fp32
// value of k-step e for the 16x16x4 MFMA.
template <bool BF16>
struct TokReg;
template <>
struct TokReg<true> {
  i16x4 hi, lo;
};
template <>
struct TokReg<false> {
  float v[4];
};

// Every member is a multiple of 16 bytes, so the 16-byte alignment of the
// whole lets every float4 access be one 128-bit LDS operation.
template <bool BF16>
struct alignas(16) Smem {
  using Tile = typename std::conditional<BF16, TileBf16, TileF32>::type;
  Tile ring[RING];
  float Zt[D][ZPAD];       // z of the next serial pass, by feature
  float Dt[2][D][ZPAD];    // delta of a tile, by feature
  float Cc[2][BT][BT];     // -eta_s (k_s . k_t) of a tile (negated: the serial pass adds)
  float Cd[2][BT];         // its superdiagonal eta_s (k_s . k_{s+1})
  float Mg[2][BT][ZPAD];   // -(k_s . q_t), s <= t, of a tile, at [t][s]
  float Xg[BT][ZPAD];      // -(k_s . k'_t) of a tile and the next one, at [t][s]
  float Ob[2][BT][KPAD];   // gated outputs awaiting write-back
};

// ---------------------------------------------------------------------------
// input staging (one wave): global loads into registers, then LDS layouts
// ---------------------------------------------------------------------------
template <bool BF16>
struct Stage {
  static constexpr int kVE = BF16 ? 8 : 4;             // elements per 16-byte vector
  static constexpr int kPerLane = BT * D / kVE / 64;   // vectors per lane per array
  uint4 v[4][kPerLane];                                // q, k, v, gate
  uint32_t eta;                                        // raw bits
};

// The array loop is unrolled, so each base pointer is a kernel argument and
// the loads issue as global loads (counted by vmcnt only).
// skip: the tile is a skipped chunk (the dual form's chunk is the tile); it
// needs only q and the gate, so its keys and values stay zero and are not
// read from memory, and its eta_logit is -inf
template <bool BF16>
__device__ __forceinline__ void load_tile(Stage<BF16>& st, const void* const src[4],
                                          const void* etap, int64_t bhT, int64_t t0, int64_t T,
                                          int lane, bool skip) {
  using In = typename std::conditional<BF16, uint16_t, float>::type;
  using S = Stage<BF16>;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const In* base = static_cast<const In*>(src[a]) + (bhT + t0) * D;
#pragma unroll
    for (int r = 0; r < S::kPerLane; ++r) {
      const int vid = lane + 64 * r;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (t0 + (vid * S::kVE) / D < T && !(skip && (a == 1 || a == 2)))
        x = *reinterpret_cast<const uint4*>(base + vid * S::kVE);
      st.v[a][r] = x;
    }
  }
  st.eta = 0u;
  if (lane < BT && t0 + lane < T) {
    // a skipped chunk: eta_logit = -inf, whose sigmoid is exactly 0
    if (skip) {
      st.eta = BF16 ? 0xFF80u : 0xFF800000u;
    } else {
      const In* e = static_cast<const In*>(etap) + bhT + t0 + lane;
      if constexpr (BF16)
        st.eta = *e;
      else
        st.eta = __float_as_uint(*e);
    }
  }
}

// sb[e]: beta of feature j0 + e (the same features for every vector of a
// lane), or 0 without LayerNorm, where VB holds v itself.
// silu(x) = x sigmoid(x) on two packed bf16 values, each result rounded to bf16
__device__ __forceinline__ uint32_t silu_bf16x2(uint32_t w) {
  const float a = __uint_as_float(w << 16), b = __uint_as_float(w & 0xFFFF0000u);
  return pack_bf16(a * fast_sigmoid(a), b * fast_sigmoid(b));
}

// silu: the :mlp variant's SiLU on q and k (on the bf16 path the activated
// values are rounded back to bf16, the matrix cores' operand type)
// skip: a skipped chunk's keys and values are never read, so they are not stored
template <bool BF16, int LN>
__device__ __forceinline__ void store_tile(const Stage<BF16>& st,
                                           typename Smem<BF16>::Tile& tl, int64_t t0, int64_t T,
                                           int lane, const float (&sb)[Stage<BF16>::kVE],
                                           bool silu, bool skip = false) {
  using S = Stage<BF16>;
  auto vb = [&](float v, int e) { return LN == kLnNone ? v : sb[e] - v; };
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    if (skip && (a == 1 || a == 2)) continue;
#pragma unroll
    for (int r = 0; r < S::kPerLane; ++r) {
      const int vid = lane + 64 * r;
      const int t = (vid * S::kVE) / D;
      const int j0 = (vid * S::kVE) % D;
      uint4 x = st.v[a][r];
      if constexpr (BF16) {
        if (silu && a <= 1)
          x = make_uint4(silu_bf16x2(x.x), silu_bf16x2(x.y), silu_bf16x2(x.z), silu_bf16x2(x.w));
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
        if (a <= 1) {
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
              tl.KT[j / 16][(j % 16) + 16 * (t / 4)][t % 4] = bits ^ 0x8000u;   // -k
            else
              tl.VB[j][t] = vb(__uint_as_float(static_cast<uint32_t>(bits) << 16), e);
          }
        }
        if (a == 3) {
          float f[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            f[2 * i] = fast_sigmoid(__uint_as_float(w[i] << 16));
            f[2 * i + 1] = fast_sigmoid(__uint_as_float(w[i] & 0xFFFF0000u));
          }
          *reinterpret_cast<float4*>(&tl.SG[t][j0]) = make_float4(f[0], f[1], f[2], f[3]);
          *reinterpret_cast<float4*>(&tl.SG[t][j0 + 4]) = make_float4(f[4], f[5], f[6], f[7]);
        }
      } else {
        float4 f = make_float4(__uint_as_float(x.x), __uint_as_float(x.y),
                               __uint_as_float(x.z), __uint_as_float(x.w));
        if (silu && a <= 1)
          f = make_float4(f.x * fast_sigmoid(f.x), f.y * fast_sigmoid(f.y),
                          f.z * fast_sigmoid(f.z), f.w * fast_sigmoid(f.w));
        if (a == 0) *reinterpret_cast<float4*>(&tl.Q[t][j0]) = f;
        if (a == 1) *reinterpret_cast<float4*>(&tl.K[t][j0]) = f;
        if (a == 2) {
          tl.VB[j0][t] = vb(f.x, 0);
          tl.VB[j0 + 1][t] = vb(f.y, 1);
          tl.VB[j0 + 2][t] = vb(f.z, 2);
          tl.VB[j0 + 3][t] = vb(f.w, 3);
        }
        if (a == 3)
          *reinterpret_cast<float4*>(&tl.SG[t][j0]) =
              make_float4(fast_sigmoid(f.x), fast_sigmoid(f.y), fast_sigmoid(f.z),
                          fast_sigmoid(f.w));
      }
    }
  }
  if (lane < BT) {
    const float x = BF16 ? __uint_as_float(st.eta << 16) : __uint_as_float(st.eta);
    tl.ETA[lane] = (t0 + lane < T) ? fast_sigmoid(x) * (1.0f / D) : 0.0f;
  }
}

// ---------------------------------------------------------------------------
// the serial LayerNorm pass (one wave, lane = feature i)
// ---------------------------------------------------------------------------
// Step K of a sum over the 64 lanes of a wave: an inclusive scan inside each
// 16-lane row (row_shr 1, 2, 4, 8; out-of-row sources add zero), then
// row_bcast:15 and row_bcast:31.  After the six steps lane 63 holds the total
// (rows 1 and 3 pick up the rows below them, then rows 2 and 3 pick up lane
// 31); the other lanes hold partial sums that are never read.
template <int K>
__device__ __forceinline__ float red_step(float x) {
  // not contracted into the producer of x (z*z + dpp(z*z) would become a
  // dpp move plus an fma, one more step on the chain)
#pragma clang fp contract(off)
  constexpr int kCtrl[6] = {0x111, 0x112, 0x114, 0x118, 0x142, 0x143};
  return x + __int_as_float(
                 __builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl[K], 0xF, 0xF, true));
}
__device__ __forceinline__ float lane63(float x) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
// x minus its value in lane 0: the LayerNorm is invariant to a common shift of
// z, and a shift by one of the token's own entries keeps the sums of the
// shifted values within a few standard deviations of zero, so that the
// one-pass variance E[y^2] - E[y]^2 does not cancel when |mean(z)| >> std(z)
__device__ __forceinline__ float shift_by_lane0(float x) {
  return x - __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// The two sums of the straight-through LayerNorm in one register: a
// v_permlane32_swap of (a, b) plus an add leaves a of lanes l and l + 32 in
// lane l < 32 and b of lanes l - 32 and l in lane l >= 32; the row scans and
// row_bcast:15 (steps 0 .. 4 above) then sum each half, so that lane 31 holds
// the total of a and lane 63 that of b.  Seven instructions on the chain
// instead of twelve for two interleaved full sums.
__device__ __forceinline__ float pair_step0(float a, float b) {
#pragma clang fp contract(off)
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float lane31(float x) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
}
__device__ __forceinline__ void wave_pair_total(float& a, float& b) {
  float r = pair_step0(a, b);
  r = red_step<0>(r); r = red_step<1>(r); r = red_step<2>(r); r = red_step<3>(r);
  r = red_step<4>(r);
  a = lane31(r);
  b = lane63(r);
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

// delta for one token from y (lane = feature i) and the wave sums s1 = sum y,
// s2 = sum y^2, where y = z - c is z shifted by one of its own entries c (the
// LayerNorm of y equals that of z).  The mean of y, s1/d, is a few standard
// deviations at most, so with the exact power-of-two scalings
// Q := d s2 - s1^2 + d^2 eps = d^2 (var + eps) the difference does not cancel,
// and Q >= d^2 eps up to rounding, so |Q| guards the square root at no cost (a
// source modifier).  The terms that do not depend on the sums are formed off
// the critical path.
// Straight-through form: gz = d gamma_i y, bv = beta_i - v_t[i], and
// delta = rsqrt(Q) (d gamma_i y - gamma_i s1) + bv.
// Exact form: gz = gamma_i^2, bv = gamma_i (beta_i - v_t[i]); with
// x = (y - s1/d) rsqrt(var + eps) and g = gamma_i (gamma_i x + beta_i - v_t[i])
// = gz x + bv, delta = rsqrt(var + eps) (g - mean(g) - x mean(g x)), the two
// means from a second round of wave sums.
template <int LN>
__device__ __forceinline__ float delta_from_sums(float z, float gz, float s1, float s2, float bv,
                                                 float gam, float eps) {
  if constexpr (LN == kLnST) {
    const float c = fmaf(-s1, s1, float(D * D) * eps);
    const float q = fmaf(s2, float(D), c);
    return fmaf(__builtin_amdgcn_rsqf(fabsf(q)), fmaf(-gam, s1, gz), bv);
  } else {
    const float a = s1 * (1.0f / D);
    const float c = fmaf(-s1, s1, float(D * D) * eps);
    const float q = fmaf(s2, float(D), c);
    const float rs = float(D) * __builtin_amdgcn_rsqf(fabsf(q));
    const float xh = (z - a) * rs;
    const float g = fmaf(gz, xh, bv);
    float sg = g, sgx = g * xh;
    wave_total2(sg, sgx);
    return rs * fmaf(-xh, sgx * (1.0f / D), fmaf(sg, -1.0f / D, g));
  }
}

// delta for one token from z (lane = feature i); bv = beta_i - v_t[i] (v_t[i]
// without LayerNorm).
template <int LN>
__device__ __forceinline__ float token_delta(float z, float bv, float gam, float eps) {
  if constexpr (LN == kLnNone) {
    return z - bv;
  } else {
    const float y = shift_by_lane0(z);
    float s1 = y, s2 = y * y;
    if constexpr (LN == kLnST) {
      wave_pair_total(s1, s2);
      return delta_from_sums<LN>(y, (gam * float(D)) * y, s1, s2, bv, gam, eps);
    } else {
      wave_total2(s1, s2);
      return delta_from_sums<LN>(y, gam * gam, s1, s2, gam * bv, gam, eps);
    }
  }
}

// The serial pass over one tile.  zq[t / 4][t % 4] = (W_c k_t)_i on entry
// (lane = feature i; the 16 rows as four 4-row groups); cc points at the
// negated coefficients -eta_s (k_s . k_t) in LDS (row s, column t) and cd[s]
// holds the superdiagonal eta_s (k_s . k_{s+1}) in registers.  Token s's delta
// is applied to row s+1 at once.  Its updates of rows s+2.. are made during
// token s+1: the rows of the 4-row group that holds row s+2 on the vector ALU
// (coefficients broadcast from LDS), and each later group with one
// v_mfma_f32_4x4x1f32.  That product's 16 blocks put lane 4b + j in block b,
// column j, so with A = the lane pattern -eta_s (k_s . k_{4g + lane % 4}),
// B = delta_s (lane = feature) and C = D = the group's four row registers it
// is exactly the four updates zq[g][i] += A[4g + i] delta_s[lane], one issue
// slot instead of four.  A group is a product target only while every row in
// it lies two or more tokens ahead, so the vector ALU touches its rows no
// sooner than a token after its last product.  Coefficient rows are read two
// tokens ahead of their use.  Row s+1 is shifted by its lane-0 entry before
// token s's own correction, so off the dependency chain (with the
// straight-through form, possibly before the last of the deferred updates
// reach it: any common shift leaves the LayerNorm unchanged, and a lane-0
// entry a few updates old still keeps the mean of the shifted row within a few
// standard deviations); the LayerNorm of token s+1 then runs on the shifted
// row.
template <int LN>
__device__ __forceinline__ void serial_tile(f32x4 (&zq)[4], const float (&bv)[BT],
                                            const float* cc, int lane,
                                            const float (&cd)[BT], float gam, float eps,
                                            float (&dr)[BT]) {
  // Row r of the coefficients (used in token r + 1, for the rows r + 2 ..):
  // cq = its entries in the group g0 = (r + 2) / 4 (broadcast), cp[g - g0 - 1]
  // = its lane pattern for each later group g.  Rows r - 1 .. r + 2 in a ring.
  float4 cq[4];
  float cp[4][3];
  const float* ap = cc + (lane & 3);
  auto load_row = [&](int r) {
    const int g0 = (r + 2) >> 2;
    cq[r % 4] = *reinterpret_cast<const float4*>(&cc[r * BT + 4 * g0]);
#pragma unroll
    for (int g = g0 + 1; g < 4; ++g) cp[r % 4][g - g0 - 1] = ap[r * BT + 4 * g];
  };
  load_row(0);
  load_row(1);
  const float gam_d = gam * float(D);
  if constexpr (LN != kLnNone) zq[0][0] = shift_by_lane0(zq[0][0]);
  float dprev = 0.0f;
#pragma unroll
  for (int s = 0; s < BT; ++s) {
    // the row loads stay at the top of their token: left to itself the
    // scheduler sinks them next to their use and the wait lands on the chain
    __builtin_amdgcn_sched_barrier(0);
    if (s + 2 < BT - 2) load_row(s + 2);
    __builtin_amdgcn_sched_barrier(0);
    const float z = zq[s >> 2][s & 3];
    // the deferred updates of delta_{s-1} (rows s+1 ..), in six slots: slot 0
    // takes row s+1 (needed first) and the group products, slots 1 .. 3 the
    // other vector-ALU rows of row s+1's group
    constexpr int kSlots = 6;
    auto fill = [&](int k) {
      if (s == 0 || s + 1 >= BT) return;
      const int r = s - 1, g0 = (s + 1) >> 2;
      const float4 c4 = cq[r % 4];
      const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
      const int t = s + 1 + k;
      if (k < 4 && t <= 4 * g0 + 3) zq[g0][t & 3] = fmaf(cv[t & 3], dprev, zq[g0][t & 3]);
      if (k == 0) {
#pragma unroll
        for (int g = g0 + 1; g < 4; ++g)
          zq[g] = __builtin_amdgcn_mfma_f32_4x4x1f32(cp[r % 4][g - g0 - 1], dprev, zq[g], 0, 0,
                                                     0);
      }
    };
    float dl;
    if constexpr (LN == kLnNone) {
#pragma unroll
      for (int k = 0; k < kSlots; ++k) fill(k);
      dl = z - bv[s];
    } else {
      float a = z, b = z * z;
      if constexpr (LN == kLnST) {
        // two interleaved sums (each fills the other's DPP wait states; the
        // pairing through one lane-half swap that the dual form uses is two
        // dependent steps longer, which shows here, where the chain's latency
        // sets the pace), the deferred updates in the remaining gaps, and row
        // s+1 shifted early, so that its correction by delta_s below waits for
        // delta_s alone
        const float gz = gam_d * z;
        a = red_step<0>(a); b = red_step<0>(b); fill(0);
        a = red_step<1>(a); b = red_step<1>(b);
        a = red_step<2>(a); b = red_step<2>(b); fill(1);
        a = red_step<3>(a); b = red_step<3>(b);
        a = red_step<4>(a); b = red_step<4>(b); fill(2);
        if (s + 1 < BT) zq[(s + 1) >> 2][(s + 1) & 3] = shift_by_lane0(zq[(s + 1) >> 2][(s + 1) & 3]);
        a = red_step<5>(a); b = red_step<5>(b);
        const float s1 = lane63(a), s2 = lane63(b);
        fill(3);
        const float c = fmaf(-s1, s1, float(D * D) * eps);
        const float q = fmaf(s2, float(D), c);
        fill(4);
        const float rq = __builtin_amdgcn_rsqf(fabsf(q));
        fill(5);
        dl = fmaf(rq, fmaf(-gam, s1, gz), bv[s]);
      } else {
        const float g2 = gam * gam;
        const float gbv = gam * bv[s];
        // the exact form's two rounds of sums (delta_from_sums written out),
        // the deferred updates spread over both
        a = red_step<0>(a); b = red_step<0>(b); fill(0);
        a = red_step<1>(a); b = red_step<1>(b);
        if (s + 1 < BT) zq[(s + 1) >> 2][(s + 1) & 3] = shift_by_lane0(zq[(s + 1) >> 2][(s + 1) & 3]);
        a = red_step<2>(a); b = red_step<2>(b); fill(1);
        a = red_step<3>(a); b = red_step<3>(b);
        a = red_step<4>(a); b = red_step<4>(b); fill(2);
        a = red_step<5>(a); b = red_step<5>(b);
        const float s1 = lane63(a), s2 = lane63(b);
        const float am = s1 * (1.0f / D);
        const float c = fmaf(-s1, s1, float(D * D) * eps);
        const float q = fmaf(s2, float(D), c);
        const float rs = float(D) * __builtin_amdgcn_rsqf(fabsf(q));
        const float xh = (z - am) * rs;
        const float g = fmaf(g2, xh, gbv);
        float sg = g, sgx = g * xh;
        sg = red_step<0>(sg); sgx = red_step<0>(sgx); fill(3);
        sg = red_step<1>(sg); sgx = red_step<1>(sgx);
        sg = red_step<2>(sg); sgx = red_step<2>(sgx); fill(4);
        sg = red_step<3>(sg); sgx = red_step<3>(sgx);
        sg = red_step<4>(sg); sgx = red_step<4>(sgx); fill(5);
        sg = red_step<5>(sg); sgx = red_step<5>(sgx);
        // both lane reads first (two scalar registers: a read used at once
        // stalls the chain on its hazard)
        sg = lane63(sg);
        sgx = lane63(sgx);
        dl = rs * fmaf(-xh, sgx * (1.0f / D), fmaf(sg, -1.0f / D, g));
      }
    }
    dr[s] = dl;
    if (s + 1 < BT)
      zq[(s + 1) >> 2][(s + 1) & 3] = fmaf(-cd[s], dl, zq[(s + 1) >> 2][(s + 1) & 3]);
    dprev = dl;
  }
}

// What the serial wave holds for a tile before its pass: beta - v (v without
// LayerNorm) and the superdiagonal coefficients eta_s (k_s . k_{s+1}), read
// while the W slices form z.
struct SerialIn {
  float cd[BT];
  float bv[BT];
};

template <bool BF16>
__device__ __forceinline__ void serial_prefetch(SerialIn& in, const typename Smem<BF16>::Tile& tl,
                                                const float* cd, int lane) {
#pragma unroll
  for (int q4 = 0; q4 < BT / 4; ++q4) {
    const float4 x = *reinterpret_cast<const float4*>(&tl.VB[lane][4 * q4]);
    in.bv[4 * q4] = x.x; in.bv[4 * q4 + 1] = x.y; in.bv[4 * q4 + 2] = x.z; in.bv[4 * q4 + 3] = x.w;
    const float4 y = *reinterpret_cast<const float4*>(&cd[4 * q4]);
    in.cd[4 * q4] = y.x; in.cd[4 * q4 + 1] = y.y; in.cd[4 * q4 + 2] = y.z; in.cd[4 * q4 + 3] = y.w;
  }
}

// One serial (or, in the dual form, parallel) LayerNorm pass: z from Zt,
// delta into dt.
template <bool BF16, int LN, bool DUAL>
__device__ __forceinline__ void ln_pass(Smem<BF16>& sm, const SerialIn& in, const float (*cc)[BT],
                                        float (*dt)[ZPAD], int lane, float gam, float eps) {
  f32x4 zq[BT / 4];
  float dr[BT];
#pragma unroll
  for (int q4 = 0; q4 < BT / 4; ++q4) {
    const float4 x = *reinterpret_cast<const float4*>(&sm.Zt[lane][4 * q4]);
    zq[q4] = f32x4{x.x, x.y, x.z, x.w};
  }
  static_assert(!DUAL, "the dual form runs dual_ln_pass");
  serial_tile<LN>(zq, in.bv, &cc[0][0], lane, in.cd, gam, eps, dr);
#pragma unroll
  for (int q4 = 0; q4 < BT / 4; ++q4)
    *reinterpret_cast<float4*>(&dt[lane][4 * q4]) =
        make_float4(dr[4 * q4], dr[4 * q4 + 1], dr[4 * q4 + 2], dr[4 * q4 + 3]);
}

// The dual form's tokens are independent: two waves on different SIMDs each
// take half a tile (tokens t0 .. t0+7).
struct DualIn {
  float bv[BT / 2];
};

template <bool BF16>
__device__ __forceinline__ void dual_prefetch(DualIn& in, const typename Smem<BF16>::Tile& tl,
                                              int lane, int t0) {
#pragma unroll
  for (int q4 = 0; q4 < 2; ++q4) {
    const float4 x = *reinterpret_cast<const float4*>(&tl.VB[lane][t0 + 4 * q4]);
    in.bv[4 * q4] = x.x; in.bv[4 * q4 + 1] = x.y; in.bv[4 * q4 + 2] = x.z; in.bv[4 * q4 + 3] = x.w;
  }
}

template <bool BF16, int LN>
__device__ __forceinline__ void dual_ln_pass(Smem<BF16>& sm, const DualIn& in, float (*dt)[ZPAD],
                                             int lane, int t0, float gam, float eps) {
  float zr[BT / 2], dr[BT / 2];
#pragma unroll
  for (int q4 = 0; q4 < 2; ++q4) {
    const float4 x = *reinterpret_cast<const float4*>(&sm.Zt[lane][t0 + 4 * q4]);
    zr[4 * q4] = x.x; zr[4 * q4 + 1] = x.y; zr[4 * q4 + 2] = x.z; zr[4 * q4 + 3] = x.w;
  }
#pragma unroll
  for (int t = 0; t < BT / 2; ++t) dr[t] = token_delta<LN>(zr[t], in.bv[t], gam, eps);
#pragma unroll
  for (int q4 = 0; q4 < 2; ++q4)
    *reinterpret_cast<float4*>(&dt[lane][t0 + 4 * q4]) =
        make_float4(dr[4 * q4], dr[4 * q4 + 1], dr[4 * q4 + 2], dr[4 * q4 + 3]);
}

// ---------------------------------------------------------------------------
// products of a W slice
// ---------------------------------------------------------------------------
// bf16 hi/lo B operands of W^T for the two 32-deep k-steps
struct WOps {
  bf16x8 hi[2], lo[2];
};
__device__ __forceinline__ WOps split_w(const f32x4 (&Wt)[4]) {
  WOps w;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const f32x4& x = Wt[2 * ks + p / 2];
      split2(x[2 * (p % 2)], x[2 * (p % 2) + 1], h[p], l[p]);
    }
    w.hi[ks] = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
    w.lo[ks] = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
  }
  return w;
}

// rows (k or q) of a tile times W^T -> [token][feature slice] accumulator
__device__ __forceinline__ f32x4 rows_times_wt(const uint16_t (*A)[64][8], const WOps& w,
                                               int lane) {
  f32x4 acc = {0, 0, 0, 0};
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(&A[ks][lane][0]);
    acc = mfma_k32(a, w.hi[ks], acc);
    acc = mfma_k32(a, w.lo[ks], acc);
  }
  return acc;
}
__device__ __forceinline__ f32x4 rows_times_wt(const float (*A)[KPAD], const f32x4 (&Wt)[4],
                                               int l16, int G) {
  f32x4 acc = {0, 0, 0, 0};
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    const float4 a = *reinterpret_cast<const float4*>(&A[l16][16 * jt + 4 * G]);
    acc = mfma_k4(a.x, Wt[jt][0], acc);
    acc = mfma_k4(a.y, Wt[jt][1], acc);
    acc = mfma_k4(a.z, Wt[jt][2], acc);
    acc = mfma_k4(a.w, Wt[jt][3], acc);
  }
  return acc;
}

// acc += A (16 x 16 token matrix) times B[s][slice feature], B = b[e] for s = 4G + e
__device__ __forceinline__ f32x4 tok_mul(const TokReg<true>& a, const TokReg<true>& b, f32x4 acc) {
  return mfma_k16x3(a.hi, a.lo, b.hi, b.lo, acc);
}
__device__ __forceinline__ f32x4 tok_mul(const TokReg<false>& a, const TokReg<false>& b,
                                         f32x4 acc) {
  acc = mfma_k4(a.v[0], b.v[0], acc);
  acc = mfma_k4(a.v[1], b.v[1], acc);
  acc = mfma_k4(a.v[2], b.v[2], acc);
  return mfma_k4(a.v[3], b.v[3], acc);
}
__device__ __forceinline__ void make_tok(TokReg<true>& a, const float (&x)[4]) {
  split4(x, a.hi, a.lo);
}
__device__ __forceinline__ void make_tok(TokReg<false>& a, const float (&x)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) a.v[e] = x[e];
}

// Wt[jt] -= sum_s K[s][16jt + i] E[s][slice feature], E = eta * delta as the
// B operand of tok_mul (the bf16 tile holds K^T negated)
__device__ __forceinline__ void update_w(f32x4 (&Wt)[4], const TileBf16& tl, const TokReg<true>& e,
                                         int lane, int, int) {
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    const i16x4 nkt = *reinterpret_cast<const i16x4*>(&tl.KT[jt][lane][0]);
    Wt[jt] = mfma_k16(nkt, e.hi, Wt[jt]);
    Wt[jt] = mfma_k16(nkt, e.lo, Wt[jt]);
  }
}
__device__ __forceinline__ void update_w(f32x4 (&Wt)[4], const TileF32& tl,
                                         const TokReg<false>& e, int, int l16, int G) {
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
    for (int q = 0; q < 4; ++q) Wt[jt] = mfma_k4(tl.K[4 * G + q][16 * jt + l16], -e.v[q], Wt[jt]);
  }
}

// ---------------------------------------------------------------------------
// Gram matrices of two staged tiles: D[s][t] = a_s . b_t, at lane
// (s = 4G + r, t = l16), r = 0..3 -- the A layout of the 16 x 16 matrix D^T
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 gram(const uint16_t (*A)[64][8], const uint16_t (*B)[64][8],
                                      int lane, int, int) {
  f32x4 acc = {0, 0, 0, 0};
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    acc = mfma_k32(*reinterpret_cast<const bf16x8*>(&A[ks][lane][0]),
                   *reinterpret_cast<const bf16x8*>(&B[ks][lane][0]), acc);
  return acc;
}
__device__ __forceinline__ f32x4 gram(const float (*A)[KPAD], const float (*B)[KPAD], int,
                                      int l16, int G) {
  f32x4 acc = {0, 0, 0, 0};
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    const float4 a = *reinterpret_cast<const float4*>(&A[l16][16 * jt + 4 * G]);
    const float4 b = *reinterpret_cast<const float4*>(&B[l16][16 * jt + 4 * G]);
    acc = mfma_k4(a.x, b.x, acc);
    acc = mfma_k4(a.y, b.y, acc);
    acc = mfma_k4(a.z, b.z, acc);
    acc = mfma_k4(a.w, b.w, acc);
  }
  return acc;
}
__device__ __forceinline__ const uint16_t (*krows(const TileBf16& t))[64][8] { return t.KA; }
__device__ __forceinline__ const uint16_t (*qrows(const TileBf16& t))[64][8] { return t.QA; }
__device__ __forceinline__ const float (*krows(const TileF32& t))[KPAD] { return t.K; }
__device__ __forceinline__ const float (*qrows(const TileF32& t))[KPAD] { return t.Q; }

// write back the gated outputs of one tile (one wave, 16-byte stores)
__device__ __forceinline__ void write_tile_out(const float (*ob)[KPAD], float* out, int64_t bhT,
                                               int64_t t0, int64_t T, int lane) {
  const int rows = static_cast<int>(min<int64_t>(BT, T - t0));
  float* dst = out + (bhT + t0) * D;
#pragma unroll
  for (int k = 0; k < BT * D / 4 / 64; ++k) {
    const int i = lane + 64 * k;
    const int t = i / (D / 4), c4 = i % (D / 4);
    if (t < rows)
      *reinterpret_cast<float4*>(dst + t * D + 4 * c4) =
          *reinterpret_cast<const float4*>(&ob[t][4 * c4]);
  }
}

// ---------------------------------------------------------------------------
// REC: also record delta_t and W at the start of every tile (for the backward;
// in the dual form the tiles are the chunks).  MASK (dual form only): one
// SKIP/UPDATE decision per chunk in upd_mask; a skipped chunk applies no
// update (eta = 0), so only its outputs (W_c q_t) sigmoid(gate_t) are formed:
// its keys, values and eta are not loaded, and its z, LayerNorm pass, key
// Gram matrices, in-chunk correction and W update are left out.
template <bool BF16, int LN, bool DUAL, bool REC, bool MASK = false>
__global__ void __launch_bounds__(NT)
scan_mfma_kernel(const void* __restrict__ qp, const void* __restrict__ kp,
                 const void* __restrict__ vp, const void* __restrict__ etap,
                 const void* __restrict__ gatep, const float* __restrict__ W0,
                 const float* __restrict__ gamma, const float* __restrict__ beta,
                 float* __restrict__ out, float* __restrict__ W_final, int H, int64_t T,
                 float eps, float* __restrict__ rec_delta, float* __restrict__ rec_W,
                 const uint8_t* __restrict__ upd_mask, int silu) {
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
  const int64_t ntiles = (T + BT - 1) / BT;
  using R = Roles<BF16, DUAL>;
  static_assert(!MASK || (DUAL && !REC), "the chunk mask is a dual-form forward option");
  const uint8_t* mrow = MASK ? upd_mask + bh * ntiles : nullptr;
  // The decisions of tiles wb .. wb+127 as two 64-bit words (bit i of mw0:
  // tile wb + i is skipped; mw1: tile wb + 64 + i), formed by a ballot over
  // the wave's lanes; moved on by 64 tiles once tile wb + 64 is the oldest
  // one a period asks about.  No decision is read from memory inside a period.
  int64_t wb = 0;
  uint64_t mw0 = 0, mw1 = 0;
  auto mask_bits = [&](int64_t base) -> uint64_t {
    const int64_t u = base + lane;
    return __ballot(u < ntiles && mrow[u] == 0);
  };
  if constexpr (MASK) {
    mw0 = mask_bits(0);
    mw1 = mask_bits(64);
  }
  // whether tile u (wb <= u < wb + 128) is a skipped chunk (never, without the mask)
  auto skipped = [&](int64_t u) -> bool {
    if constexpr (!MASK) {
      return false;
    } else {
      const int64_t i = u - wb;
      return i < 64 ? ((mw0 >> i) & 1) != 0 : ((mw1 >> (i - 64)) & 1) != 0;
    }
  };
  const int slice = R::slice_of(wave);
  const int irow = 16 * slice + l16;   // W row (feature i) held by this lane, slice waves

  // slice waves: W^T tiles, Wt[jt][r] = W[irow][16 jt + 4G + r]; P, U accumulators
  f32x4 Wt[4] = {};
  f32x4 P = {0, 0, 0, 0}, U = {0, 0, 0, 0};
  TokReg<BF16> Mreg{}, Xreg{};   // slices forming their own token matrices: M and X below
  // LayerNorm waves: the serial wave (the dual form: it and the odd staging
  // wave, half a tile each); LayerNorm affine of feature `lane`, and the
  // inputs of the next tile
  const int ln_half = wave == kSerialWave ? 0 : (DUAL && wave == R::kLnHalf) ? 1 : -1;
  const int ln_t0 = (BT / 2) * ln_half;
  float gam = 1.0f;
  SerialIn sin;
  DualIn din;
  Stage<BF16> st;   // staging waves: the tile in flight

  if (slice >= 0) {
    const float* w = W0 + bh * D * D + irow * D + 4 * G;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      const float4 x = *reinterpret_cast<const float4*>(w + 16 * jt);
      Wt[jt] = f32x4{x.x, x.y, x.z, x.w};
    }
  }
  if (ln_half >= 0 && LN != kLnNone) gam = gamma[h * D + lane];
  __builtin_amdgcn_s_waitcnt(0);
  // staging prologue: tiles 0 and 1 into LDS, tiles 2 and 3 in flight
  const int stage_parity = wave == R::kStageEven ? 0 : wave == R::kStageOdd ? 1 : -1;
  // staging lanes: beta of the features their vectors of v cover
  float sb[Stage<BF16>::kVE] = {};
  if (stage_parity >= 0 && LN != kLnNone) {
    constexpr int kVE = Stage<BF16>::kVE;
#pragma unroll
    for (int e = 0; e < kVE; ++e) sb[e] = beta[h * D + (lane * kVE) % D + e];
  }
  if (stage_parity >= 0) {
    const int u = stage_parity;
    if (u < ntiles) {
      load_tile<BF16>(st, src, etap, bhT, u * BT, T, lane, skipped(u));
      store_tile<BF16, LN>(st, sm.ring[u], u * BT, T, lane, sb, silu != 0, skipped(u));
    }
    if (u + 2 < ntiles)
      load_tile<BF16>(st, src, etap, bhT, (u + 2) * BT, T, lane, skipped(u + 2));
  }
  __syncthreads();
  // z of tile 0 and its coefficients
  if (slice >= 0 && ntiles > 0) {
    f32x4 Z;
    if constexpr (BF16)
      Z = rows_times_wt(krows(sm.ring[0]), split_w(Wt), lane);
    else
      Z = rows_times_wt(krows(sm.ring[0]), Wt, l16, G);
    *reinterpret_cast<float4*>(&sm.Zt[irow][4 * G]) = make_float4(Z[0], Z[1], Z[2], Z[3]);
  }
  if (!DUAL && wave == R::kCoefWave && ntiles > 0) {
    const auto& t0 = sm.ring[0];
    const f32x4 g = gram(krows(t0), krows(t0), lane, l16, G);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float cv = t0.ETA[4 * G + r] * g[r];
      sm.Cc[0][4 * G + r][l16] = -cv;
      if (4 * G + r + 1 == l16) sm.Cd[0][4 * G + r] = cv;
    }
  }

  // M = -(k_s . q_t), s <= t: with E = eta * delta, the in-tile part of the
  // outputs of tile c is M E
  auto tok_m = [&](const typename Smem<BF16>::Tile& tc, float (&m)[4]) {
    const f32x4 kq = gram(krows(tc), qrows(tc), lane, l16, G);
#pragma unroll
    for (int r = 0; r < 4; ++r) m[r] = (4 * G + r <= l16) ? -kq[r] : 0.0f;
  };
  // E = eta_s delta_s[i] of a tile for the slice's features, as a B operand
  auto tok_e = [&](int64_t c) {
    const auto& tc = sm.ring[c % RING];
    const float4 d4 = *reinterpret_cast<const float4*>(&sm.Dt[c & 1][irow][4 * G]);
    const float4 e4 = *reinterpret_cast<const float4*>(&tc.ETA[4 * G]);
    const float ev[4] = {e4.x * d4.x, e4.y * d4.y, e4.z * d4.z, e4.w * d4.w};
    TokReg<BF16> e;
    make_tok(e, ev);
    return e;
  };
  TokReg<BF16> Ereg{};   // E of the last tile, formed after its serial pass
  // X = -(k_t(c+1) . k_s(c)): carries delta of tile c into z of tile c+1
  auto tok_x = [&](const typename Smem<BF16>::Tile& tc, const typename Smem<BF16>::Tile& tn,
                   float (&x)[4]) {
    const f32x4 g = gram(krows(tc), krows(tn), lane, l16, G);
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = -g[r];
  };

  for (int64_t c = 0; c <= ntiles; ++c) {
    __syncthreads();   // S_c
    if constexpr (MASK) {
      // a period asks about tiles c-1 .. c+3
      if (c - 1 == wb + 64) {
        wb += 64;
        mw0 = mw1;
        mw1 = mask_bits(wb + 64);
      }
    }
    const bool live = c < ntiles;
    const bool skip_p = c >= 1 && skipped(c - 1), skip_c = skipped(c), skip_n = skipped(c + 1);
    if (DUAL && ln_half >= 0 && live && !skip_c) {
      if (c == 0) dual_prefetch<BF16>(din, sm.ring[0], lane, ln_t0);
      dual_ln_pass<BF16, LN>(sm, din, sm.Dt[c & 1], lane, ln_t0, gam, eps);
    }
    if (wave == kSerialWave) {
      if constexpr (!DUAL) {
        if (live) {
          if (c == 0) serial_prefetch<BF16>(sin, sm.ring[0], sm.Cd[0], lane);
          ln_pass<BF16, LN, DUAL>(sm, sin, sm.Cc[c & 1], sm.Dt[c & 1], lane, gam, eps);
        }
      }
    } else if (slice >= 0) {
      // One straight block, so the MFMA chains of its independent parts can
      // interleave: the token Gram matrices of tile c, the outputs of tile
      // c-1 and the update W_c = W_{c-1} - E_{c-1}^T K_{c-1}, then
      // K_{c+1} W_c^T (for z of the next tile) and Q_c W_c^T.  At c = 0 there
      // is no previous tile: the outputs written to Ob[1] are overwritten
      // before they are read, and the update is skipped (its ring slot may
      // not hold a tile yet, and a stale NaN times E = 0 would not be 0).  In
      // the last period the products run on a stale ring slot and are not
      // used.  With the mask, a skipped tile's parts are left out.
      if (c == ntiles && !skip_p) Ereg = tok_e(c - 1);   // no z of a next tile was formed
      const auto& tp = sm.ring[(c + RING - 1) % RING];
      const auto& tc = sm.ring[c % RING];
      const auto& tn = sm.ring[(c + 1) % RING];
      TokReg<BF16> Mn{}, Xn{};
      if constexpr (R::kTokInSlices) {
        if (!skip_c) {
          float m[4];
          tok_m(tc, m);
          make_tok(Mn, m);
        }
        if (!skip_c && !skip_n) {
          float x[4];
          tok_x(tc, tn, x);
          make_tok(Xn, x);
        }
      } else if (!skip_p) {
        const float4 m4 = *reinterpret_cast<const float4*>(&sm.Mg[(c + 1) & 1][l16][4 * G]);
        const float mv[4] = {m4.x, m4.y, m4.z, m4.w};
        make_tok(Mreg, mv);
      }
      if (!skip_p) U = tok_mul(Mreg, Ereg, U);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * G + r;
        sm.Ob[(c + 1) & 1][t][irow] = U[r] * tp.SG[t][irow];
      }
      if (c >= 1 && !skip_p) update_w(Wt, tp, Ereg, lane, l16, G);
      if (REC && live) {
        float* w = rec_W + ((bh * ntiles + c) * D + irow) * D + 4 * G;
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
          *reinterpret_cast<float4*>(w + 16 * jt) =
              make_float4(Wt[jt][0], Wt[jt][1], Wt[jt][2], Wt[jt][3]);
      }
      if constexpr (BF16) {
        const WOps w = split_w(Wt);
        if (!skip_n) P = rows_times_wt(krows(tn), w, lane);
        U = rows_times_wt(qrows(tc), w, lane);
      } else {
        if (!skip_n) P = rows_times_wt(krows(tn), Wt, l16, G);
        U = rows_times_wt(qrows(tc), Wt, l16, G);
      }
      if constexpr (R::kTokInSlices) {
        Mreg = Mn;
        Xreg = Xn;
      }
    } else {
      if (stage_parity >= 0) {
        // a staging wave alternates: tile c+2 into LDS, then (next period)
        // the loads of tile c+3 into the freed registers.  A period that both
        // stores a tile and issues loads holds the next barrier up well past
        // the last wave's arrival.
        if ((c & 1) == stage_parity) {
          if (c + 2 < ntiles)
            store_tile<BF16, LN>(st, sm.ring[(c + 2) % RING], (c + 2) * BT, T, lane, sb,
                                 silu != 0, skipped(c + 2));
        } else if (c + 3 < ntiles) {
          load_tile<BF16>(st, src, etap, bhT, (c + 3) * BT, T, lane, skipped(c + 3));
        }
      }
      if (wave == R::kOutWave && c >= 2)
        write_tile_out(sm.Ob[(c - 2) & 1], out, bhT, (c - 2) * BT, T, lane);
      if (REC && wave == R::kOutWave && c >= 1) {
        const int64_t t0 = (c - 1) * BT;
        const int rows = static_cast<int>(min<int64_t>(BT, T - t0));
        float* dst = rec_delta + (bhT + t0) * D + lane;
        for (int t = 0; t < rows; ++t) dst[t * D] = sm.Dt[(c - 1) & 1][lane][t];
      }
      if constexpr (!R::kTokInSlices) {
        if (wave == R::kStageEven && live && !skip_c) {
          float m[4];
          tok_m(sm.ring[c % RING], m);
          *reinterpret_cast<float4*>(&sm.Mg[c & 1][l16][4 * G]) =
              make_float4(m[0], m[1], m[2], m[3]);
        }
        if (wave == R::kStageOdd && c + 1 < ntiles && !skip_c && !skip_n) {
          float x[4];
          tok_x(sm.ring[c % RING], sm.ring[(c + 1) % RING], x);
          *reinterpret_cast<float4*>(&sm.Xg[l16][4 * G]) = make_float4(x[0], x[1], x[2], x[3]);
        }
      }
      if (!DUAL && wave == R::kCoefWave && c + 1 < ntiles) {
        // eta_s (k_s . k_t) of tile c+1 for its serial pass
        const auto& tn = sm.ring[(c + 1) % RING];
        const float4 f4 = *reinterpret_cast<const float4*>(&tn.ETA[4 * G]);
        const float fe[4] = {f4.x, f4.y, f4.z, f4.w};
        const f32x4 g = gram(krows(tn), krows(tn), lane, l16, G);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float cv = fe[r] * g[r];
          sm.Cc[(c + 1) & 1][4 * G + r][l16] = -cv;
          if (4 * G + r + 1 == l16) sm.Cd[(c + 1) & 1][4 * G + r] = cv;
        }
      }
    }
    __syncthreads();   // G_c
    // the LayerNorm waves load their inputs of tile c+1 while the slices form z
    if (ln_half >= 0 && c + 1 < ntiles && !skip_n) {
      if constexpr (DUAL)
        dual_prefetch<BF16>(din, sm.ring[(c + 1) % RING], lane, ln_t0);
      else
        serial_prefetch<BF16>(sin, sm.ring[(c + 1) % RING], sm.Cd[(c + 1) & 1], lane);
    }
    // z of tile c+1: K_{c+1} W_c^T - (K_{c+1} K_c^T) E_c (E_c of a skipped
    // tile is zero; a skipped tile c+1 needs no z)
    if (slice >= 0 && c + 1 < ntiles) {
      if (!skip_c) Ereg = tok_e(c);
      if (!skip_n) {
        f32x4 Z = P;
        if (!skip_c) {
          if constexpr (!R::kTokInSlices) {
            const float4 x4 = *reinterpret_cast<const float4*>(&sm.Xg[l16][4 * G]);
            const float xv[4] = {x4.x, x4.y, x4.z, x4.w};
            make_tok(Xreg, xv);
          }
          Z = tok_mul(Xreg, Ereg, P);
        }
        *reinterpret_cast<float4*>(&sm.Zt[irow][4 * G]) = make_float4(Z[0], Z[1], Z[2], Z[3]);
      }
    }
  }
  __syncthreads();
  // outputs of the last tile (staged in the final period)
  if (wave == R::kOutWave && ntiles > 0)
    write_tile_out(sm.Ob[(ntiles - 1) & 1], out, bhT, (ntiles - 1) * BT, T, lane);
  if (slice >= 0 && W_final != nullptr) {
    float* w = W_final + bh * D * D + irow * D + 4 * G;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
      *reinterpret_cast<float4*>(w + 16 * jt) =
          make_float4(Wt[jt][0], Wt[jt][1], Wt[jt][2], Wt[jt][3]);
  }
}

template <bool BF16, int LN, bool DUAL>
hipError_t launch_one(const ScanArgs& a, hipStream_t s) {
  if (a.rec_delta != nullptr) {
    hipLaunchKernelGGL((scan_mfma_kernel<BF16, LN, DUAL, true>),
                       dim3(static_cast<unsigned>(a.B * a.H)), dim3(NT), 0, s, a.q, a.k, a.v,
                       a.eta_logit, a.gate_logit, a.W0, a.gamma, a.beta, a.out, a.W_final,
                       static_cast<int>(a.H), a.T, a.eps, a.rec_delta, a.rec_W, a.upd_mask,
                       a.silu_qk ? 1 : 0);
    return hipGetLastError();
  }
  if constexpr (DUAL) {
    if (a.upd_mask != nullptr) {
      hipLaunchKernelGGL((scan_mfma_kernel<BF16, LN, true, false, true>),
                         dim3(static_cast<unsigned>(a.B * a.H)), dim3(NT), 0, s, a.q, a.k, a.v,
                         a.eta_logit, a.gate_logit, a.W0, a.gamma, a.beta, a.out, a.W_final,
                         static_cast<int>(a.H), a.T, a.eps, static_cast<float*>(nullptr),
                         static_cast<float*>(nullptr), a.upd_mask, a.silu_qk ? 1 : 0);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((scan_mfma_kernel<BF16, LN, DUAL, false>), dim3(static_cast<unsigned>(a.B * a.H)),
                     dim3(NT), 0, s, a.q, a.k, a.v, a.eta_logit, a.gate_logit, a.W0, a.gamma,
                     a.beta, a.out, a.W_final, static_cast<int>(a.H), a.T, a.eps,
                     static_cast<float*>(nullptr), static_cast<float*>(nullptr), a.upd_mask,
                     a.silu_qk ? 1 : 0);
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
