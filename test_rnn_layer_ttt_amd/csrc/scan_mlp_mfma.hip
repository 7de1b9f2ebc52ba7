// Matrix-core dual-form chunk scan with the two-layer inner model
// f(x) = W2 silu(W1 x), d = 64, chunks of 16 tokens, bf16 inputs (gfx950).
//
// Inner model: "Edifice.Recurrent.TTT", Options, `:variant` (the `:mlp`
// variant makes the hidden state a two-layer MLP with SiLU) and "Error
// Correction in Trained TTT Layers", abstract (TTT-MLP under the LayerNorm
// squared-error objective); per-token steps, 1/d learning-rate scaling and
// the gated output of the updated model: "Edifice.Recurrent.TTT", "Equations
// (TTT-Linear)"; chunk-start gradients: "PonderTTT", "Technical
// Architecture" (dual form).
//
// In the dual form every token of a chunk takes its gradient at the
// chunk-start weights P1, P2, so with K, Q the chunk's keys and queries as
// columns (d x 16) and E = diag(eta) the whole chunk is dense algebra:
//   H = P1 K, A = silu(H), Z = P2 A, Delta = dL/dZ column by column
//   (LayerNorm per token), DH = (P2^T Delta) * silu'(H)
//   W1 = P1 - DH E K^T,  W2 = P2 - Delta E A^T
//   HQ_t = P1 q_t - sum_{s<=t} eta_s dh_s (k_s.q_t)     (= W1_t q_t)
//   Y_t  = W2 aq_t + sum_{s>t} eta_s delta_s (a_s.aq_t) (= W2_t aq_t), aq = silu(HQ)
//   o_t  = Y_t * sigmoid(gate_t)
// (the last line takes the chunk-end W2 and adds back the updates of the
// chunk's later tokens, so the output product runs after the update).
//
// One workgroup owns one (batch, head) scan; block w covers hidden units
// 16w..16w+15 and outputs 16w..16w+15.  The weights stay fp32 in MFMA
// accumulator tiles: in the 16x16 accumulator layout lane l holds
// X[4(l/16) + r][l % 16], r = 0..3, which is also the B operand of X and the
// A operand of X^T for a 16-deep product whose contraction runs over X's row
// index (and two such tiles side by side feed a 32-deep product).  W1 is held
// as W1^T tiles (rows: inputs, contracted by P1 k and P1 q), and W2 twice: as
// W2^T tiles (rows: hidden units, contracted by P2 a) and as W2 tiles (rows:
// outputs, contracted by P2^T delta).  Both copies of W2 take the same update.
// Activations are formed with the tokens as rows (H^T = K^T P1^T, DA^T =
// Delta^T P2), the orientation the rank-16 updates contract over; what other
// waves need crosses LDS, written once and read in the layout each product
// wants.
//
// Precision: every product runs on the bf16 16x16x32 MFMA with fp32
// accumulation; fp32 operands (weights, activations, errors, Gram entries)
// are split into bf16 hi + lo parts (x - hi - lo ~2^-17 relative); the
// 32-deep products drop the lo*lo term (~2^-17 relative), the 16-deep ones
// keep it; the bf16 inputs are exact.  The LayerNorm, SiLU and gating run in
// fp32 on the vector ALUs.
//
// Eight waves, two per SIMD: on SIMD w a hidden-side wave holds W1^T and W2
// for hidden block w and runs the chain of a chunk, and an output-side wave
// holds W2^T for output block w, forms z and the outputs, and stages the
// inputs.  Per chunk c, three barriers:
//   X_c  a_c and aq_{c-1} in LDS: output-side Z_c; hidden-side the W2 update
//        of chunk c-1 (off the chain) and (P1 Q)^T, G1 of chunk c
//   Z_c  Z_c in LDS: hidden-side the LayerNorm of four tokens each, Delta out;
//        output-side the in-chunk output term of chunk c-1
//   D_c  Delta_c in LDS: hidden-side DA^T, DH, the W1 update, the next chunk's
//        a, HQ_c and aq_c; output-side the outputs of chunk c-1 (W2 before
//        this chunk's update), the W2^T update, the staging two chunks ahead
#include "scan_common.h"

namespace ttt {
namespace {

constexpr int D = 64;
constexpr int BT = 16;       // tokens per chunk
constexpr int NT = 512;      // eight waves, two per SIMD
constexpr int RING = 3;      // staged input chunks in LDS
constexpr int APAD = 72;     // padded bf16 row of the [token][unit] activation tiles

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float fast_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

__device__ __forceinline__ unsigned short bf16_bits(float x) {
  return __builtin_bit_cast(unsigned short, static_cast<__bf16>(x));
}
__device__ __forceinline__ float bf16_val(unsigned short b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two fp32 values to two bf16 (round to nearest even each) in one register:
// one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

// x = hi + lo, both bf16 (round to nearest even each), two elements per
// conversion; the residual x - hi is exact in fp32
__device__ __forceinline__ void split4(const f32x4& x, i16x4& hi, i16x4& lo) {
  const uint32_t h01 = pack_bf16(x[0], x[1]);
  const uint32_t h23 = pack_bf16(x[2], x[3]);
  const uint32_t l01 = pack_bf16(x[0] - __uint_as_float(h01 << 16),
                                 x[1] - __uint_as_float(h01 & 0xFFFF0000u));
  const uint32_t l23 = pack_bf16(x[2] - __uint_as_float(h23 << 16),
                                 x[3] - __uint_as_float(h23 & 0xFFFF0000u));
  hi = __builtin_bit_cast(i16x4, make_uint2(h01, h23));
  lo = __builtin_bit_cast(i16x4, make_uint2(l01, l23));
}

__device__ __forceinline__ bf16x8 cat8(const i16x4& a, const i16x4& b) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Every product is the 16x16x32 MFMA.  The 16x16x16 form is not used: built
// for gfx950, a weight tile kept outside the accumulator registers was copied
// into the accumulator input of an in-flight 16x16x16 product three to six
// wait states after its issue, and that product read the copy (wrong updates
// of the W2 tiles, deterministic for one build, gone in another); the
// 16x16x32 form's accumulator input is never overwritten that way here.
__device__ __forceinline__ f32x4 mfma32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// An fp32 operand of a 32-deep contraction as bf16 hi and lo parts (slots
// 0-3 from the first 16-block of the contraction, 4-7 from the second).
struct Op32 {
  bf16x8 hi, lo;
};
// An fp32 operand of a 16-deep contraction.
struct Op16 {
  i16x4 hi, lo;
};

__device__ __forceinline__ Op32 op32(const f32x4& x0, const f32x4& x1) {
  i16x4 h0, l0, h1, l1;
  split4(x0, h0, l0);
  split4(x1, h1, l1);
  return Op32{cat8(h0, h1), cat8(l0, l1)};
}
__device__ __forceinline__ Op16 op16(const f32x4& x) {
  Op16 o;
  split4(x, o.hi, o.lo);
  return o;
}

// c + a b over a 32-deep contraction of two fp32 operands (lo*lo dropped)
__device__ __forceinline__ f32x4 prod3(const Op32& a, const Op32& b, f32x4 c) {
  c = mfma32(a.hi, b.hi, c);
  c = mfma32(a.hi, b.lo, c);
  return mfma32(a.lo, b.hi, c);
}
// c + a b over a 16-deep contraction of two fp32 operands: two 32-deep
// products that share the A operand (a.hi, a.lo), against (b.hi, b.hi) and
// (b.lo, b.lo), so all four terms hi*hi, lo*hi, hi*lo and lo*lo are summed
// (no zero padding to build, and the split operands are multiplied exactly)
__device__ __forceinline__ f32x4 prod3_16(const Op16& a, const Op16& b, f32x4 c) {
  const bf16x8 ah = cat8(a.hi, a.lo);
  c = mfma32(ah, cat8(b.hi, b.hi), c);
  return mfma32(ah, cat8(b.lo, b.lo), c);
}

__device__ __forceinline__ i16x4 ld4(const uint16_t* p) {
  return __builtin_bit_cast(i16x4, *reinterpret_cast<const uint2*>(p));
}
__device__ __forceinline__ void st4(uint16_t* p, const i16x4& v) {
  *reinterpret_cast<uint2*>(p) = __builtin_bit_cast(uint2, v);
}

// ---------------------------------------------------------------------------
// LDS
// ---------------------------------------------------------------------------
// One staged chunk.  KA / QA: keys / queries in the operand layout of the
// 16x16x32 product (lane l = t + 16G holds, in slot e, feature
// j = 32ks + 16(e/4) + 4G + e%4 of token t); KT: -K^T in the A layout of the
// 16x16x16 product (lane l = j%16 + 16G of feature tile jb holds tokens
// 4G + e of feature j); V and SG (the gate logits) by [token][feature].
struct alignas(16) Chunk {
  uint16_t KA[2][64][8];
  uint16_t QA[2][64][8];
  uint16_t KT[4][64][4];
  float V[BT][D];
  float SG[BT][D];        // gate logits (the sigmoid is taken at the output)
  float ETA[BT];          // sigmoid(eta_logit)/d, 0 past the end
  float pad_[4];
};

struct alignas(16) Smem {
  Chunk ring[RING];
  // activations a (and aq) by [token][unit] (hi, lo) and a by [unit][token]
  uint16_t A1[2][2][BT][APAD];   // [chunk parity][hi/lo]
  uint16_t A2[2][2][D][BT];      // [chunk parity][hi/lo]
  uint16_t AQ[2][2][BT][APAD];   // [chunk parity][hi/lo]
  float Z[BT][D];                // z by [token][output]
  uint16_t DS[2][BT][APAD];      // delta by [token][output] (hi, lo)
  uint16_t DT[2][2][D][BT];      // -eta delta by [output][token] ([chunk parity][hi/lo])
};

// ---------------------------------------------------------------------------
// input staging: every thread loads two 16-byte vectors of one array
// ---------------------------------------------------------------------------
struct Stage {
  uint4 v[2];       // 8 bf16 each
  uint32_t eta;     // raw bf16 bits (threads 0..15)
};

// thread tid: array a = tid / 64 (q, k, v, gate), vectors (tid % 64) and
// (tid % 64) + 64 of that array's 128 vectors in the chunk.  `src` is this
// wave's array, chosen among the kernel's pointer arguments by a select, so
// the loads stay global loads (an indexed array of pointers would make them
// flat loads, which every LDS wait then waits for as well).
__device__ __forceinline__ void load_chunk(Stage& st, const uint16_t* src, const uint16_t* eta,
                                           int64_t t0, int64_t T, int tid) {
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int vid = (tid & 63) + 64 * r;
    const int t = vid >> 3;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (t0 + t < T) x = *reinterpret_cast<const uint4*>(src + (t0 + t) * D + (vid & 7) * 8);
    st.v[r] = x;
  }
  st.eta = 0u;
  if (tid < BT && t0 + tid < T) st.eta = eta[t0 + tid];
}

__device__ __forceinline__ void store_chunk(const Stage& st, Chunk& ck, int64_t t0, int64_t T,
                                            int tid) {
  const int a = tid >> 6;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int vid = (tid & 63) + 64 * r;
    const int t = vid >> 3;
    const int j0 = (vid & 7) * 8;
    const uint4 x = st.v[r];
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    if (a <= 1) {
      uint16_t(*dst)[64][8] = (a == 0) ? ck.QA : ck.KA;
      const int ks = j0 / 32, hh = (j0 % 32) / 16, g = (j0 % 16) / 4;
      *reinterpret_cast<uint2*>(&dst[ks][t + 16 * g][4 * hh]) = make_uint2(w[0], w[1]);
      *reinterpret_cast<uint2*>(&dst[ks][t + 16 * (g + 1)][4 * hh]) = make_uint2(w[2], w[3]);
      if (a == 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = j0 + e;
          const uint16_t bits = (e & 1) ? static_cast<uint16_t>(w[e / 2] >> 16)
                                        : static_cast<uint16_t>(w[e / 2] & 0xFFFFu);
          ck.KT[j / 16][(j % 16) + 16 * (t / 4)][t % 4] = bits ^ 0x8000u;   // -k
        }
      }
    } else {
      float f[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
      float* dst = (a == 2) ? &ck.V[t][j0] : &ck.SG[t][j0];
      *reinterpret_cast<float4*>(dst) = make_float4(f[0], f[1], f[2], f[3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(f[4], f[5], f[6], f[7]);
    }
  }
  if (tid < BT) {
    const float x = __uint_as_float(st.eta << 16);
    ck.ETA[tid] = (t0 + tid < T) ? fast_sigmoid(x) * (1.0f / D) : 0.0f;
  }
}

// a 16x32 slice of a [token][unit] activation tile as the 32-deep operand
// with the tokens on the lanes (slot e of lane t + 16g: unit
// 32ks + 16(e/4) + 4g + e%4)
__device__ __forceinline__ Op32 act_op(const uint16_t (*hl)[BT][APAD], int ks, int n, int g) {
  Op32 o;
  o.hi = cat8(ld4(&hl[0][n][32 * ks + 4 * g]), ld4(&hl[0][n][32 * ks + 16 + 4 * g]));
  o.lo = cat8(ld4(&hl[1][n][32 * ks + 4 * g]), ld4(&hl[1][n][32 * ks + 16 + 4 * g]));
  return o;
}

// 16-byte rows of the A operand from a [unit][token] tile (lane m = unit
// 16b + n, slots: tokens 4g..4g+3)
__device__ __forceinline__ Op16 col_op(const uint16_t (*hl)[D][BT], int b, int n, int g) {
  return Op16{ld4(&hl[0][16 * b + n][4 * g]), ld4(&hl[1][16 * b + n][4 * g])};
}

template <int LN>
__global__ void __launch_bounds__(NT)
mlp_mfma_kernel(const uint16_t* __restrict__ qp, const uint16_t* __restrict__ kp,
                const uint16_t* __restrict__ vp, const uint16_t* __restrict__ etap,
                const uint16_t* __restrict__ gatep, const float* __restrict__ W1_0,
                const float* __restrict__ W2_0, const float* __restrict__ gamma,
                const float* __restrict__ beta, float* __restrict__ out,
                float* __restrict__ W1_final, float* __restrict__ W2_final, int H, int64_t T,
                float eps) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int w = wv & 3;            // the block of hidden units and of outputs
  const bool hid = wv < 4;         // hidden-side wave (else output-side), both on SIMD w
  const int n = lane & 15;
  const int g = lane >> 4;
  const int64_t bh = blockIdx.x;
  const int h = static_cast<int>(bh % H);
  const int64_t nc = (T + BT - 1) / BT;

  // output-side waves stage the inputs: wave 4 + a stages array a (q, k, v, gate)
  const int stid = tid - 4 * 64;
  const uint16_t* src = (w == 0 ? qp : w == 1 ? kp : w == 2 ? vp : gatep) + bh * T * D;
  const uint16_t* eta = etap + bh * T;
  float* dst_out = out + bh * T * D;
  const float* w1 = W1_0 + bh * D * D;
  const float* w2 = W2_0 + bh * D * D;

  // ---- weights in accumulator tiles
  // hidden-side:  p1t[jb][r] = W1[16w + n][16jb + 4g + r]  (W1^T: rows inputs, own hidden cols)
  //               p2n[ib][r] = W2[16ib + 4g + r][16w + n]  (W2: rows outputs, own hidden cols)
  // output-side:  p2t[ub][r] = W2[16w + n][16ub + 4g + r]  (W2^T: rows hidden, own output cols)
  f32x4 p1t[4], p2t[4], p2n[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (hid) {
      const float4 x = *reinterpret_cast<const float4*>(w1 + (16 * w + n) * D + 16 * b + 4 * g);
      p1t[b] = f32x4{x.x, x.y, x.z, x.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) p2n[b][r] = w2[(16 * b + 4 * g + r) * D + 16 * w + n];
      p2t[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    } else {
      const float4 y = *reinterpret_cast<const float4*>(w2 + (16 * w + n) * D + 16 * b + 4 * g);
      p2t[b] = f32x4{y.x, y.y, y.z, y.w};
      p1t[b] = p2n[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }

  // LayerNorm affine of the four features a lane handles in the LayerNorm
  // pass (features 4n..4n+3)
  float gam[4] = {1.0f, 1.0f, 1.0f, 1.0f}, bet[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (LN != kLnNone && hid) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      gam[e] = gamma[h * D + 4 * n + e];
      bet[e] = beta[h * D + 4 * n + e];
    }
  }

  // ---- H^T = K^T P1^T of a chunk (rows tokens, cols own hidden units), and
  // the same with Q; G1^T[s][t] = k_s . q_t
  auto w1_operands = [&](Op32 (&p1)[2]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) p1[ks] = op32(p1t[2 * ks], p1t[2 * ks + 1]);
  };
  // (one accumulation chain: no second zeroed accumulator and no adds)
  auto keys_times_w1 = [&](const uint16_t (*XA)[64][8], const Op32 (&p1)[2]) -> f32x4 {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 x = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(XA[ks][lane]));
      acc = mfma32(x, p1[ks].hi, acc);
      acc = mfma32(x, p1[ks].lo, acc);
    }
    return acc;
  };
  auto gram_kq = [&](const Chunk& ck) -> f32x4 {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ck.KA[ks][lane]));
      const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ck.QA[ks][lane]));
      acc = mfma32(a, b, acc);
    }
    return acc;
  };
  // a = silu(h) of this wave's hidden units, to LDS in both layouts; s' = silu'(h)
  auto activate_and_share = [&](const f32x4& ht, f32x4& spt, int par) {
    f32x4 at;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x = ht[r];
      const float sg = fast_sigmoid(x);
      at[r] = x * sg;
      spt[r] = sg * fmaf(x, 1.0f - sg, 1.0f);
    }
    Op16 o = op16(at);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sm.A1[par][0][4 * g + r][16 * w + n] = static_cast<uint16_t>(o.hi[r]);
      sm.A1[par][1][4 * g + r][16 * w + n] = static_cast<uint16_t>(o.lo[r]);
    }
    st4(&sm.A2[par][0][16 * w + n][4 * g], o.hi);
    st4(&sm.A2[par][1][16 * w + n][4 * g], o.lo);
  };
  // A operand of W2 for the own outputs (contraction over hidden units)
  auto w2_operands = [&](Op32 (&p2)[2]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) p2[ks] = op32(p2t[2 * ks], p2t[2 * ks + 1]);
  };

  // ---- the outputs of chunk cp (rows own outputs, cols tokens), from W2 after
  // chunk cp's update: Y = W2 aq + sum_{s>t} eta_s delta_s (a_s . aq_t), gated.
  // The in-chunk term and the W2 product run in different stages.
  auto outputs_inchunk = [&](int64_t cp) -> f32x4 {
    const int par = static_cast<int>(cp & 1);
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    // G2[s][t] = a_s . aq_t
    f32x4 g2 = prod3(act_op(sm.A1[par], 0, n, g), act_op(sm.AQ[par], 0, n, g), zero);
    g2 = prod3(act_op(sm.A1[par], 1, n, g), act_op(sm.AQ[par], 1, n, g), g2);
    // strictly later tokens only, negated (DT holds -eta delta)
#pragma unroll
    for (int r = 0; r < 4; ++r) g2[r] = (4 * g + r > n) ? -g2[r] : 0.0f;
    return prod3_16(col_op(sm.DT[par], w, n, g), op16(g2), zero);
  };
  auto outputs = [&](int64_t cp, const Op32 (&p2)[2], const f32x4& inchunk) {
    const int par = static_cast<int>(cp & 1);
    const Chunk& ck = sm.ring[cp % RING];
    const f32x4 y = prod3(p2[1], act_op(sm.AQ[par], 1, n, g),
                          prod3(p2[0], act_op(sm.AQ[par], 0, n, g), inchunk));
    const int64_t t = cp * BT + n;
    if (t < T) {
      const float4 gl = *reinterpret_cast<const float4*>(&ck.SG[n][16 * w + 4 * g]);
      *reinterpret_cast<float4*>(dst_out + t * D + 16 * w + 4 * g) =
          make_float4(y[0] * fast_sigmoid(gl.x), y[1] * fast_sigmoid(gl.y),
                      y[2] * fast_sigmoid(gl.z), y[3] * fast_sigmoid(gl.w));
    }
  };

  // ---- prologue: chunks 0 and 1 staged, chunk 2 in flight (output-side waves)
  Stage st;
  if (!hid) {
    load_chunk(st, src, eta, 0, T, stid);
    store_chunk(st, sm.ring[0], 0, T, stid);
    if (nc > 1) {
      load_chunk(st, src, eta, BT, T, stid);
      store_chunk(st, sm.ring[1], BT, T, stid);
    }
    if (nc > 2) load_chunk(st, src, eta, 2 * BT, T, stid);
  }
  __syncthreads();

  // hidden-side state of the current chunk: silu'(h)^T, (P1 Q)^T and G1^T;
  // output-side: W2's A operand, split once per update, and the in-chunk
  // output term of the previous chunk
  f32x4 spt = {0.0f, 0.0f, 0.0f, 0.0f}, hq0t = spt, g1t = spt, yin = spt;
  Op32 p2op[2], p1op[2];   // W2's and W1's operands, split once per update
  if (!hid) w2_operands(p2op);
  if (hid) {
    w1_operands(p1op);
    activate_and_share(keys_times_w1(sm.ring[0].KA, p1op), spt, 0);
  }
  __syncthreads();

  for (int64_t c = 0; c < nc; ++c) {
    const int par = static_cast<int>(c & 1);
    const Chunk& ck = sm.ring[c % RING];

    // ---- X_c: a_c in LDS
    if (hid) {
      // W2 (rows outputs, own hidden cols) -= eta Delta A^T of the previous chunk
      if (c > 0) {
        const int pp = par ^ 1;
        const Op16 oa = col_op(sm.A2[pp], w, n, g);   // a_{t}[own hidden], by token rows
#pragma unroll
        for (int b = 0; b < 4; ++b) p2n[b] = prod3_16(col_op(sm.DT[pp], b, n, g), oa, p2n[b]);
      }
      // (P1 Q)^T and G1^T of this chunk, with W1 at its start
      hq0t = keys_times_w1(ck.QA, p1op);
      g1t = gram_kq(ck);
    } else {
      const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
      const f32x4 z = prod3(p2op[1], act_op(sm.A1[par], 1, n, g),
                            prod3(p2op[0], act_op(sm.A1[par], 0, n, g), zero));
      *reinterpret_cast<float4*>(&sm.Z[n][16 * w + 4 * g]) = make_float4(z[0], z[1], z[2], z[3]);
    }
    __syncthreads();

    // ---- Z_c: the LayerNorm (hidden-side waves, tokens 4w..4w+3); the
    // previous chunk's in-chunk output term (output-side waves)
    if (hid) {
      const int t = 4 * w + g;
      const float4 z4 = *reinterpret_cast<const float4*>(&sm.Z[t][4 * n]);
      const float4 v4 = *reinterpret_cast<const float4*>(&ck.V[t][4 * n]);
      const float z[4] = {z4.x, z4.y, z4.z, z4.w};
      const float v[4] = {v4.x, v4.y, v4.z, v4.w};
      // sum over the 16 lanes of a row (quad_perm [1,0,3,2], [2,3,0,1], row_ror 4, 8)
      auto row_sum = [](float x) {
        x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
        x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
        x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xF, 0xF, true));
        x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, true));
        return x;
      };
      float dl[4];
      if constexpr (LN == kLnNone) {
#pragma unroll
        for (int e = 0; e < 4; ++e) dl[e] = z[e] - v[e];
      } else {
        const float mu = row_sum((z[0] + z[1]) + (z[2] + z[3])) * (1.0f / D);
        float m2 = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) m2 = fmaf(z[e] - mu, z[e] - mu, m2);
        const float rs = __builtin_amdgcn_rsqf(row_sum(m2) * (1.0f / D) + eps);
        float xh[4], er[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xh[e] = (z[e] - mu) * rs;
          er[e] = fmaf(gam[e], xh[e], bet[e]) - v[e];
        }
        if constexpr (LN == kLnExact) {
          float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s1 = fmaf(gam[e], er[e], s1);
            s2 = fmaf(gam[e] * er[e], xh[e], s2);
          }
          s1 = row_sum(s1) * (1.0f / D);
          s2 = row_sum(s2) * (1.0f / D);
#pragma unroll
          for (int e = 0; e < 4; ++e) dl[e] = rs * (gam[e] * er[e] - s1 - xh[e] * s2);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) dl[e] = er[e];
        }
      }
      const f32x4 d4 = {dl[0], dl[1], dl[2], dl[3]};
      const float et = ck.ETA[t];
      const f32x4 de = {-et * dl[0], -et * dl[1], -et * dl[2], -et * dl[3]};
      const Op16 od = op16(d4), oe = op16(de);
      st4(&sm.DS[0][t][4 * n], od.hi);
      st4(&sm.DS[1][t][4 * n], od.lo);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sm.DT[par][0][4 * n + e][t] = static_cast<uint16_t>(oe.hi[e]);
        sm.DT[par][1][4 * n + e][t] = static_cast<uint16_t>(oe.lo[e]);
      }
    } else if (c > 0) {
      yin = outputs_inchunk(c - 1);
    }
    __syncthreads();

    // ---- D_c: Delta_c in LDS
    if (hid) {
      // DA^T = Delta^T P2 (rows tokens, own hidden cols), at the chunk-start W2
      const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
      const f32x4 dat = prod3(act_op(sm.DS, 1, n, g), op32(p2n[2], p2n[3]),
                              prod3(act_op(sm.DS, 0, n, g), op32(p2n[0], p2n[1]), zero));
      // eta DH^T
      f32x4 edh;
#pragma unroll
      for (int r = 0; r < 4; ++r) edh[r] = ck.ETA[4 * g + r] * (dat[r] * spt[r]);
      const Op16 oedh = op16(edh);
      // W1^T (rows inputs, own hidden cols) -= K eta DH^T  (KT holds -K^T)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const i16x4 kt = ld4(ck.KT[b][lane]);
        p1t[b] = mfma32(cat8(kt, kt), cat8(oedh.hi, oedh.lo), p1t[b]);
      }
      // the next chunk's a with the updated W1
      w1_operands(p1op);
      if (c + 1 < nc) activate_and_share(keys_times_w1(sm.ring[(c + 1) % RING].KA, p1op), spt, par ^ 1);
      // HQ^T = (P1 Q)^T - G1 (eta DH^T), s <= t; aq = silu(HQ)
      {
        f32x4 gm;
#pragma unroll
        for (int r = 0; r < 4; ++r) gm[r] = (4 * g + r <= n) ? -g1t[r] : 0.0f;
        const f32x4 hqt = prod3_16(op16(gm), oedh, hq0t);
        f32x4 aqt;
#pragma unroll
        for (int r = 0; r < 4; ++r) aqt[r] = hqt[r] * fast_sigmoid(hqt[r]);
        const Op16 o = op16(aqt);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sm.AQ[par][0][4 * g + r][16 * w + n] = static_cast<uint16_t>(o.hi[r]);
          sm.AQ[par][1][4 * g + r][16 * w + n] = static_cast<uint16_t>(o.lo[r]);
        }
      }
    } else {
      // the previous chunk's outputs, from W2 before this chunk's update
      if (c > 0) outputs(c - 1, p2op, yin);
      // W2^T (rows hidden, own output cols) -= A eta Delta^T
      const Op16 od = col_op(sm.DT[par], w, n, g);
#pragma unroll
      for (int b = 0; b < 4; ++b) p2t[b] = prod3_16(col_op(sm.A2[par], b, n, g), od, p2t[b]);
      w2_operands(p2op);
      // stage chunk c + 2, load chunk c + 3
      if (c + 2 < nc) {
        store_chunk(st, sm.ring[(c + 2) % RING], (c + 2) * BT, T, stid);
        if (c + 3 < nc) load_chunk(st, src, eta, (c + 3) * BT, T, stid);
      }
    }
    __syncthreads();
  }

  // ---- the last chunk's outputs, the final weights
  if (!hid && nc > 0) outputs(nc - 1, p2op, outputs_inchunk(nc - 1));
  if (hid && W1_final != nullptr) {
    float* o = W1_final + bh * D * D;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      *reinterpret_cast<float4*>(o + (16 * w + n) * D + 16 * b + 4 * g) =
          make_float4(p1t[b][0], p1t[b][1], p1t[b][2], p1t[b][3]);
  }
  if (!hid && W2_final != nullptr) {
    float* o = W2_final + bh * D * D;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      *reinterpret_cast<float4*>(o + (16 * w + n) * D + 16 * b + 4 * g) =
          make_float4(p2t[b][0], p2t[b][1], p2t[b][2], p2t[b][3]);
  }
}

template <int LN>
hipError_t launch_ln(const ScanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((mlp_mfma_kernel<LN>), dim3(static_cast<unsigned>(a.B * a.H)), dim3(NT), 0,
                     s, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.eta_logit),
                     static_cast<const uint16_t*>(a.gate_logit), a.W0, a.W2_0, a.gamma, a.beta,
                     a.out, a.W_final, a.W2_final, static_cast<int>(a.H), a.T, a.eps);
  return hipGetLastError();
}

}  // namespace

bool mlp_mfma_supports(const ScanArgs& a) {
  return a.d == D && a.dual && a.chunk == BT && a.in_bf16 && !a.silu_qk &&
         a.upd_mask == nullptr;
}

hipError_t launch_mlp_mfma(const ScanArgs& a, hipStream_t s) {
  if (!mlp_mfma_supports(a)) return hipErrorNotSupported;
  switch (a.ln) {
    case kLnST: return launch_ln<kLnST>(a, s);
    case kLnExact: return launch_ln<kLnExact>(a, s);
    default: return launch_ln<kLnNone>(a, s);
  }
}

}  // namespace ttt
