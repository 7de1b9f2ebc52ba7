// Backward of the TTT-Linear scan on the vector ALUs (gfx950): every d the
// vector-ALU forward runs (16, 32, 64, 128), the per-token modes and the dual
// form with any chunk length.
//
// Recurrence: "Edifice.Recurrent.TTT", "Equations (TTT-Linear)"; exact
// LayerNorm gradient: "Error Correction in Trained TTT Layers", abstract;
// chunk-start gradients: "PonderTTT", "Technical Architecture" (dual-form
// updates).  The gradients are those of a loss L through out and W_final,
// reverse-mode through every step of the forward:
//
//   y_t = W_t q_t, o_t = y_t sigmoid(g_t)    ->  dy_t = dout_t sigmoid(g_t)
//   W_t = W_{t-1} - a_t delta_t k_t^T,  a_t = sigmoid(eta_t) / d
//   delta_t = the inner gradient at z_t = P k_t  (P = W_{t-1}, or the dual
//             form's chunk-start W)
//
// With G the gradient with respect to the running W (dW_final after the last
// token), token t adds dy_t q_t^T to G; then d delta_t = -a_t G k_t,
// d a_t = -delta_t . G k_t, dk_t = -a_t G^T delta_t + P^T dz_t and
// dq_t = W_t^T dy_t, dz_t being the vector-Jacobian product of the inner
// gradient; dz_t k_t^T joins G at once (per token) or when the walk reaches
// the chunk's first token (dual form).
//
// A recording forward leaves delta_t of every token and the running W before
// every 16th token.  The walk takes those 16-token tiles last to first: W is
// replayed from the tile's recorded W to the tile's end with the forward's own
// operations, then taken back one token at a time (W_{t-1} = W_t + a_t
// delta_t k_t^T).  The dual form's chunk-start W is replayed from the recorded
// W at or before the chunk's start (at most 15 tokens).
//
// Layout as in the vector-ALU forward: one workgroup per (b,h); row i of W, G
// (and of the dual form's chunk-start W and its pending gradient) lives in the
// four lanes of a DPP quad, each holding d/4 columns.  Row sums (W q, G k,
// P k) are quad reductions; sums over the d rows (the LayerNorm's statistics
// and its vector-Jacobian product) cross the waves through LDS; column sums
// (W^T dy, G^T delta, P^T dz) are reduced within a wave by a butterfly that
// halves the columns a lane carries at each of four shuffle steps, then
// across the waves through LDS once per group of tokens.
#include "bwd_valu.h"

#include <type_traits>

namespace ttt {
namespace {

constexpr int kTok = static_cast<int>(kRecTile);   // tokens per tile of the walk

__device__ __forceinline__ float sigmoid_(float x) {
  // exp(-x) saturates to +inf for x = -inf (result 0) and to 0 for +inf (result 1)
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// DPP controls: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_shl:4, row_shr:4,
// row_ror:4, row_ror:8 (row = 16 lanes; row_shl:n reads lane + n, row_shr:n
// lane - n, row_ror:8 pairs each lane with lane ^ 8)
constexpr int kQuadXor1 = 0xB1;
constexpr int kQuadXor2 = 0x4E;
constexpr int kRowShl4 = 0x104;
constexpr int kRowShr4 = 0x114;
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

__device__ __forceinline__ float quad_sum(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  return x;
}

// v_permlane32_swap / v_permlane16_swap (vector ALU, no LDS round trip): for
// registers a, b the pair (a', b') with a' + b' = a of this lane plus a of
// lane ^ 32 (resp. ^ 16) where that bit of the lane is clear, and b of this
// lane plus b of lane ^ 32 (^ 16) where it is set.
__device__ __forceinline__ float swap32_sum(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap16_sum(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over the 16 quads of a wave of a value that is uniform within each quad.
__device__ __forceinline__ float quads_sum(float x) {
  x += dpp<kRowRor4>(x);
  x += dpp<kRowRor8>(x);
  x = swap16_sum(x, x);
  return swap32_sum(x, x);
}

// One step of the column butterfly over the wave's 16 quads (quad bit
// 3 - STAGE, lane distance M = 32 >> STAGE).  While a lane carries more than
// one column it keeps half (the upper half where its bit is set) and adds the
// partner's partial sums of that half; with one column left it adds the
// partner's.  Lane distances 32 and 16 exchange through the lane swaps, 8 and
// 4 through DPP within the row.
template <int N, int STAGE>
__device__ __forceinline__ void col_step(float (&v)[N], int lane, int& off) {
  constexpr int M = 32 >> STAGE;
  constexpr int HAVE = (N >> STAGE) > 0 ? (N >> STAGE) : 1;
  constexpr int HALF = HAVE > 1 ? HAVE / 2 : 1;
  const bool hi = (lane & M) != 0;
#pragma unroll
  for (int i = 0; i < HALF; ++i) {
    const float a = v[i];
    const float b = HAVE > 1 ? v[i + HALF] : v[i];
    if constexpr (M == 32) {
      v[i] = swap32_sum(a, b);
    } else if constexpr (M == 16) {
      v[i] = swap16_sum(a, b);
    } else {
      // keep = the half this lane sums, send = the half its partner sums; the
      // DPP moves run on every lane (a DPP read of a lane masked off by a
      // branch would return zero), the choices are selects
      const float keep = hi ? b : a;
      const float send = hi ? a : b;
      if constexpr (M == 8) {
        v[i] = keep + dpp<kRowRor8>(send);
      } else {
        const float from_above = dpp<kRowShl4>(send);   // lane + 4
        const float from_below = dpp<kRowShr4>(send);   // lane - 4
        v[i] = keep + (hi ? from_below : from_above);
      }
    }
  }
  if (HAVE > 1 && hi) off += HALF;
}

template <bool BF16>
__device__ __forceinline__ float4 load4(const void* p, int64_t e) {
  if constexpr (BF16) {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + e);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
  } else {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + e);
  }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* p, int64_t e) {
  if constexpr (BF16)
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[e]) << 16);
  else
    return static_cast<const float*>(p)[e];
}

__device__ __forceinline__ float silu_(float x) { return x * sigmoid_(x); }
__device__ __forceinline__ float silu_grad_(float x) {
  const float s = sigmoid_(x);
  return s * fmaf(x, 1.0f - s, 1.0f);
}

template <int D, bool BF16, int LN, bool DUAL>
__global__ void __launch_bounds__(4 * D)
bwd_valu_kernel(const void* __restrict__ qp, const void* __restrict__ kp,
                const void* __restrict__ vp, const void* __restrict__ etap,
                const void* __restrict__ gatep, const float* __restrict__ gamma,
                const float* __restrict__ beta, const float* __restrict__ dout,
                const float* __restrict__ dW_final, const float* __restrict__ rec_delta,
                const float* __restrict__ rec_W, float* __restrict__ dq, float* __restrict__ dk,
                float* __restrict__ dv, float* __restrict__ deta, float* __restrict__ dgate,
                float* __restrict__ dW0, float* __restrict__ gb_part, int H, int64_t T,
                int64_t chunk, float eps, int silu) {
  constexpr int NT = 4 * D;                        // threads
  constexpr int NW = NT / 64;                      // waves
  constexpr int C = D / 4;                         // columns per lane
  constexpr int TE = kTok * D;                     // elements per array per tile
  constexpr int PT = D <= 64 ? kTok : kTok / 2;    // tokens per column-sum group
  constexpr int NV = C >= 16 ? C / 16 : 1;         // columns a lane holds after the butterfly
  constexpr float kInvD = 1.0f / D;
  constexpr int kRowsPerWave = 16;
  static_assert(TE == 4 * NT, "one float4 per thread per staged array");

  __shared__ __align__(16) float sK[TE];     // k (after SiLU)
  __shared__ __align__(16) float sQ[TE];     // q (after SiLU)
  __shared__ __align__(16) float sV[TE];     // v, then dv
  __shared__ __align__(16) float sSG[TE];    // sigmoid(gate_logit), then dgate_logit
  __shared__ __align__(16) float sDO[TE];    // dout
  __shared__ __align__(16) float sDel[TE];   // recorded delta
  __shared__ __align__(16) float sKd[TE];    // silu'(k)
  __shared__ __align__(16) float sQd[TE];    // silu'(q)
  __shared__ __align__(16) float sCol[2][NW][PT][D];   // per-wave column sums of dq, dk
  __shared__ float sA[kTok];                 // a_t = sigmoid(eta_logit) / d
  __shared__ float sAd[kTok];                // d a_t / d eta_logit
  __shared__ float sDeta[kTok];
  __shared__ float4 sRed[4][2][NW];          // [reduction][token parity][wave]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row = tid >> 2;
  const int seg = tid & 3;
  const int64_t bh = blockIdx.x;
  const int h = static_cast<int>(bh % H);
  const int64_t seq0 = bh * T;                         // this scan's first token
  const int64_t ntiles = (T + kTok - 1) / kTok;        // recorded W per scan
  const float* recW = rec_W + bh * ntiles * D * D;

  // G: the gradient with respect to the running W; Wc, Zc: the dual form's
  // chunk-start W and the gradient pending for it (unused per token)
  float G[C], W[C], Wc[C], Zc[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    G[c] = 0.0f;
    Wc[c] = 0.0f;
    Zc[c] = 0.0f;
  }
  float gam = 1.0f, bet = 0.0f;
  if constexpr (LN != kLnNone) {
    gam = gamma[h * D + row];
    bet = beta[h * D + row];
  }
  float dgam = 0.0f, dbet = 0.0f;
  int par = 0;

  auto load_row = [&](const float* src, float (&dst)[C]) {
    const float4* s4 = reinterpret_cast<const float4*>(src + row * D + seg * C);
#pragma unroll
    for (int c = 0; c < C / 4; ++c) {
      const float4 x = s4[c];
      dst[4 * c] = x.x; dst[4 * c + 1] = x.y; dst[4 * c + 2] = x.z; dst[4 * c + 3] = x.w;
    }
  };
  if (dW_final != nullptr) load_row(dW_final + bh * D * D, G);
  auto lds_cols = [&](const float* src, float (&dst)[C]) {
    const float4* s4 = reinterpret_cast<const float4*>(src + seg * C);
#pragma unroll
    for (int c = 0; c < C / 4; ++c) {
      const float4 x = s4[c];
      dst[4 * c] = x.x; dst[4 * c + 1] = x.y; dst[4 * c + 2] = x.z; dst[4 * c + 3] = x.w;
    }
  };

  // Sums over the d rows of the first n of four per-row values (uniform
  // within each quad); every thread gets them.
  auto rows_sum = [&](float4 x, int slot, int n) -> float4 {
    x.x = quads_sum(x.x);
    if (n > 1) x.y = quads_sum(x.y);
    if (n > 2) x.z = quads_sum(x.z);
    if (n > 3) x.w = quads_sum(x.w);
    if constexpr (NW == 1) {
      return x;
    } else {
      if (lane == 0) sRed[slot][par][wave] = x;
      __syncthreads();
      float4 r = sRed[slot][par][0];
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        const float4 y = sRed[slot][par][w];
        r.x += y.x;
        r.y += y.y;
        r.z += y.z;
        r.w += y.w;
      }
      return r;
    }
  };
  // Mean and biased variance of z over the d rows, as the forward forms them:
  // each wave shifts its rows by one of its own entries, the waves' means and
  // squared deviations then combine exactly.
  auto ln_stats = [&](float z) -> float2 {
    const float c = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(z)));
    const float y = z - c;
    const float a = quads_sum(y);
    const float b = quads_sum(y * y);
    const float mw = fmaf(a, 1.0f / kRowsPerWave, c);
    const float m2w = fmaxf(fmaf(-a, a * (1.0f / kRowsPerWave), b), 0.0f);
    if constexpr (NW == 1) {
      return make_float2(mw, m2w * kInvD);
    } else {
      if (lane == 0) sRed[0][par][wave] = make_float4(mw, m2w, 0.0f, 0.0f);
      __syncthreads();
      float mu = 0.0f, m2 = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float4 x = sRed[0][par][w];
        mu += x.x;
        m2 += x.y;
      }
      mu *= 1.0f / NW;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float dm = sRed[0][par][w].x - mu;
        m2 = fmaf(kRowsPerWave * dm, dm, m2);
      }
      return make_float2(mu, m2 * kInvD);
    }
  };
  // The straight-through mode's one exchange per token: the LayerNorm
  // statistics of z and the two sums its vector-Jacobian product needs,
  // sum gamma dd and sum gamma dd (z - mu), together with sum delta (G k) for
  // d eta.  Each wave sums over its rows with z shifted by one of its own
  // entries c; the parts combine exactly (the shifts enter only through
  // c - mu, a few standard deviations at most).  Returns mu, var and the three
  // sums in *st.
  auto st_round = [&](float z, float gdd, float dgk, float4* st) {
    const float c = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(z)));
    const float y = z - c;
    const float sy = quads_sum(y);
    const float syy = quads_sum(y * y);
    const float sa = quads_sum(gdd);
    const float sb = quads_sum(gdd * y);
    const float sd = quads_sum(dgk);
    const float mw = fmaf(sy, 1.0f / kRowsPerWave, c);
    const float m2w = fmaxf(fmaf(-sy, sy * (1.0f / kRowsPerWave), syy), 0.0f);
    if constexpr (NW == 1) {
      st[0] = make_float4(mw, m2w * kInvD, sa, fmaf(c - mw, sa, sb));
      st[1].x = sd;
    } else {
      if (lane == 0) {
        sRed[0][par][wave] = make_float4(mw, m2w, sa, sb);
        sRed[1][par][wave] = make_float4(c, sd, 0.0f, 0.0f);
      }
      __syncthreads();
      float mu = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) mu += sRed[0][par][w].x;
      mu *= 1.0f / NW;
      float m2 = 0.0f, ta = 0.0f, tb = 0.0f, td = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float4 x = sRed[0][par][w];
        const float4 u = sRed[1][par][w];
        const float dm = x.x - mu;
        m2 += fmaf(kRowsPerWave * dm, dm, x.y);
        ta += x.z;
        tb += fmaf(u.x - mu, x.z, x.w);
        td += u.y;
      }
      st[0] = make_float4(mu, m2 * kInvD, ta, tb);
      st[1].x = td;
    }
  };
  // The wave's column sums of part (this thread's row, its C columns) into
  // sCol[which][wave][slot]; the lanes of a quad group that share a column
  // after the butterfly write it once.
  auto store_cols = [&](float (&part)[C], int which, int slot) {
    int off = 0;
    col_step<C, 0>(part, lane, off);
    col_step<C, 1>(part, lane, off);
    col_step<C, 2>(part, lane, off);
    col_step<C, 3>(part, lane, off);
    if (C >= 16 || ((lane >> 2) & (16 / C - 1)) == 0) {
#pragma unroll
      for (int j = 0; j < NV; ++j) sCol[which][wave][slot][seg * C + off + j] = part[j];
    }
  };
  // dq, dk of tokens [lo, hi) of the tile starting at token t0: the waves'
  // column sums, times silu' with SiLU on q and k
  auto flush_cols = [&](int lo, int hi, int64_t t0) {
    __syncthreads();
    const int e = tid * 4;
    const int tk = lo + e / D;
    const int col = e % D;
    if (e < (hi - lo) * D) {
      const int slot = tk % PT;
      float4 sq = make_float4(0.0f, 0.0f, 0.0f, 0.0f), sk = sq;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float4 x = *reinterpret_cast<const float4*>(&sCol[0][w][slot][col]);
        const float4 y = *reinterpret_cast<const float4*>(&sCol[1][w][slot][col]);
        sq.x += x.x; sq.y += x.y; sq.z += x.z; sq.w += x.w;
        sk.x += y.x; sk.y += y.y; sk.z += y.z; sk.w += y.w;
      }
      if (silu) {
        const float4 fq = *reinterpret_cast<const float4*>(sQd + tk * D + col);
        const float4 fk = *reinterpret_cast<const float4*>(sKd + tk * D + col);
        sq.x *= fq.x; sq.y *= fq.y; sq.z *= fq.z; sq.w *= fq.w;
        sk.x *= fk.x; sk.y *= fk.y; sk.z *= fk.z; sk.w *= fk.w;
      }
      const int64_t o = (seq0 + t0 + tk) * D + col;
      *reinterpret_cast<float4*>(dq + o) = sq;
      *reinterpret_cast<float4*>(dk + o) = sk;
    }
    __syncthreads();
  };
  // tile j's inputs into LDS: one float4 of each array per thread
  auto stage = [&](int64_t j, int nt) {
    const int e = tid * 4;
    const int64_t g = (seq0 + j * kTok) * D + e;
    if (e / D < nt) {
      float4 kx = load4<BF16>(kp, g), qx = load4<BF16>(qp, g);
      if (silu) {
        *reinterpret_cast<float4*>(sKd + e) = make_float4(
            silu_grad_(kx.x), silu_grad_(kx.y), silu_grad_(kx.z), silu_grad_(kx.w));
        *reinterpret_cast<float4*>(sQd + e) = make_float4(
            silu_grad_(qx.x), silu_grad_(qx.y), silu_grad_(qx.z), silu_grad_(qx.w));
        kx = make_float4(silu_(kx.x), silu_(kx.y), silu_(kx.z), silu_(kx.w));
        qx = make_float4(silu_(qx.x), silu_(qx.y), silu_(qx.z), silu_(qx.w));
      }
      *reinterpret_cast<float4*>(sK + e) = kx;
      *reinterpret_cast<float4*>(sQ + e) = qx;
      *reinterpret_cast<float4*>(sV + e) = load4<BF16>(vp, g);
      const float4 gx = load4<BF16>(gatep, g);
      *reinterpret_cast<float4*>(sSG + e) =
          make_float4(sigmoid_(gx.x), sigmoid_(gx.y), sigmoid_(gx.z), sigmoid_(gx.w));
      *reinterpret_cast<float4*>(sDO + e) = *reinterpret_cast<const float4*>(dout + g);
      *reinterpret_cast<float4*>(sDel + e) = *reinterpret_cast<const float4*>(rec_delta + g);
    }
    if (tid < nt) {
      const float s = sigmoid_(load1<BF16>(etap, seq0 + j * kTok + tid));
      sA[tid] = s * kInvD;
      sAd[tid] = s * (1.0f - s) * kInvD;
    }
  };
  // The dual form's chunk-start W (the running W before token c0): the
  // recorded W at or before c0, replayed over the tokens between them.
  // t0: first token of the staged tile.
  auto chunk_start = [&](int64_t c0, int64_t t0) {
    const int64_t m = c0 / kTok;
    load_row(recW + m * D * D, Wc);
    if (m * kTok == t0) {
      for (int s = 0; s < static_cast<int>(c0 - t0); ++s) {
        const float ci = sA[s] * sDel[s * D + row];
        const float* ks = sK + s * D + seg * C;
#pragma unroll
        for (int c = 0; c < C; ++c) Wc[c] = fmaf(-ci, ks[c], Wc[c]);
      }
    } else {
      for (int64_t s = m * kTok; s < c0; ++s) {
        const float ci = sigmoid_(load1<BF16>(etap, seq0 + s)) * kInvD *
                         rec_delta[(seq0 + s) * D + row];
#pragma unroll
        for (int c = 0; c < C / 4; ++c) {
          float4 x = load4<BF16>(kp, (seq0 + s) * D + seg * C + 4 * c);
          if (silu) x = make_float4(silu_(x.x), silu_(x.y), silu_(x.z), silu_(x.w));
          Wc[4 * c] = fmaf(-ci, x.x, Wc[4 * c]);
          Wc[4 * c + 1] = fmaf(-ci, x.y, Wc[4 * c + 1]);
          Wc[4 * c + 2] = fmaf(-ci, x.z, Wc[4 * c + 2]);
          Wc[4 * c + 3] = fmaf(-ci, x.w, Wc[4 * c + 3]);
        }
      }
    }
  };

  int64_t cur_chunk = -1, cur_c0 = 0;
  for (int64_t j = ntiles - 1; j >= 0; --j) {
    const int64_t t0 = j * kTok;
    const int nt = static_cast<int>(T - t0 < kTok ? T - t0 : kTok);
    __syncthreads();   // the previous tile's LDS is no longer read
    stage(j, nt);
    __syncthreads();
    // W at the tile's start, replayed to its end as the forward formed it
    load_row(recW + j * D * D, W);
    for (int tt = 0; tt < nt; ++tt) {
      const float ci = sA[tt] * sDel[tt * D + row];
      const float* kt = sK + tt * D + seg * C;
#pragma unroll
      for (int c = 0; c < C; ++c) W[c] = fmaf(-ci, kt[c], W[c]);
    }
    int grp_hi = nt;   // end of the tokens whose column sums are pending
    for (int tt = nt - 1; tt >= 0; --tt) {
      const int64_t t = t0 + tt;
      if constexpr (DUAL) {
        if (t / chunk != cur_chunk) {
          cur_chunk = t / chunk;
          cur_c0 = cur_chunk * chunk;
          chunk_start(cur_c0, t0);
        }
      }
      const int ri = tt * D + row;
      const float a = sA[tt];
      const float sg = sSG[ri], dout_i = sDO[ri], del = sDel[ri], vi = sV[ri];
      float kv[C], part[C];
      lds_cols(sK + tt * D, kv);
      const float4* q4 = reinterpret_cast<const float4*>(sQ + tt * D + seg * C);
      // the output: y = W_t q, dy = dout sigmoid(g); dq = W_t^T dy; and
      // G = dL/dW_t = (the gradient after t) + dy q^T
      const float u = dout_i * sg;
      float y = 0.0f;
#pragma unroll
      for (int c = 0; c < C / 4; ++c) {
        const float4 x = q4[c];
        y = fmaf(W[4 * c], x.x, y);
        y = fmaf(W[4 * c + 1], x.y, y);
        y = fmaf(W[4 * c + 2], x.z, y);
        y = fmaf(W[4 * c + 3], x.w, y);
        G[4 * c] = fmaf(u, x.x, G[4 * c]);
        G[4 * c + 1] = fmaf(u, x.y, G[4 * c + 1]);
        G[4 * c + 2] = fmaf(u, x.z, G[4 * c + 2]);
        G[4 * c + 3] = fmaf(u, x.w, G[4 * c + 3]);
      }
      y = quad_sum(y);
      const float dgt = dout_i * y * sg * (1.0f - sg);
#pragma unroll
      for (int c = 0; c < C; ++c) part[c] = W[c] * u;
      store_cols(part, 0, tt % PT);
      // the update's gradients
      float gk = 0.0f;
#pragma unroll
      for (int c = 0; c < C; ++c) gk = fmaf(G[c], kv[c], gk);
      gk = quad_sum(gk);
      const float dd = -a * gk;   // d delta_t
      const float cd = a * del;
      // part: -a G^T delta; W_{t-1}; z = P k with P = W_{t-1}, or the chunk-start W
      float z = 0.0f;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        part[c] = -cd * G[c];
        W[c] = fmaf(cd, kv[c], W[c]);
        z = fmaf(DUAL ? Wc[c] : W[c], kv[c], z);
      }
      z = quad_sum(z);
      // vector-Jacobian product of the inner gradient
      float dz, dvi, sdk;   // sdk = sum_i delta_i (G k)_i
      if constexpr (LN == kLnNone) {
        dz = dd;
        dvi = -dd;
        sdk = rows_sum(make_float4(del * gk, 0.0f, 0.0f, 0.0f), 1, 1).x;
      } else {
        if constexpr (LN == kLnST) {
          // sum dxh = sum gamma dd; sum dxh xh = rs sum gamma dd (z - mu)
          const float dxh = gam * dd;
          float4 r[2];
          st_round(z, dxh, del * gk, r);
          const float rs = __builtin_amdgcn_rsqf(r[0].y + eps);
          const float xh = (z - r[0].x) * rs;
          dz = rs * (dxh - r[0].z * kInvD - xh * (rs * r[0].w * kInvD));
          dvi = -dd;
          dgam = fmaf(dd, xh, dgam);
          dbet += dd;
          sdk = r[1].x;
        } else {
          const float2 st = ln_stats(z);
          const float rs = __builtin_amdgcn_rsqf(st.y + eps);
          const float xh = (z - st.x) * rs;
          const float e = fmaf(gam, xh, bet) - vi;
          const float g = gam * e;
          const float4 ra = rows_sum(make_float4(g, g * xh, 0.0f, 0.0f), 1, 2);
          const float m2 = ra.y * kInvD;
          const float p = rs * dd;
          const float4 rb = rows_sum(make_float4(p, p * xh, del * gk, 0.0f), 2, 3);
          const float mp1 = rb.x * kInvD, mp2 = rb.y * kInvD;
          sdk = rb.z;
          const float dg = p - mp1 - xh * mp2;
          const float dxh = gam * gam * dg - p * m2 - g * mp2;
          const float4 rc = rows_sum(make_float4(dxh, dxh * xh, 0.0f, 0.0f), 3, 2);
          const float ddel = -a * sdk;   // d delta . delta
          dz = rs * (dxh - rc.x * kInvD - xh * (rc.y * kInvD)) - ddel * rs * xh * kInvD;
          dvi = -gam * dg;
          dbet = fmaf(gam, dg, dbet);
          dgam = fmaf(dg, e + gam * xh, dgam);
        }
      }
      if (tid == 0) sDeta[tt] = -sdk * sAd[tt];
      // dk = -a G^T delta + P^T dz
#pragma unroll
      for (int c = 0; c < C; ++c) part[c] = fmaf(dz, DUAL ? Wc[c] : W[c], part[c]);
      store_cols(part, 1, tt % PT);
      // dz k^T: the gradient of P
      if constexpr (DUAL) {
#pragma unroll
        for (int c = 0; c < C; ++c) Zc[c] = fmaf(dz, kv[c], Zc[c]);
        if (t == cur_c0) {
#pragma unroll
          for (int c = 0; c < C; ++c) {
            G[c] += Zc[c];
            Zc[c] = 0.0f;
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < C; ++c) G[c] = fmaf(dz, kv[c], G[c]);
      }
      if (seg == 0) {
        sV[ri] = dvi;
        sSG[ri] = dgt;
      }
      par ^= 1;
      if (tt % PT == 0) {
        flush_cols(tt, grp_hi, t0);
        grp_hi = tt;
      }
    }
    // the tile's per-row outputs (the last flush ended with a barrier)
    {
      const int e = tid * 4;
      if (e / D < nt) {
        const int64_t g = (seq0 + t0) * D + e;
        *reinterpret_cast<float4*>(dv + g) = *reinterpret_cast<const float4*>(sV + e);
        *reinterpret_cast<float4*>(dgate + g) = *reinterpret_cast<const float4*>(sSG + e);
      }
      if (tid < nt) deta[seq0 + t0 + tid] = sDeta[tid];
    }
  }

  {
    float4* w4 = reinterpret_cast<float4*>(dW0 + bh * D * D + row * D + seg * C);
#pragma unroll
    for (int c = 0; c < C / 4; ++c)
      w4[c] = make_float4(G[4 * c], G[4 * c + 1], G[4 * c + 2], G[4 * c + 3]);
  }
  if (LN != kLnNone && gb_part != nullptr && seg == 0) {
    gb_part[(bh * 2) * D + row] = dgam;
    gb_part[(bh * 2 + 1) * D + row] = dbet;
  }
}

// dgamma[h][i] = sum over the batch of the per-scan parts, dbeta likewise (fixed order)
__global__ void gb_sum_kernel(const float* __restrict__ gb_part, float* __restrict__ dgamma,
                              float* __restrict__ dbeta, int64_t B, int64_t H, int D) {
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

template <int D, bool BF16, int LN, bool DUAL>
hipError_t launch_one(const BwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((bwd_valu_kernel<D, BF16, LN, DUAL>), dim3(static_cast<unsigned>(a.B * a.H)),
                     dim3(4 * D), 0, s, a.q, a.k, a.v, a.eta_logit, a.gate_logit, a.gamma,
                     a.beta, a.dout, a.dW_final, a.rec_delta, a.rec_W, a.dq, a.dk, a.dv,
                     a.deta_logit, a.dgate_logit, a.dW0,
                     LN == kLnNone ? nullptr : a.gb_part, static_cast<int>(a.H), a.T,
                     a.dual ? a.chunk : int64_t(1), a.eps, a.silu_qk ? 1 : 0);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || LN == kLnNone) return err;
  const int64_t n = a.H * D;
  hipLaunchKernelGGL(gb_sum_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                     s, a.gb_part, a.dgamma, a.dbeta, a.B, a.H, D);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_d(const BwdArgs& a, hipStream_t s) {
  if (a.dual) {
    switch (a.ln) {
      case kLnST: return launch_one<D, BF16, kLnST, true>(a, s);
      case kLnExact: return launch_one<D, BF16, kLnExact, true>(a, s);
      default: return launch_one<D, BF16, kLnNone, true>(a, s);
    }
  }
  switch (a.ln) {
    case kLnST: return launch_one<D, BF16, kLnST, false>(a, s);
    case kLnExact: return launch_one<D, BF16, kLnExact, false>(a, s);
    default: return launch_one<D, BF16, kLnNone, false>(a, s);
  }
}

template <int D>
hipError_t launch_dt(const BwdArgs& a, hipStream_t s) {
  return a.in_bf16 ? launch_d<D, true>(a, s) : launch_d<D, false>(a, s);
}

}  // namespace

hipError_t launch_bwd_valu(const BwdArgs& a, hipStream_t s) {
  switch (a.d) {
    case 16: return launch_dt<16>(a, s);
    case 32: return launch_dt<32>(a, s);
    case 64: return launch_dt<64>(a, s);
    case 128: return launch_dt<128>(a, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace ttt
