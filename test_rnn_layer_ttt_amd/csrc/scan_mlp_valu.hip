// TTT-MLP scan on the vector ALUs (gfx950): the recurrence of the linear
// scan with the inner model f(x) = W2 silu(W1 x), both weights d x d.
//
// Inner model: "Edifice.Recurrent.TTT", Options, `:variant` (the `:mlp`
// variant makes the hidden state a two-layer MLP with SiLU) and "Error
// Correction in Trained TTT Layers", abstract (TTT-MLP under the LayerNorm
// squared-error objective); the per-token steps, the 1/d learning-rate
// scaling and the gated output of the updated model: "Edifice.Recurrent.TTT",
// "Equations (TTT-Linear)"; chunk-start gradients: "PonderTTT", "Technical
// Architecture" (dual form).
//
// Per token, with P1, P2 the weights the gradient is taken at (the current
// ones, or the chunk-start ones in the dual form):
//   h = P1 k, a = silu(h), z = P2 a, delta = dL/dz (straight-through, exact
//   LayerNorm Jacobian, or no LayerNorm), da = P2^T delta,
//   dh = da * silu'(h);  W1 -= eta dh k^T,  W2 -= eta delta a^T
//   o = (W2 silu(W1 q)) * sigmoid(gate)        (updated weights)
//
// One workgroup owns one (batch, head) scan.  Row r of W1 (hidden unit r),
// of W2 (output r) and of a copy of W2^T (hidden unit r) live in the VGPRs
// of four adjacent lanes (a DPP quad), each holding d/4 contiguous columns.
// The copy of W2^T makes the back-propagated error P2^T delta another
// quad-local product instead of a reduction over all rows; both copies take
// the same rank-1 update (the same products, so they stay equal).
// Two exchanges through LDS per token, each behind one barrier:
//   1. a = silu(h) of every row, with the previous token's silu(W1 q); every
//      lane reads its d/4 entries of each, finishes the previous token's
//      output and forms z = P2 a;
//   2. z of every row; every lane reads its d/4 entries, reduces the
//      LayerNorm statistics within its quad (two passes: the mean, then the
//      squared deviations from it, so a large mean does not cancel the
//      variance) and forms delta for its own columns and its own row.
// Inputs are staged through LDS in tiles of 2048 elements per array,
// prefetched into registers one tile ahead; outputs are staged in LDS and
// written back as 16-byte stores.
#include "scan_common.h"

#include <type_traits>

namespace ttt {
namespace {

constexpr int kTileElems = 2048;  // elements per array per LDS tile

__device__ __forceinline__ float fast_sigmoid(float x) {
  // exp(-x) saturates to +inf for x = -inf (result 0) and to 0 for +inf (result 1)
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// DPP quad_perm [1,0,3,2] and [2,3,0,1]
__device__ __forceinline__ float quad_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  return x;
}

template <bool BF16>
__device__ __forceinline__ void unpack16(const uint4& w, float* f) {
  if constexpr (BF16) {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(u[i] << 16);
      f[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  } else {
    f[0] = __uint_as_float(w.x);
    f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z);
    f[3] = __uint_as_float(w.w);
  }
}

template <int C>
__device__ __forceinline__ void load_row(const float* p, float (&x)[C]) {
  const float4* p4 = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int c = 0; c < C / 4; ++c) {
    const float4 a = p4[c];
    x[4 * c] = a.x; x[4 * c + 1] = a.y; x[4 * c + 2] = a.z; x[4 * c + 3] = a.w;
  }
}

template <int C>
__device__ __forceinline__ float dot(const float* a, const float* b) {
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < C; ++c) s = fmaf(a[c], b[c], s);
  return s;
}

// delta for one feature from its LayerNorm residual (one definition for the
// row and the column passes, so both give the same bits)
template <int LN>
__device__ __forceinline__ float delta_of(float xh, float e, float gam, float rs, float s1,
                                          float s2) {
  if constexpr (LN == kLnExact) {
    return rs * (gam * e - s1 - xh * s2);
  } else {
    return e;
  }
}

template <int D, bool BF16, int LN, bool DUAL>
__global__ void __launch_bounds__(4 * D)
mlp_valu_kernel(const void* __restrict__ qp, const void* __restrict__ kp,
                const void* __restrict__ vp, const void* __restrict__ etap,
                const void* __restrict__ gatep, const float* __restrict__ W1_0,
                const float* __restrict__ W2_0, const float* __restrict__ gamma,
                const float* __restrict__ beta, float* __restrict__ out,
                float* __restrict__ W1_final, float* __restrict__ W2_final, int H, int64_t T,
                int64_t chunk, float eps) {
  using In = typename std::conditional<BF16, uint16_t, float>::type;
  constexpr int NT = 4 * D;               // threads
  constexpr int C = D / 4;                // columns per lane
  constexpr int TT = kTileElems / D;      // tokens per tile
  constexpr int VE = BF16 ? 8 : 4;        // elements per 16-byte vector
  constexpr int NVEC = kTileElems / VE;   // vectors per array per tile
  constexpr int NV = (NVEC + NT - 1) / NT;
  constexpr int NE = (TT + NT - 1) / NT;  // eta values per thread per tile
  constexpr float kInvD = 1.0f / D;

  __shared__ __align__(16) float sK[kTileElems];
  __shared__ __align__(16) float sQ[kTileElems];
  __shared__ __align__(16) float sV[kTileElems];
  __shared__ __align__(16) float sG[kTileElems];   // sigmoid(gate_logit)
  __shared__ __align__(16) float sO[kTileElems];
  __shared__ float sEta[TT];                       // sigmoid(eta_logit) / d
  __shared__ __align__(16) float sA[D];            // silu(h) of the current token
  __shared__ __align__(16) float sAQ[D];           // silu(W1 q) of the previous token
  __shared__ __align__(16) float sZ[D];            // z of the current token

  const int tid = threadIdx.x;
  const int row = tid >> 2;
  const int seg = tid & 3;
  const int col0 = seg * C;
  const int64_t bh = blockIdx.x;
  const int h = static_cast<int>(bh % H);

  const In* src[4] = {static_cast<const In*>(qp) + bh * T * D,
                      static_cast<const In*>(kp) + bh * T * D,
                      static_cast<const In*>(vp) + bh * T * D,
                      static_cast<const In*>(gatep) + bh * T * D};
  const In* eta = static_cast<const In*>(etap) + bh * T;
  float* dst_out = out + bh * T * D;

  // W1[row][cols], W2[row][cols], W2T[row][cols] = W2[cols][row]
  float W1[C], W2[C], W2T[C];
  float P1[DUAL ? C : 1], P2[DUAL ? C : 1], P2T[DUAL ? C : 1];
  load_row<C>(W1_0 + bh * D * D + row * D + col0, W1);
  load_row<C>(W2_0 + bh * D * D + row * D + col0, W2);
#pragma unroll
  for (int c = 0; c < C; ++c) W2T[c] = W2_0[bh * D * D + (col0 + c) * D + row];

  float gam_r = 1.0f, bet_r = 0.0f;
  float gam_c[C], bet_c[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    gam_c[c] = 1.0f;
    bet_c[c] = 0.0f;
  }
  if constexpr (LN != kLnNone) {
    gam_r = gamma[h * D + row];
    bet_r = beta[h * D + row];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      gam_c[c] = gamma[h * D + col0 + c];
      bet_c[c] = beta[h * D + col0 + c];
    }
  }

  uint4 pre[4][NV];
  float pre_eta[NE];
  auto load_tile = [&](int64_t tile) {
    const int64_t base = tile * TT * D;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
      for (int r = 0; r < NV; ++r) {
        const int vid = tid + r * NT;
        uint4 x = make_uint4(0, 0, 0, 0);
        if (vid < NVEC && tile * TT + (vid * VE) / D < T)
          x = *reinterpret_cast<const uint4*>(src[a] + base + vid * VE);
        pre[a][r] = x;
      }
    }
#pragma unroll
    for (int r = 0; r < NE; ++r) {
      const int j = tid + r * NT;
      const int64_t t = tile * TT + j;
      float x = 0.0f;
      if (j < TT && t < T) {
        if constexpr (BF16)
          x = __uint_as_float(static_cast<uint32_t>(eta[t]) << 16);
        else
          x = eta[t];
      }
      pre_eta[r] = x;
    }
  };
  auto store_tile = [&]() {
    float* dstl[4] = {sQ, sK, sV, sG};
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
      for (int r = 0; r < NV; ++r) {
        const int vid = tid + r * NT;
        if (vid < NVEC) {
          float f[VE];
          unpack16<BF16>(pre[a][r], f);
          if (a == 3) {
#pragma unroll
            for (int j = 0; j < VE; ++j) f[j] = fast_sigmoid(f[j]);
          }
#pragma unroll
          for (int j = 0; j < VE; j += 4)
            *reinterpret_cast<float4*>(dstl[a] + vid * VE + j) =
                make_float4(f[j], f[j + 1], f[j + 2], f[j + 3]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < NE; ++r) {
      const int j = tid + r * NT;
      if (j < TT) sEta[j] = fast_sigmoid(pre_eta[r]) * kInvD;
    }
  };

  // output of the previous token: y = W2 silu(W1 q) from the shared aq
  float gate_prev = 0.0f;
  auto finish_prev = [&](int slot) {
    float aq[C];
    load_row<C>(sAQ + col0, aq);
    const float y = quad_sum(dot<C>(W2, aq));
    if (seg == 0) sO[slot * D + row] = y * gate_prev;
  };

  const int64_t ntiles = (T + TT - 1) / TT;
  int64_t ck = 0;  // position inside the current chunk (dual form)
  if (ntiles > 0) {
    load_tile(0);
    store_tile();
  }
  __syncthreads();
  for (int64_t tile = 0; tile < ntiles; ++tile) {
    if (tile + 1 < ntiles) load_tile(tile + 1);
    const int nt = static_cast<int>(T - tile * TT < TT ? T - tile * TT : TT);
    float aq_prev = 0.0f;
    for (int tt = 0; tt < nt; ++tt) {
      if constexpr (DUAL) {
        if (ck == 0) {
#pragma unroll
          for (int c = 0; c < C; ++c) {
            P1[c] = W1[c];
            P2[c] = W2[c];
            P2T[c] = W2T[c];
          }
        }
        ck = (ck + 1 == chunk) ? 0 : ck + 1;
      }
      // the weights the gradient is taken at
      const float* G1 = DUAL ? P1 : W1;
      const float* G2 = DUAL ? P2 : W2;
      const float* G2T = DUAL ? P2T : W2T;

      float kv[C], qv[C];
      load_row<C>(sK + tt * D + col0, kv);
      load_row<C>(sQ + tt * D + col0, qv);
      const float hk = quad_sum(dot<C>(G1, kv));      // P1 k
      const float hq0 = quad_sum(dot<C>(W1, qv));     // W1_{t-1} q
      const float kq = quad_sum(dot<C>(kv, qv));
      const float sg = fast_sigmoid(hk);
      const float a_r = hk * sg;                       // silu(h)
      const float sp = sg * fmaf(hk, 1.0f - sg, 1.0f); // silu'(h)

      // exchange 1: a of this token, aq of the previous one
      if (seg == 0) {
        sA[row] = a_r;
        if (tt > 0) sAQ[row] = aq_prev;
      }
      __syncthreads();
      if (tt > 0) finish_prev(tt - 1);
      float av[C];
      load_row<C>(sA + col0, av);
      const float z_r = quad_sum(dot<C>(G2, av));      // P2 a

      // exchange 2: z
      if (seg == 0) sZ[row] = z_r;
      __syncthreads();
      float zv[C], vv[C], dv[C];
      load_row<C>(sZ + col0, zv);
      load_row<C>(sV + tt * D + col0, vv);
      const float v_r = sV[tt * D + row];
      float d_r;
      if constexpr (LN == kLnNone) {
#pragma unroll
        for (int c = 0; c < C; ++c) dv[c] = zv[c] - vv[c];
        d_r = z_r - v_r;
      } else {
        float s = 0.0f;
#pragma unroll
        for (int c = 0; c < C; ++c) s += zv[c];
        const float mu = quad_sum(s) * kInvD;
        float m2 = 0.0f;
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const float y = zv[c] - mu;
          m2 = fmaf(y, y, m2);
        }
        const float rs = __builtin_amdgcn_rsqf(quad_sum(m2) * kInvD + eps);
        float xh[C], e[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
          xh[c] = (zv[c] - mu) * rs;
          e[c] = fmaf(gam_c[c], xh[c], bet_c[c]) - vv[c];
        }
        const float xh_r = (z_r - mu) * rs;
        const float e_r = fmaf(gam_r, xh_r, bet_r) - v_r;
        float s1 = 0.0f, s2 = 0.0f;
        if constexpr (LN == kLnExact) {
#pragma unroll
          for (int c = 0; c < C; ++c) {
            const float g = gam_c[c] * e[c];
            s1 += g;
            s2 = fmaf(g, xh[c], s2);
          }
          s1 = quad_sum(s1) * kInvD;
          s2 = quad_sum(s2) * kInvD;
        }
#pragma unroll
        for (int c = 0; c < C; ++c) dv[c] = delta_of<LN>(xh[c], e[c], gam_c[c], rs, s1, s2);
        d_r = delta_of<LN>(xh_r, e_r, gam_r, rs, s1, s2);
      }
      const float da = quad_sum(dot<C>(G2T, dv));     // P2^T delta
      const float dh = da * sp;
      const float et = sEta[tt];
      const float c1 = et * dh;
      const float c2 = et * d_r;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        W1[c] = fmaf(-c1, kv[c], W1[c]);
        W2[c] = fmaf(-c2, av[c], W2[c]);
        W2T[c] = fmaf(-(et * dv[c]), a_r, W2T[c]);
      }
      // W1_t q = W1_{t-1} q - eta dh (k.q); its silu waits for exchange 1 of
      // the next token (or the flush below)
      const float hq = fmaf(-c1, kq, hq0);
      aq_prev = hq * fast_sigmoid(hq);
      gate_prev = sG[tt * D + row];
    }
    // the tile's last output
    if (seg == 0) sAQ[row] = aq_prev;
    __syncthreads();
    finish_prev(nt - 1);
    __syncthreads();
    {
      const int nvec_out = nt * D / 4;
      float4* o4 = reinterpret_cast<float4*>(dst_out + tile * TT * D);
      const float4* s4 = reinterpret_cast<const float4*>(sO);
      for (int i = tid; i < nvec_out; i += NT) o4[i] = s4[i];
    }
    if (tile + 1 < ntiles) store_tile();
    __syncthreads();
  }

  if (W1_final != nullptr) {
    float4* w4 = reinterpret_cast<float4*>(W1_final + bh * D * D + row * D + col0);
#pragma unroll
    for (int c = 0; c < C / 4; ++c)
      w4[c] = make_float4(W1[4 * c], W1[4 * c + 1], W1[4 * c + 2], W1[4 * c + 3]);
  }
  if (W2_final != nullptr) {
    float4* w4 = reinterpret_cast<float4*>(W2_final + bh * D * D + row * D + col0);
#pragma unroll
    for (int c = 0; c < C / 4; ++c)
      w4[c] = make_float4(W2[4 * c], W2[4 * c + 1], W2[4 * c + 2], W2[4 * c + 3]);
  }
}

template <int D, bool BF16, int LN, bool DUAL>
hipError_t launch_one(const ScanArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.B * a.H));
  const dim3 block(4 * D);
  hipLaunchKernelGGL((mlp_valu_kernel<D, BF16, LN, DUAL>), grid, block, 0, s, a.q, a.k, a.v,
                     a.eta_logit, a.gate_logit, a.W0, a.W2_0, a.gamma, a.beta, a.out,
                     a.W_final, a.W2_final, static_cast<int>(a.H), a.T,
                     a.dual ? a.chunk : int64_t(1), a.eps);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_d(const ScanArgs& a, hipStream_t s) {
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
hipError_t launch_dt(const ScanArgs& a, hipStream_t s) {
  return a.in_bf16 ? launch_d<D, true>(a, s) : launch_d<D, false>(a, s);
}

}  // namespace

hipError_t launch_mlp_valu(const ScanArgs& a, hipStream_t s) {
  switch (a.d) {
    case 16: return launch_dt<16>(a, s);
    case 32: return launch_dt<32>(a, s);
    case 64: return launch_dt<64>(a, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace ttt
