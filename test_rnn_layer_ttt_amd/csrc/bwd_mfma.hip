// Backward of the per-token TTT-Linear scan for d = 64 (gfx950).
//
// Recurrence: "Edifice.Recurrent.TTT", "Equations (TTT-Linear)"; exact
// LayerNorm gradient: "Error Correction in Trained TTT Layers", abstract.  The
// gradients are those of a loss L through out and W_final: reverse-mode
// through every step of the forward.
//
// A forward pass first records delta_t and W at the start of every tile of 16
// tokens.  The tiles are then walked backwards.  With W_c the weight at the
// tile start, E_s = eta_s delta_s, H the gradient with respect to the weight
// after the tile, dy_t = dout_t * sigmoid(g_t), and G_t the gradient with
// respect to W_t, the tile's algebra is (rows are tokens):
//
//   z_t  = W_c k_t - sum_{s<t} (k_s.k_t) E_s           (z of the forward)
//   y_t  = W_c q_t - sum_{s<=t} (q_t.k_s) E_s          (W_t q_t)
//   a_t  = G_t k_t = H k_t + sum_{t'>=t} (q_t'.k_t) dy_t' + sum_{t'>t} (k_t'.k_t) dz_t'
//   d delta_t = -eta_t a_t,  d eta_t = -delta_t . a_t,  dz_t = VJP of delta(z_t)
//   dk_t = -eta_t G_t^T delta_t + W_{t-1}^T dz_t
//        = -eta_t [H^T delta_t + sum_{t'>=t} (delta_t.dy_t') q_t' + sum_{t'>t} (delta_t.dz_t') k_t']
//          + W_c^T dz_t - sum_{s<t} eta_s (delta_s.dz_t) k_s
//   dq_t = W_t^T dy_t = W_c^T dy_t - sum_{s<=t} eta_s (delta_s.dy_t) k_s
//   H   <- H + sum_t dy_t q_t^T + sum_t dz_t k_t^T          (gradient before the tile)
//
// Everything but the dz_t chain is a dense tile contraction on the matrix
// cores (fp32 16x16x4, all operands from LDS, so either orientation of a
// matrix is only a matter of addressing).  The chain (the a_t corrections and
// the LayerNorm VJP, one wave, lane = feature) is serial.  One workgroup of 8
// waves per (batch, head); phases separated by barriers.
#include "scan_common.h"

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

// D[4G + r][l16] += sum_k A[l16][k] B[k][l16] over a 4-deep k-step
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// sum over the 64 lanes, in every lane (row scan, two row broadcasts, readlane)
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
#pragma clang fp contract(off)
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float rl63(float x) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
__device__ __forceinline__ float wave_sum1(float a) {
  a = dpp_add<0x111>(a);
  a = dpp_add<0x112>(a);
  a = dpp_add<0x114>(a);
  a = dpp_add<0x118>(a);
  a = dpp_add<0x142>(a);
  a = dpp_add<0x143>(a);
  return rl63(a);
}
__device__ __forceinline__ void wave_sum2(float& a, float& b) {
  a = dpp_add<0x111>(a); b = dpp_add<0x111>(b);
  a = dpp_add<0x112>(a); b = dpp_add<0x112>(b);
  a = dpp_add<0x114>(a); b = dpp_add<0x114>(b);
  a = dpp_add<0x118>(a); b = dpp_add<0x118>(b);
  a = dpp_add<0x142>(a); b = dpp_add<0x142>(b);
  a = dpp_add<0x143>(a); b = dpp_add<0x143>(b);
  a = rl63(a); b = rl63(b);
}
__device__ __forceinline__ void wave_sum3(float& a, float& b, float& c) {
  a = dpp_add<0x111>(a); b = dpp_add<0x111>(b); c = dpp_add<0x111>(c);
  a = dpp_add<0x112>(a); b = dpp_add<0x112>(b); c = dpp_add<0x112>(c);
  a = dpp_add<0x114>(a); b = dpp_add<0x114>(b); c = dpp_add<0x114>(c);
  a = dpp_add<0x118>(a); b = dpp_add<0x118>(b); c = dpp_add<0x118>(c);
  a = dpp_add<0x142>(a); b = dpp_add<0x142>(b); c = dpp_add<0x142>(c);
  a = dpp_add<0x143>(a); b = dpp_add<0x143>(b); c = dpp_add<0x143>(c);
  a = rl63(a); b = rl63(b); c = rl63(c);
}

struct alignas(16) BwdSmem {
  float Wc[D][KP];         // W at the tile start, [i][j]
  float Hm[2][D][KP];      // gradient w.r.t. the weight after the tile, [i][j]
  float Q[BT][KP], K[BT][KP], V[BT][KP], DO[BT][KP], SG[BT][KP], De[BT][KP];
  float Z[BT][KP], A0[BT][KP], DZ[BT][KP], XH[BT][KP];
  float KK[BT][TP], QK[BT][TP], DeDY[BT][TP], DeDZ[BT][TP];
  float ETA[BT], ELD[BT], RS[BT];   // eta, sigmoid'(eta_logit)/d, 1/sqrt(var+eps)
};

template <bool BF16>
__device__ __forceinline__ float ld_in(const void* p, int64_t i) {
  if constexpr (BF16)
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
  else
    return static_cast<const float*>(p)[i];
}

// one 16 x 16 output block: sum over k-steps of A(m, k) B(k, n) (accessors
// take the lane's row m = l16 and column n = l16 and the k index)
template <typename FA, typename FB>
__device__ __forceinline__ f32x4 block_mfma(int ksteps, FA A, FB B, f32x4 acc, int l16, int G) {
  for (int ks = 0; ks < ksteps; ++ks) {
    const int k = 4 * ks + G;
    acc = mfma4(A(l16, k), B(k, l16), acc);
  }
  return acc;
}

template <bool BF16, int LN>
__global__ void __launch_bounds__(NT)
bwd_mfma_kernel(const void* __restrict__ qp, const void* __restrict__ kp,
                const void* __restrict__ vp, const void* __restrict__ etap,
                const void* __restrict__ gatep, const float* __restrict__ gamma,
                const float* __restrict__ beta, const float* __restrict__ dout,
                const float* __restrict__ dW_final, const float* __restrict__ rec_delta,
                const float* __restrict__ rec_W, float* __restrict__ dq, float* __restrict__ dk,
                float* __restrict__ dv, float* __restrict__ deta, float* __restrict__ dgate,
                float* __restrict__ dW0, float* __restrict__ gb_part, int H, int64_t T,
                float eps) {
  __shared__ BwdSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int G = lane >> 4;
  const int64_t bh = blockIdx.x;
  const int h = static_cast<int>(bh % H);
  const int64_t bhT = bh * T;
  const int64_t ntiles = (T + BT - 1) / BT;

  // H starts as dL/dW_final
  for (int e = tid; e < D * D; e += NT) {
    const int i = e / D, j = e % D;
    sm.Hm[0][i][j] = dW_final != nullptr ? dW_final[bh * D * D + e] : 0.0f;
  }
  // serial wave: LayerNorm affine of feature `lane`, gradient accumulators
  float gam = 1.0f, bet = 0.0f, dgam = 0.0f, dbet = 0.0f;
  if (wave == 0 && LN != kLnNone) {
    gam = gamma[h * D + lane];
    bet = beta[h * D + lane];
  }
  int cur = 0;

  for (int64_t c = ntiles - 1; c >= 0; --c) {
    const int64_t t0 = c * BT;
    const int n = static_cast<int>(min<int64_t>(BT, T - t0));
    // ---- load the tile (rows past the end are zero) and W_c ----
    for (int e = tid; e < BT * D; e += NT) {
      const int t = e / D, i = e % D;
      const bool in = t < n;
      const int64_t g = (bhT + t0 + t) * D + i;
      sm.Q[t][i] = in ? ld_in<BF16>(qp, g) : 0.0f;
      sm.K[t][i] = in ? ld_in<BF16>(kp, g) : 0.0f;
      sm.V[t][i] = in ? ld_in<BF16>(vp, g) : 0.0f;
      sm.DO[t][i] = in ? dout[g] : 0.0f;
      sm.SG[t][i] = in ? sigmoidf_(ld_in<BF16>(gatep, g)) : 0.0f;
      sm.De[t][i] = in ? rec_delta[g] : 0.0f;
      sm.DZ[t][i] = 0.0f;
    }
    if (tid < BT) {
      const bool in = tid < n;
      const float s = in ? sigmoidf_(ld_in<BF16>(etap, bhT + t0 + tid)) : 0.0f;
      sm.ETA[tid] = s * (1.0f / D);
      sm.ELD[tid] = s * (1.0f - s) * (1.0f / D);
    }
    for (int e = tid; e < D * D / 4; e += NT) {
      const int i = (4 * e) / D, j = (4 * e) % D;
      const float4 w = *reinterpret_cast<const float4*>(rec_W + ((bh * ntiles + c) * D + i) * D + j);
      *reinterpret_cast<float4*>(&sm.Wc[i][j]) = w;
    }
    __syncthreads();
    // ---- token Gram matrices KK[s][t] = k_s.k_t, QK[t][s] = q_t.k_s ----
    if (wave < 2) {
      const float (*A)[KP] = wave == 0 ? sm.K : sm.Q;
      f32x4 acc = {0, 0, 0, 0};
      acc = block_mfma(16, [&](int m, int k) { return A[m][k]; },
                       [&](int k, int nn) { return sm.K[nn][k]; }, acc, l16, G);
      float (*O)[TP] = wave == 0 ? sm.KK : sm.QK;
#pragma unroll
      for (int r = 0; r < 4; ++r) O[4 * G + r][l16] = acc[r];
    }
    __syncthreads();
    // ---- z (waves 0-3), y and dgate (waves 0-3), a0 (waves 4-7), by feature slice ----
    {
      const int sl = wave & 3;
      const int f = 16 * sl + l16;
      const float (*Hc)[KP] = sm.Hm[cur];
      if (wave < 4) {
        // z_t = W_c k_t - sum_{s<t} (k_s.k_t) eta_s delta_s
        f32x4 z = {0, 0, 0, 0};
        z = block_mfma(16, [&](int m, int k) { return sm.K[m][k]; },
                       [&](int k, int nn) { return sm.Wc[16 * sl + nn][k]; }, z, l16, G);
        z = block_mfma(4, [&](int m, int k) { return k < m ? -sm.KK[m][k] : 0.0f; },
                       [&](int k, int nn) { return sm.ETA[k] * sm.De[k][16 * sl + nn]; }, z, l16, G);
        // y_t = W_c q_t - sum_{s<=t} (q_t.k_s) eta_s delta_s
        f32x4 y = {0, 0, 0, 0};
        y = block_mfma(16, [&](int m, int k) { return sm.Q[m][k]; },
                       [&](int k, int nn) { return sm.Wc[16 * sl + nn][k]; }, y, l16, G);
        y = block_mfma(4, [&](int m, int k) { return k <= m ? -sm.QK[m][k] : 0.0f; },
                       [&](int k, int nn) { return sm.ETA[k] * sm.De[k][16 * sl + nn]; }, y, l16, G);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 4 * G + r;
          sm.Z[t][f] = z[r];
          if (t < n) {
            const float s = sm.SG[t][f];
            dgate[(bhT + t0 + t) * D + f] = sm.DO[t][f] * y[r] * s * (1.0f - s);
          }
        }
      } else {
        // a0_t = H k_t + sum_{t'>=t} (q_t'.k_t) dy_t'
        f32x4 a = {0, 0, 0, 0};
        a = block_mfma(16, [&](int m, int k) { return sm.K[m][k]; },
                       [&](int k, int nn) { return Hc[16 * sl + nn][k]; }, a, l16, G);
        a = block_mfma(4, [&](int m, int k) { return k >= m ? sm.QK[k][m] : 0.0f; },
                       [&](int k, int nn) { return sm.DO[k][16 * sl + nn] * sm.SG[k][16 * sl + nn]; },
                       a, l16, G);
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.A0[4 * G + r][f] = a[r];
      }
    }
    __syncthreads();
    // ---- LayerNorm statistics of z: two tokens per wave ----
    if (LN != kLnNone) {
      for (int t = 2 * wave; t < 2 * wave + 2; ++t) {
        const float z = sm.Z[t][lane];
        float s1 = z, s2 = z * z;
        wave_sum2(s1, s2);
        const float mu = s1 * (1.0f / D);
        const float var = fmaf(s2, 1.0f / D, -mu * mu);
        const float rs = __builtin_amdgcn_rsqf(fmaxf(var + eps, eps));
        sm.XH[t][lane] = (z - mu) * rs;
        if (lane == 0) sm.RS[t] = rs;
      }
    }
    __syncthreads();
    // ---- the serial chain, t descending (wave 0, lane = feature) ----
    if (wave == 0) {
      float dzr[BT];
#pragma unroll
      for (int t = 0; t < BT; ++t) dzr[t] = 0.0f;
#pragma unroll
      for (int t = BT - 1; t >= 0; --t) {
        if (t < n) {
          float a = sm.A0[t][lane];
#pragma unroll
          for (int tp = t + 1; tp < BT; ++tp) a = fmaf(sm.KK[t][tp], dzr[tp], a);
          const float eta = sm.ETA[t];
          const float dd = -eta * a;
          const float del = sm.De[t][lane];
          float dz, dvv;
          float deta_sum = -del * a;
          if constexpr (LN == kLnNone) {
            deta_sum = wave_sum1(deta_sum);
            dz = dd;
            dvv = -dd;
          } else if constexpr (LN == kLnST) {
            const float xh = sm.XH[t][lane];
            const float rs = sm.RS[t];
            const float w = gam * dd;
            float sw = w, swx = w * xh;
            wave_sum3(deta_sum, sw, swx);
            dz = rs * (w - sw * (1.0f / D) - xh * (swx * (1.0f / D)));
            dvv = -dd;
            dgam = fmaf(dd, xh, dgam);
            dbet += dd;
          } else {
            // delta = rs (g - mean g - xh mean(g xh)), g = gam e, e = gam xh + bet - v
            const float xh = sm.XH[t][lane];
            const float rs = sm.RS[t];
            const float e = fmaf(gam, xh, bet - sm.V[t][lane]);
            const float g = gam * e;
            float mg = g, mgx = g * xh;
            wave_sum3(mg, mgx, deta_sum);
            mg *= (1.0f / D);
            mgx *= (1.0f / D);
            const float P = g - mg - xh * mgx;
            const float dP = rs * dd;
            float drs = dd * P, sdp = dP, sdpx = dP * xh;
            wave_sum3(drs, sdp, sdpx);
            const float dmgx = -sdpx;
            const float dg = dP - sdp * (1.0f / D) + dmgx * xh * (1.0f / D);
            float dxh = -dP * mgx + dmgx * g * (1.0f / D);
            const float de = gam * dg;
            dgam += fmaf(e, dg, xh * de);
            dbet += de;
            dvv = -de;
            dxh = fmaf(gam, de, dxh);
            float sx = dxh, sxx = dxh * xh;
            wave_sum2(sx, sxx);
            dz = rs * (dxh - sx * (1.0f / D) - xh * (sxx * (1.0f / D)))
                 - drs * rs * rs * xh * (1.0f / D);
          }
          dzr[t] = dz;
          sm.DZ[t][lane] = dz;
          dv[(bhT + t0 + t) * D + lane] = dvv;
          if (lane == 0) deta[bhT + t0 + t] = deta_sum * sm.ELD[t];
        }
      }
    }
    __syncthreads();
    // ---- Gram matrices DeDY[s][t'] = delta_s.dy_t', DeDZ[s][t'] = delta_s.dz_t' ----
    if (wave < 2) {
      f32x4 acc = {0, 0, 0, 0};
      if (wave == 0)
        acc = block_mfma(16, [&](int m, int k) { return sm.De[m][k]; },
                         [&](int k, int nn) { return sm.DO[nn][k] * sm.SG[nn][k]; }, acc, l16, G);
      else
        acc = block_mfma(16, [&](int m, int k) { return sm.De[m][k]; },
                         [&](int k, int nn) { return sm.DZ[nn][k]; }, acc, l16, G);
      float (*O)[TP] = wave == 0 ? sm.DeDY : sm.DeDZ;
#pragma unroll
      for (int r = 0; r < 4; ++r) O[4 * G + r][l16] = acc[r];
    }
    __syncthreads();
    // ---- dK, dQ (waves 0-3 / 4-7 by column slice) and the new H (all waves) ----
    {
      const int sl = wave & 3;
      const int j = 16 * sl + l16;
      const float (*Hc)[KP] = sm.Hm[cur];
      if (wave < 4) {
        f32x4 b1 = {0, 0, 0, 0}, b2 = {0, 0, 0, 0};
        b1 = block_mfma(16, [&](int m, int k) { return sm.De[m][k]; },
                        [&](int k, int nn) { return Hc[k][16 * sl + nn]; }, b1, l16, G);
        b1 = block_mfma(4, [&](int m, int k) { return k >= m ? sm.DeDY[m][k] : 0.0f; },
                        [&](int k, int nn) { return sm.Q[k][16 * sl + nn]; }, b1, l16, G);
        b1 = block_mfma(4, [&](int m, int k) { return k > m ? sm.DeDZ[m][k] : 0.0f; },
                        [&](int k, int nn) { return sm.K[k][16 * sl + nn]; }, b1, l16, G);
        b2 = block_mfma(16, [&](int m, int k) { return sm.DZ[m][k]; },
                        [&](int k, int nn) { return sm.Wc[k][16 * sl + nn]; }, b2, l16, G);
        b2 = block_mfma(4, [&](int m, int k) { return k < m ? -sm.ETA[k] * sm.DeDZ[k][m] : 0.0f; },
                        [&](int k, int nn) { return sm.K[k][16 * sl + nn]; }, b2, l16, G);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 4 * G + r;
          if (t < n) dk[(bhT + t0 + t) * D + j] = fmaf(-sm.ETA[t], b1[r], b2[r]);
        }
      } else {
        f32x4 q = {0, 0, 0, 0};
        q = block_mfma(16, [&](int m, int k) { return sm.DO[m][k] * sm.SG[m][k]; },
                       [&](int k, int nn) { return sm.Wc[k][16 * sl + nn]; }, q, l16, G);
        q = block_mfma(4, [&](int m, int k) { return k <= m ? -sm.ETA[k] * sm.DeDY[k][m] : 0.0f; },
                       [&](int k, int nn) { return sm.K[k][16 * sl + nn]; }, q, l16, G);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 4 * G + r;
          if (t < n) dq[(bhT + t0 + t) * D + j] = q[r];
        }
      }
      // H_new[i][j] = H[i][j] + sum_t dy_t[i] q_t[j] + dz_t[i] k_t[j]: 16 blocks, 2 per wave
      for (int blk = wave; blk < 16; blk += NWAVES) {
        const int ib = blk / 4, jb = blk % 4;
        f32x4 acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = Hc[16 * ib + 4 * G + r][16 * jb + l16];
        acc = block_mfma(4, [&](int m, int k) { return sm.DO[k][16 * ib + m] * sm.SG[k][16 * ib + m]; },
                         [&](int k, int nn) { return sm.Q[k][16 * jb + nn]; }, acc, l16, G);
        acc = block_mfma(4, [&](int m, int k) { return sm.DZ[k][16 * ib + m]; },
                         [&](int k, int nn) { return sm.K[k][16 * jb + nn]; }, acc, l16, G);
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.Hm[cur ^ 1][16 * ib + 4 * G + r][16 * jb + l16] = acc[r];
      }
    }
    cur ^= 1;
    __syncthreads();
  }
  // dW0 and this scan's share of dgamma, dbeta
  for (int e = tid; e < D * D; e += NT) dW0[bh * D * D + e] = sm.Hm[cur][e / D][e % D];
  if (wave == 0 && gb_part != nullptr) {
    gb_part[(bh * 2) * D + lane] = dgam;
    gb_part[(bh * 2 + 1) * D + lane] = dbet;
  }
}

// dgamma[h][i] = sum_b (partial), dbeta likewise (deterministic order)
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

template <bool BF16, int LN>
hipError_t launch_bwd(const BwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((bwd_mfma_kernel<BF16, LN>), dim3(static_cast<unsigned>(a.B * a.H)), dim3(NT),
                     0, s, a.q, a.k, a.v, a.eta_logit, a.gate_logit, a.gamma, a.beta, a.dout,
                     a.dW_final, a.rec_delta, a.rec_W, a.dq, a.dk, a.dv, a.deta_logit,
                     a.dgate_logit, a.dW0, LN == kLnNone ? nullptr : a.gb_part,
                     static_cast<int>(a.H), a.T, a.eps);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || LN == kLnNone) return err;
  const int64_t n = a.H * D;
  hipLaunchKernelGGL(gamma_beta_sum_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                     0, s, a.gb_part, a.dgamma, a.dbeta, a.B, a.H);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_mfma(const BwdArgs& a, hipStream_t s) {
  if (a.d != D || a.dual) return hipErrorNotSupported;
  if (a.in_bf16) {
    switch (a.ln) {
      case kLnST: return launch_bwd<true, kLnST>(a, s);
      case kLnExact: return launch_bwd<true, kLnExact>(a, s);
      default: return launch_bwd<true, kLnNone>(a, s);
    }
  }
  switch (a.ln) {
    case kLnST: return launch_bwd<false, kLnST>(a, s);
    case kLnExact: return launch_bwd<false, kLnExact>(a, s);
    default: return launch_bwd<false, kLnNone>(a, s);
  }
}

}  // namespace ttt
