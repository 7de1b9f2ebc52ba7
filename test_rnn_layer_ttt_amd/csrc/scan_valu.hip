// Per-token TTT-Linear scan on the vector ALUs (gfx950).
//
// Recurrence: "Edifice.Recurrent.TTT", sections "Equations (TTT-Linear)" and
// "Architecture"; exact LayerNorm gradient: "Error Correction in Trained TTT
// Layers", abstract; chunk-start gradients: "PonderTTT", "Technical
// Architecture" (dual-form updates).
//
// One workgroup owns one (batch, head) scan.  Row i of W lives in the VGPRs of
// four adjacent lanes (a DPP quad), each holding d/4 contiguous columns, so
// W k and W q need only a two-step quad reduction.  The LayerNorm statistics
// of z = W k are reduced over the rows with DPP row rotations, a cross-row
// shuffle and, with more than one wave, one LDS exchange and barrier per token
// (two in exact mode); each wave sums its rows shifted by one of its own
// entries and the waves' means and squared deviations combine exactly, so the
// variance does not cancel when the mean of z is large against its spread.  Inputs are staged through LDS in tiles of 2048
// elements per array, prefetched into registers one tile ahead, converted to
// fp32 and passed through their sigmoids on the way in; outputs are staged in
// LDS and written back as 16-byte stores.
//
// The output uses the updated weight through o = W_{t-1} q - eta*delta (k.q),
// which equals W_t q exactly in real arithmetic and keeps the rank-1 update
// off the output's dependency chain.
//
// The recording instantiation (REC) also writes what the backward replays:
// delta_t of every token (staged in LDS with the outputs, written per tile)
// and the running W before every 16th token (in the dual form too, where it
// includes the chunk's updates so far).
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

// DPP controls: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_ror:4, row_ror:8
constexpr int kQuadXor1 = 0xB1;
constexpr int kQuadXor2 = 0x4E;
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

__device__ __forceinline__ float quad_sum(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  return x;
}

// x of this lane plus x of lane ^ 16 (^ 32): v_permlane16_swap /
// v_permlane32_swap of x with itself, on the vector ALU (no LDS round trip);
// the two swapped registers hold the lane's own value and its partner's
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over the 16 quads of a wave of a value that is uniform within each quad.
__device__ __forceinline__ float quads_sum(float x) {
  x += dpp<kRowRor4>(x);
  x += dpp<kRowRor8>(x);
  x = xor16_sum(x);
  return xor32_sum(x);
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

template <int D, bool BF16, int LN, bool DUAL, bool REC>
__global__ void __launch_bounds__(4 * D)
scan_valu_kernel(const void* __restrict__ qp, const void* __restrict__ kp,
                 const void* __restrict__ vp, const void* __restrict__ etap,
                 const void* __restrict__ gatep, const float* __restrict__ W0,
                 const float* __restrict__ gamma, const float* __restrict__ beta,
                 float* __restrict__ out, float* __restrict__ W_final,
                 int H, int64_t T, int64_t chunk, float eps,
                 const uint8_t* __restrict__ upd_mask, int silu,
                 float* __restrict__ rec_delta, float* __restrict__ rec_W) {
  using In = typename std::conditional<BF16, uint16_t, float>::type;
  constexpr int NT = 4 * D;               // threads
  constexpr int NW = NT / 64;             // waves
  constexpr int C = D / 4;                // W columns per lane
  constexpr int TT = kTileElems / D;      // tokens per tile
  constexpr int VE = BF16 ? 8 : 4;        // elements per 16-byte vector
  constexpr int NVEC = kTileElems / VE;   // vectors per array per tile
  constexpr int NV = (NVEC + NT - 1) / NT;
  constexpr int NE = (TT + NT - 1) / NT;   // eta values per thread per tile
  constexpr float kInvD = 1.0f / D;
  static_assert(TT % kRecTile == 0, "a tile must hold whole recorded-W intervals");

  __shared__ __align__(16) float sK[kTileElems];
  __shared__ __align__(16) float sQ[kTileElems];
  __shared__ __align__(16) float sV[kTileElems];
  __shared__ __align__(16) float sG[kTileElems];   // sigmoid(gate_logit)
  __shared__ __align__(16) float sO[kTileElems];
  __shared__ __align__(16) float sDel[REC ? kTileElems : 4];   // delta_t, recorded
  __shared__ float sEta[TT];                       // sigmoid(eta_logit) / d
  __shared__ float2 sRed[2][2][NW];                // [reduction][token parity][wave]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row = tid >> 2;
  const int seg = tid & 3;
  const int64_t bh = blockIdx.x;
  const int h = static_cast<int>(bh % H);

  const In* src[4] = {static_cast<const In*>(qp) + bh * T * D,
                      static_cast<const In*>(kp) + bh * T * D,
                      static_cast<const In*>(vp) + bh * T * D,
                      static_cast<const In*>(gatep) + bh * T * D};
  const In* eta = static_cast<const In*>(etap) + bh * T;
  // dual form: SKIP (0) / UPDATE decisions of this scan's chunks
  const uint8_t* mrow =
      (DUAL && upd_mask != nullptr) ? upd_mask + bh * ((T + chunk - 1) / chunk) : nullptr;
  float* dst_out = out + bh * T * D;
  const int64_t nrec = (T + kRecTile - 1) / kRecTile;   // recorded W per scan

  float W[C];
  float Wc[DUAL ? C : 1];
  {
    const float4* w4 = reinterpret_cast<const float4*>(W0 + bh * D * D + row * D + seg * C);
#pragma unroll
    for (int c = 0; c < C / 4; ++c) {
      const float4 x = w4[c];
      W[4 * c] = x.x; W[4 * c + 1] = x.y; W[4 * c + 2] = x.z; W[4 * c + 3] = x.w;
    }
  }
  float gam = 1.0f, bet = 0.0f;
  if constexpr (LN != kLnNone) {
    gam = gamma[h * D + row];
    bet = beta[h * D + row];
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
        // a skipped chunk: eta_logit = -inf, whose sigmoid is exactly 0
        if (mrow != nullptr && mrow[t / chunk] == 0) x = -__builtin_huge_valf();
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
          if (silu && a <= 1) {
            // the :mlp variant: SiLU on q and k before the inner model
#pragma unroll
            for (int j = 0; j < VE; ++j) f[j] = f[j] * fast_sigmoid(f[j]);
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

  int par = 0;
  // Mean and biased variance of z over the d rows; every thread gets them.
  // Each wave shifts its 16 rows by one of its own entries, sums the shifted
  // values and their squares, and turns them into the wave's mean and its sum
  // of squared deviations from that mean; the waves' parts then combine in the
  // parallel form of the variance (the spread of the wave means is added
  // explicitly).  No E[z^2] - E[z]^2 of a large mean is ever formed, so the
  // statistic does not cancel when |mean(z)| >> std(z).
  constexpr int kRowsPerWave = 16;
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
      if (lane == 0) sRed[0][par][wave] = make_float2(mw, m2w);
      __syncthreads();
      float mu = 0.0f, m2 = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float2 x = sRed[0][par][w];
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
  // Sum of two per-row values over all d rows; every thread gets the result.
  auto rows_sum2 = [&](float a, float b, int red) -> float2 {
    a = quads_sum(a);
    b = quads_sum(b);
    if constexpr (NW == 1) {
      return make_float2(a, b);
    } else {
      if (lane == 0) sRed[red][par][wave] = make_float2(a, b);
      __syncthreads();
      float2 r = sRed[red][par][0];
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        const float2 x = sRed[red][par][w];
        r.x += x.x;
        r.y += x.y;
      }
      return r;
    }
  };

  const int64_t ntiles = (T + TT - 1) / TT;
  int64_t ck = 0;  // position inside the current chunk (dual mode)
  if (ntiles > 0) {
    load_tile(0);
    store_tile();
  }
  __syncthreads();
  for (int64_t tile = 0; tile < ntiles; ++tile) {
    if (tile + 1 < ntiles) load_tile(tile + 1);
    const int nt = static_cast<int>(T - tile * TT < TT ? T - tile * TT : TT);
    for (int tt = 0; tt < nt; ++tt) {
      if constexpr (REC) {
        // W before token tile*TT + tt, at every 16th token (TT is a multiple of 16)
        if (tt % kRecTile == 0) {
          float4* w4 = reinterpret_cast<float4*>(
              rec_W + ((bh * nrec + (tile * TT + tt) / kRecTile) * D + row) * D + seg * C);
#pragma unroll
          for (int c = 0; c < C / 4; ++c)
            w4[c] = make_float4(W[4 * c], W[4 * c + 1], W[4 * c + 2], W[4 * c + 3]);
        }
      }
      if constexpr (DUAL) {
        if (ck == 0) {
#pragma unroll
          for (int c = 0; c < C; ++c) Wc[c] = W[c];
        }
        ck = (ck + 1 == chunk) ? 0 : ck + 1;
      }
      float kv[C], qv[C];
      {
        const float4* k4 = reinterpret_cast<const float4*>(sK + tt * D + seg * C);
        const float4* q4 = reinterpret_cast<const float4*>(sQ + tt * D + seg * C);
#pragma unroll
        for (int c = 0; c < C / 4; ++c) {
          const float4 a = k4[c];
          const float4 b = q4[c];
          kv[4 * c] = a.x; kv[4 * c + 1] = a.y; kv[4 * c + 2] = a.z; kv[4 * c + 3] = a.w;
          qv[4 * c] = b.x; qv[4 * c + 1] = b.y; qv[4 * c + 2] = b.z; qv[4 * c + 3] = b.w;
        }
      }
      float z = 0.0f, u = 0.0f, kq = 0.0f;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        z = fmaf(DUAL ? Wc[DUAL ? c : 0] : W[c], kv[c], z);
        u = fmaf(W[c], qv[c], u);
        kq = fmaf(kv[c], qv[c], kq);
      }
      z = quad_sum(z);
      u = quad_sum(u);
      kq = quad_sum(kq);
      const float vi = sV[tt * D + row];
      const float gi = sG[tt * D + row];
      const float et = sEta[tt];
      float delta;
      if constexpr (LN == kLnNone) {
        delta = z - vi;
      } else {
        const float2 st = ln_stats(z);
        const float mu = st.x;
        const float rs = __builtin_amdgcn_rsqf(st.y + eps);
        const float xh = (z - mu) * rs;
        const float e = fmaf(gam, xh, bet) - vi;
        if constexpr (LN == kLnST) {
          delta = e;
        } else {
          const float g = gam * e;
          const float2 s2 = rows_sum2(g, g * xh, 1);
          delta = rs * (g - s2.x * kInvD - xh * (s2.y * kInvD));
        }
      }
      const float ci = et * delta;
#pragma unroll
      for (int c = 0; c < C; ++c) W[c] = fmaf(-ci, kv[c], W[c]);
      const float o = fmaf(-ci, kq, u) * gi;
      if (seg == 0) {
        sO[tt * D + row] = o;
        if constexpr (REC) sDel[tt * D + row] = delta;
      }
      par ^= 1;
    }
    __syncthreads();
    {
      const int nvec_out = nt * D / 4;
      float4* o4 = reinterpret_cast<float4*>(dst_out + tile * TT * D);
      const float4* s4 = reinterpret_cast<const float4*>(sO);
      for (int i = tid; i < nvec_out; i += NT) o4[i] = s4[i];
      if constexpr (REC) {
        float4* d4 = reinterpret_cast<float4*>(rec_delta + (bh * T + tile * TT) * D);
        const float4* sd4 = reinterpret_cast<const float4*>(sDel);
        for (int i = tid; i < nvec_out; i += NT) d4[i] = sd4[i];
      }
    }
    if (tile + 1 < ntiles) store_tile();
    __syncthreads();
  }

  if (W_final != nullptr) {
    float4* w4 = reinterpret_cast<float4*>(W_final + bh * D * D + row * D + seg * C);
#pragma unroll
    for (int c = 0; c < C / 4; ++c)
      w4[c] = make_float4(W[4 * c], W[4 * c + 1], W[4 * c + 2], W[4 * c + 3]);
  }
}

template <int D, bool BF16, int LN, bool DUAL>
hipError_t launch_one(const ScanArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.B * a.H));
  const dim3 block(4 * D);
  if (a.rec_delta != nullptr)
    hipLaunchKernelGGL((scan_valu_kernel<D, BF16, LN, DUAL, true>), grid, block, 0, s, a.q, a.k,
                       a.v, a.eta_logit, a.gate_logit, a.W0, a.gamma, a.beta, a.out, a.W_final,
                       static_cast<int>(a.H), a.T, a.dual ? a.chunk : int64_t(1), a.eps,
                       a.upd_mask, a.silu_qk ? 1 : 0, a.rec_delta, a.rec_W);
  else
    hipLaunchKernelGGL((scan_valu_kernel<D, BF16, LN, DUAL, false>), grid, block, 0, s, a.q,
                       a.k, a.v, a.eta_logit, a.gate_logit, a.W0, a.gamma, a.beta, a.out,
                       a.W_final, static_cast<int>(a.H), a.T, a.dual ? a.chunk : int64_t(1),
                       a.eps, a.upd_mask, a.silu_qk ? 1 : 0, nullptr, nullptr);
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

hipError_t launch_scan_valu(const ScanArgs& a, hipStream_t s) {
  switch (a.d) {
    case 16: return launch_dt<16>(a, s);
    case 32: return launch_dt<32>(a, s);
    case 64: return launch_dt<64>(a, s);
    case 128: return launch_dt<128>(a, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace ttt
