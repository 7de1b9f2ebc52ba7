// Input projections of the TTT-Linear layer for d = 64 (gfx950): one bf16
// matrix product that turns x into q, k, v, gate_logit and eta_logit of every
// head, written straight into the scan's input layouts.
//
// "Edifice.Recurrent.TTT", "Equations (TTT-Linear)" (q_t = W_q x_t,
// k_t = W_k x_t, v_t = W_v x_t, the learning-rate gate from W_eta x_t) and
// "Architecture" (the layer projects its input to Q, K, V, eta and gate).
// x [B,T,hidden] and the stacked weights w_proj [H,4d+1,hidden] (per head the
// W_q, W_k, W_v, W_gate rows, then the W_eta row) are bf16; products
// accumulate in fp32 on the 16x16x32 bf16 MFMA; an optional fp32 bias is added
// and the result is stored as bf16 (the scan's bf16 inputs) or fp32.
//
// x is read once for all five projections of all heads.  Output tiles are
// 128 tokens x 128 weight rows of one head (q with k, or v with gate), plus
// tiles holding the eta rows of up to 128 heads.  K runs in steps of 32
// through double-buffered LDS; four waves each own a 64 x 64 block of 4 x 4
// MFMA tiles.  In a 32-deep step lane group G holds k = 8G..8G+7 of its row
// for both operands, so every operand fetch is one 16-byte LDS read; LDS rows
// are padded to 80 bytes so that the 16-byte reads of neighbouring rows fall
// in different banks.  The global loads of the next step are issued before a
// step's MFMAs and are unconditional (a row past the end reads row 0 and is
// replaced by zeros when it is stored to LDS), so their wait comes after the
// MFMAs.
#include "scan_common.h"

#include <cstdint>

namespace ttt {
namespace {

constexpr int D = 64;
constexpr int R = 4 * D + 1;    // weight rows per head
constexpr int TM = 128;         // tokens per tile
constexpr int TN = 128;         // weight rows per tile
constexpr int TK = 32;          // k per step
constexpr int KPAD = TK + 8;    // padded LDS row (bf16): 80 bytes
constexpr int NT = 256;         // threads: four waves
constexpr int NXCD = 8;         // workgroups are dealt round-robin over the XCDs

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct alignas(16) ProjSmem {
  uint16_t A[2][TM][KPAD];   // x rows (tokens), k-contiguous
  uint16_t B[2][TN][KPAD];   // weight rows, k-contiguous
};

__device__ __forceinline__ uint16_t to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

template <bool OUT_BF16>
__global__ void __launch_bounds__(NT)
proj_mfma_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                 const float* __restrict__ bias, void* __restrict__ q, void* __restrict__ k,
                 void* __restrict__ v, void* __restrict__ gate, void* __restrict__ eta,
                 int64_t M, int64_t T, int hidden, int H, int ntn, int64_t mtiles) {
  __shared__ ProjSmem sm;
  // XCD x (workgroups are dealt to the XCDs round-robin) takes the weight
  // tiles nt = x, x + 8, ... for every token tile: its share of the weights
  // stays in its L2 while x streams through, and consecutive workgroups on it
  // share their x rows
  const int xcd = static_cast<int>(blockIdx.x % NXCD);
  const int64_t slot = blockIdx.x / NXCD;
  const int cx = (ntn - xcd + NXCD - 1) / NXCD;     // weight tiles of this XCD
  if (cx == 0) return;
  const int64_t mt = slot / cx;
  if (mt >= mtiles) return;
  const int nt = xcd + NXCD * static_cast<int>(slot % cx);
  const int64_t m0 = mt * TM;
  const bool eta_tile = nt >= 2 * H;
  const int h = eta_tile ? 0 : nt >> 1;        // head of a q/k or v/gate tile
  const int pair = nt & 1;                     // 0: q, k rows; 1: v, gate rows
  const int e0 = eta_tile ? (nt - 2 * H) * TN : 0;   // first head of an eta tile

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int G = lane >> 4;

  // global -> LDS: 512 chunks of 16 bytes per operand and step, two per thread
  const uint16_t* arow[2];
  const uint16_t* brow[2];
  bool aok[2], bok[2];
  int crow[2], cpart[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = tid + NT * j;
    crow[j] = c >> 2;
    cpart[j] = c & 3;
    const int64_t m = m0 + crow[j];
    aok[j] = m < M;
    arow[j] = x + (aok[j] ? m : 0) * hidden + 8 * cpart[j];
    int64_t wr = -1;
    if (!eta_tile) {
      wr = int64_t(h) * R + TN * pair + crow[j];
    } else if (e0 + crow[j] < H) {
      wr = int64_t(e0 + crow[j]) * R + 4 * D;
    }
    bok[j] = wr >= 0;
    brow[j] = w + (bok[j] ? wr : 0) * hidden + 8 * cpart[j];
  }
  uint4 ra[2], rb[2];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      ra[j] = *reinterpret_cast<const uint4*>(arow[j] + k0);
      rb[j] = *reinterpret_cast<const uint4*>(brow[j] + k0);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // rows past the end read a valid row; their data is replaced by zeros here,
      // after this step's MFMAs, so the loads' latency stays hidden
      *reinterpret_cast<uint4*>(&sm.A[buf][crow[j]][8 * cpart[j]]) = aok[j] ? ra[j] : uint4{0, 0, 0, 0};
      *reinterpret_cast<uint4*>(&sm.B[buf][crow[j]][8 * cpart[j]]) = bok[j] ? rb[j] : uint4{0, 0, 0, 0};
    }
  };

  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  const int nk = hidden / TK;
  fetch(0);
  stash(0);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nk) fetch((ks + 1) * TK);   // in flight during this step's MFMAs
    bf16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16x8*>(&sm.A[buf][wm + 16 * i + l16][8 * G]);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const bf16x8*>(&sm.B[buf][wn + 16 * j + l16][8 * G]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    // the other buffer was last read in the previous step, before its barrier
    if (ks + 1 < nk) stash(buf ^ 1);
    __syncthreads();
  }

  // epilogue: D[4G + r][l16] of MFMA tile (i, j) is output row
  // m0 + wm + 16i + 4G + r, weight row wn + 16j + l16 of the tile
  void* const dst4[4] = {q, k, v, gate};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = m0 + wm + 16 * i + 4 * G + r;
      if (m >= M) continue;
      const int64_t bb = m / T, t = m % T;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = wn + 16 * j + l16;
        float y = acc[i][j][r];
        int64_t off;
        void* dst;
        if (!eta_tile) {
          const int kind = 2 * pair + (col >> 6);
          if (bias) y += bias[int64_t(h) * R + TN * pair + col];
          dst = dst4[kind];
          off = ((bb * H + h) * T + t) * D + (col & 63);
        } else {
          const int hh = e0 + col;
          if (hh >= H) continue;
          if (bias) y += bias[int64_t(hh) * R + 4 * D];
          dst = eta;
          off = (bb * H + hh) * T + t;
        }
        if constexpr (OUT_BF16)
          static_cast<uint16_t*>(dst)[off] = to_bf16(y);
        else
          static_cast<float*>(dst)[off] = y;
      }
    }
  }
}

}  // namespace

bool proj_mfma_supports(const ProjArgs& a) { return a.d == D && a.hidden % TK == 0; }

hipError_t launch_proj_mfma(const ProjArgs& a, hipStream_t s) {
  if (!proj_mfma_supports(a)) return hipErrorNotSupported;
  const int64_t M = a.B * a.T;
  if (M == 0) return hipSuccess;
  const int ntn = static_cast<int>(2 * a.H + (a.H + TN - 1) / TN);
  const int64_t mtiles = (M + TM - 1) / TM;
  const int64_t cmax = (ntn + NXCD - 1) / NXCD;     // weight tiles of the busiest XCD
  const int64_t grid = NXCD * cmax * mtiles;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* w = static_cast<const uint16_t*>(a.w);
  if (a.out_bf16)
    hipLaunchKernelGGL((proj_mfma_kernel<true>), dim3(static_cast<unsigned>(grid)), dim3(NT), 0, s,
                       x, w, a.bias, a.q, a.k, a.v, a.gate, a.eta, M, a.T,
                       static_cast<int>(a.hidden), static_cast<int>(a.H), ntn, mtiles);
  else
    hipLaunchKernelGGL((proj_mfma_kernel<false>), dim3(static_cast<unsigned>(grid)), dim3(NT), 0,
                       s, x, w, a.bias, a.q, a.k, a.v, a.gate, a.eta, M, a.T,
                       static_cast<int>(a.hidden), static_cast<int>(a.H), ntn, mtiles);
  return hipGetLastError();
}

}  // namespace ttt
