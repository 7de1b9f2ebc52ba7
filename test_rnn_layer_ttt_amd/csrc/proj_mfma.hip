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
// tiles holding the eta rows of up to 128 heads.  Four waves each own a
// 64 x 64 block of 4 x 4 MFMA tiles; in a 32-deep step lane group G holds
// k = 8G..8G+7 of its row for both operands, so every operand fetch is one
// 16-byte LDS read.  Operands go from global memory straight into LDS
// (global_load_lds, 16 bytes per lane, a wave filling 1 KiB of consecutive
// LDS) through a ring of three K steps: the loads of step ks+2 are issued
// while step ks is computed, without holding registers.  LDS rows are 64
// bytes; the 16-byte chunks of a row are XOR-swizzled with the row index so
// that the reads of neighbouring rows fall in different banks.
#include "scan_common.h"

#include <cstdint>

namespace ttt {
namespace {

constexpr int D = 64;
constexpr int R = 4 * D + 1;    // weight rows per head
constexpr int TM = 128;         // tokens per tile
constexpr int TN = 128;         // weight rows per tile
constexpr int TK = 32;          // k per step
constexpr int NSTAGE = 3;       // LDS ring of K steps in flight
constexpr int NT = 256;         // threads: four waves
constexpr int NXCD = 8;         // workgroups are dealt round-robin over the XCDs

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct alignas(16) ProjSmem {
  uint16_t A[NSTAGE][TM][TK];   // x rows (tokens), k-contiguous, 16-byte chunks swizzled
  uint16_t B[NSTAGE][TN][TK];   // weight rows, likewise
};
// the 16-byte chunk of row r that holds k = 8c .. 8c+7
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 3); }

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

  // global -> LDS: the lanes of a wave fill 1 KiB of consecutive LDS (16 rows
  // of 64 bytes); the lane at physical chunk p of row r loads the chunk
  // swz(r, p) of that row.  Rows past the end load a valid row whose results
  // are never stored.
  const uint16_t* asrc[2];
  const uint16_t* bsrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = tid + NT * j;          // LDS chunk: row c / 4, physical chunk c % 4
    const int row = c >> 2, lc = swz(row, c & 3);
    const int64_t m = m0 + row;
    asrc[j] = x + (m < M ? m : 0) * hidden + 8 * lc;   // rows past the end read row 0
    int64_t wr = 0;
    if (!eta_tile)
      wr = int64_t(h) * R + TN * pair + row;
    else if (e0 + row < H)
      wr = int64_t(e0 + row) * R + 4 * D;
    bsrc[j] = w + wr * hidden + 8 * lc;
  }
  auto issue = [&](int stage, int k0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // the wave's 1 KiB block of this load: chunks (tid - lane) + NT j onward
      const int cb = (tid - lane) + NT * j;
      __builtin_amdgcn_global_load_lds(asrc[j] + k0, &sm.A[stage][cb >> 2][0], 16, 0, 0);
      __builtin_amdgcn_global_load_lds(bsrc[j] + k0, &sm.B[stage][cb >> 2][0], 16, 0, 0);
    }
  };

  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  const int nk = hidden / TK;
  issue(0, 0);
  if (nk > 1) issue(1, TK);
  for (int ks = 0; ks < nk; ++ks) {
    const int st = ks % NSTAGE;
    // this thread's loads of step ks are done (the 4 of step ks+1 may still run)
    if (ks + 1 < nk)
      __builtin_amdgcn_s_waitcnt(0x0074);   // vmcnt(4), lgkmcnt(0)
    else
      __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0), lgkmcnt(0)
    // everyone's loads of step ks landed; everyone is done reading step ks-1.
    // A bare barrier (the waits above are explicit): a fence would wait for
    // the loads of step ks+1 as well.  The empty asm statements keep the
    // compiler from moving memory accesses across it.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (ks + 2 < nk) issue((ks + 2) % NSTAGE, (ks + 2) * TK);
    bf16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm + 16 * i + l16;
      a[i] = *reinterpret_cast<const bf16x8*>(&sm.A[st][r][8 * swz(r, G)]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wn + 16 * j + l16;
      b[j] = *reinterpret_cast<const bf16x8*>(&sm.B[st][r][8 * swz(r, G)]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
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

// workgroups of a launch: 8 XCDs x the weight tiles of the busiest XCD x the token tiles
static int64_t proj_grid(int64_t B, int64_t T, int64_t H) {
  const int64_t ntn = 2 * H + (H + TN - 1) / TN;
  const int64_t mtiles = (B * T + TM - 1) / TM;
  return NXCD * ((ntn + NXCD - 1) / NXCD) * mtiles;
}

bool proj_mfma_grid_fits(int64_t B, int64_t T, int64_t H) {
  return B <= INT32_MAX && T <= INT32_MAX && H <= INT32_MAX / 4 &&
         proj_grid(B, T, H) <= INT32_MAX;
}

bool proj_mfma_supports(const ProjArgs& a) {
  return a.d == D && a.hidden % TK == 0 && proj_mfma_grid_fits(a.B, a.T, a.H);
}

hipError_t launch_proj_mfma(const ProjArgs& a, hipStream_t s) {
  if (!proj_mfma_supports(a)) return hipErrorNotSupported;
  const int64_t M = a.B * a.T;
  if (M == 0) return hipSuccess;
  const int ntn = static_cast<int>(2 * a.H + (a.H + TN - 1) / TN);
  const int64_t mtiles = (M + TM - 1) / TM;
  const int64_t grid = proj_grid(a.B, a.T, a.H);
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
