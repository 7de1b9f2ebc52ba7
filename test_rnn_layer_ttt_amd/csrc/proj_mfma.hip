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
// Tiles are 256 tokens x the 256 q, k, v, gate rows of one head, plus tiles
// of 256 tokens x the eta rows of up to 256 heads, which come last in the
// grid.  Eight waves (two per SIMD) each own 64 tokens x 128 weight rows
// (4 x 8 MFMA tiles).  K runs in steps of 32: operands go from global memory
// straight into LDS (global_load_lds, 16 bytes per lane, a wave filling 1 KiB
// of consecutive LDS) through a ring of three steps, so the loads of step
// ks+2 are in flight while step ks is computed.  Within a step each wave
// reads the next step's fragments from LDS between its MFMAs (b fragments
// double-buffered, each a fragment replaced once its row of MFMAs is
// issued).  In a 32-deep step lane group G holds k = 8G..8G+7 of its row for
// both operands, so every fragment is one 16-byte LDS read; LDS rows are 64
// bytes, their 16-byte chunks XOR-swizzled with the row so that the reads of
// neighbouring rows fall in different banks.  The weights are the MFMA's
// first operand, so a lane ends with four consecutive features of one token.
// bf16 results of a head tile go through LDS: each wave stages one output
// (64 tokens x 64 features) at a time and writes whole 128-byte token rows
// with 16-byte stores; fp32 results and eta tiles are stored directly (four
// features per lane in one 16-byte write, or single values).  Eta tiles run
// a plain K loop that issues the MFMAs of their real rows only.
#include "scan_common.h"

#include <cstdint>
#include <type_traits>

namespace ttt {
namespace {

constexpr int D = 64;
constexpr int R = 4 * D + 1;    // weight rows per head
constexpr int TM = 256;         // tokens per tile
constexpr int TN = 256;         // weight rows per tile: q, k, v, gate of a head, or eta of 256 heads
constexpr int TK = 32;          // k per step
constexpr int NSTAGE = 3;       // LDS ring of K steps
constexpr int NT = 512;         // threads: eight waves
constexpr int FI = 4;           // MFMA tiles per wave along tokens (64 tokens)
constexpr int FJ = 8;           // along weight rows (128 rows)
constexpr int ACH = TM * TK / 8 / NT;   // 16-byte chunks per thread and step: x
constexpr int BCH = TN * TK / 8 / NT;   // weights
constexpr int VM_STEP = ACH + BCH;      // global loads per thread and step
constexpr int ROWS_PER_CH = NT / 4;     // rows covered by one chunk index j
constexpr int64_t kMaxHidden = 65536;   // keeps the per-lane byte offsets in 32 bits
static_assert(TM == 4 * FI * 16 && TN == 2 * FJ * 16, "4 x 2 waves");
static_assert(VM_STEP < 16, "one vmcnt step");

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
__global__ void __launch_bounds__(NT, 1)
proj_mfma_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                 const float* __restrict__ bias, void* __restrict__ q, void* __restrict__ k,
                 void* __restrict__ v, void* __restrict__ gate, void* __restrict__ eta,
                 int64_t M, int64_t T, int hidden, int H, int ne, int64_t head_blocks) {
  __shared__ ProjSmem sm;
  // Blocks [0, head_blocks) are the (token tile, head) tiles.  Blocks are
  // dealt round-robin over the 8 XCDs (block b to XCD b % 8), and an XCD runs
  // one block per CU, about 32 at a time.  The tiles are listed in
  // supertiles of 4 token tiles x 8 heads (smaller at the ragged edges) and
  // XCD x takes one contiguous range of that list, so the blocks it runs
  // together share 4 x tiles and 8 heads' weights through its L2: each x
  // element is fetched about H/8 times chip-wide and each weight element
  // about (token tiles)/4 times, instead of 8 and H/2-ish times with the
  // tiles dealt one by one.  Any dealing still covers every tile once.
  // The eta tiles follow, (token tile, group of 256 heads).
  const bool eta_tile = int64_t(blockIdx.x) >= head_blocks;
  int64_t mt;
  int h = 0, e0 = 0;
  if (!eta_tile) {
    const int64_t b = blockIdx.x, n = head_blocks;
    const int64_t xcd = b % 8, j = b / 8;
    const int64_t wi = xcd * (n / 8) + min(xcd, n % 8) + j;   // position in the list
    const int64_t nmt = n / H;
    const int64_t ga = wi / (4 * int64_t(H));                  // token-tile group
    const int64_t r = wi - ga * 4 * H;
    const int na = static_cast<int>(min<int64_t>(4, nmt - 4 * ga));
    const int64_t gb = r / (8 * na);                            // head group
    const int r2 = static_cast<int>(r - gb * 8 * na);
    const int nb = static_cast<int>(min<int64_t>(8, H - 8 * gb));
    mt = 4 * ga + r2 / nb;
    h = static_cast<int>(8 * gb) + r2 % nb;
  } else {
    const int64_t e = int64_t(blockIdx.x) - head_blocks;
    mt = e / ne;
    e0 = static_cast<int>(e % ne) * TN;
  }
  const int64_t m0 = mt * TM;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int G = lane >> 4;

  // global -> LDS: chunk c = tid + NT j is physical chunk c % 4 of tile row
  // c / 4 and loads that row's chunk swz(row, c % 4).  Each source is a base
  // per chunk index j (rows ROWS_PER_CH j onward, scalar registers) plus a
  // 32-bit byte offset per lane.  Rows past the end load a valid row whose
  // results are never stored.
  const char* const abase = reinterpret_cast<const char*>(x + m0 * hidden);
  const char* bbase[BCH];
  uint32_t aoff[ACH], boff[BCH];
#pragma unroll
  for (int j = 0; j < ACH; ++j) {
    const int c = tid + NT * j;
    const int row = c >> 2, lc = swz(row, c & 3);
    aoff[j] = (m0 + row < M ? uint32_t(row) * hidden * 2 : 0u) + 16u * lc;
  }
#pragma unroll
  for (int j = 0; j < BCH; ++j) {
    const int c = tid + NT * j;
    const int row = c >> 2, lc = swz(row, c & 3);
    const int rel = row - ROWS_PER_CH * j;
    if (!eta_tile) {
      bbase[j] = reinterpret_cast<const char*>(w + (int64_t(h) * R + ROWS_PER_CH * j) * hidden);
      boff[j] = uint32_t(rel) * hidden * 2 + 16u * lc;
    } else {
      // eta row of head e0 + row: row (e0 + row) R + 4d of w_proj
      int jb = e0 + ROWS_PER_CH * j;
      if (jb >= H) jb = e0;
      bbase[j] = reinterpret_cast<const char*>(w + (int64_t(jb) * R + 4 * D) * hidden);
      boff[j] = (e0 + row < H ? uint32_t(e0 + row - jb) * uint32_t(R) * hidden * 2 : 0u) + 16u * lc;
    }
  }
  auto issue = [&](int stage, int k0) {
#pragma unroll
    for (int j = 0; j < ACH; ++j) {
      // the wave's 1 KiB block of this load: chunks (tid - lane) + NT j onward
      const int cb = (tid - lane) + NT * j;
      __builtin_amdgcn_global_load_lds(abase + 2 * k0 + aoff[j], &sm.A[stage][cb >> 2][0], 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < BCH; ++j) {
      const int cb = (tid - lane) + NT * j;
      __builtin_amdgcn_global_load_lds(bbase[j] + 2 * k0 + boff[j], &sm.B[stage][cb >> 2][0], 16, 0, 0);
    }
  };

  const int wm = (wave >> 1) * (FI * 16), wn = (wave & 1) * (FJ * 16);
  f32x4 acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  auto read_a = [&](int st, int i) {
    const int r = wm + 16 * i + l16;
    return *reinterpret_cast<const bf16x8*>(&sm.A[st][r][8 * swz(r, G)]);
  };
  auto read_b = [&](int st, int j) {
    const int r = wn + 16 * j + l16;
    return *reinterpret_cast<const bf16x8*>(&sm.B[st][r][8 * swz(r, G)]);
  };
  // A bare barrier (the waits are explicit): a fence would also wait for the
  // loads still in flight.  The empty asm statements keep the compiler from
  // moving memory accesses across it.
  auto bar = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  constexpr int kWaitStep = 0x0070 | VM_STEP;   // vmcnt(VM_STEP), lgkmcnt(0)
  constexpr int kWaitAll = 0x0070;              // vmcnt(0), lgkmcnt(0)

  const int nk = hidden / TK;
  bf16x8 a[FI];
  // One K step.  Its fragments are a and cb; the next step's b fragments go
  // into nb and its a fragments replace a[i] once row i's MFMAs are issued.
  // FULL: steps ks+1 .. ks+3 exist, so the step has no branches and the
  // compiler's own waits do not drain the reads of the next fragments.
  auto step = [&](auto full, int ks, bf16x8 (&cb)[FJ], bf16x8 (&nb)[FJ]) {
    constexpr bool FULL = decltype(full)::value;
    const bool more = FULL || ks + 1 < nk;
    if (more) {
      // this thread's loads of step ks+1 are done (those of ks+2 may run) and
      // its reads of step ks are done
      if (FULL || ks + 2 < nk)
        __builtin_amdgcn_s_waitcnt(kWaitStep);
      else
        __builtin_amdgcn_s_waitcnt(kWaitAll);
      // step ks+1 is in LDS for everyone, and everyone has read step ks, so
      // its stage takes step ks+3
      bar();
      if (FULL || ks + 3 < nk) issue(ks % NSTAGE, (ks + 3) * TK);
    }
    const int sn = (ks + 1) % NSTAGE;
    __builtin_amdgcn_sched_barrier(0);
    if (more) {
#pragma unroll
      for (int j = 0; j < FJ; ++j) nb[j] = read_b(sn, j);
    }
#pragma unroll
    for (int i = 0; i < FI; ++i) {
#pragma unroll
      for (int j = 0; j < FJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cb[j], a[i], acc[i][j], 0, 0, 0);
      if (more) a[i] = read_a(sn, i);
    }
    if constexpr (FULL) {
      // the b reads over the first 2 FJ MFMAs, then one a read per
      // FJ (FI - 2) / FI MFMAs (a[i] only after its row's MFMAs)
#pragma unroll
      for (int g = 0; g < FJ; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);     // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // LDS read
      }
#pragma unroll
      for (int g = 0; g < FI; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, FJ * (FI - 2) / FI, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  using full_t = std::integral_constant<bool, true>;
  using tail_t = std::integral_constant<bool, false>;
  if (eta_tile) {
    // eta tiles hold up to 256 heads' eta rows, mostly fewer: a plain K loop
    // on the same ring that issues the MFMAs of the real rows only (column
    // tiles j < nj of this wave)
    const int n_eta = H - e0 < TN ? H - e0 : TN;
    const int nj = max(0, min(FJ, (n_eta - wn + 15) / 16));
    issue(0, 0);
    if (nk > 1) issue(1, TK);
    for (int ks = 0; ks < nk; ++ks) {
      if (ks + 1 < nk)
        __builtin_amdgcn_s_waitcnt(kWaitStep);
      else
        __builtin_amdgcn_s_waitcnt(kWaitAll);
      bar();
      if (ks + 2 < nk) issue((ks + 2) % NSTAGE, (ks + 2) * TK);
      const int st = ks % NSTAGE;
      if (nj > 0) {
        bf16x8 af[FI];
#pragma unroll
        for (int i = 0; i < FI; ++i) af[i] = read_a(st, i);
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
          if (j < nj) {
            const bf16x8 bf = read_b(st, j);
#pragma unroll
            for (int i = 0; i < FI; ++i)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf, af[i], acc[i][j], 0, 0, 0);
          }
        }
      }
    }
  } else {
  bf16x8 b0[FJ], b1[FJ];
  issue(0, 0);
  if (nk > 1) issue(1, TK);
  if (nk > 1)
    __builtin_amdgcn_s_waitcnt(kWaitStep);
  else
    __builtin_amdgcn_s_waitcnt(kWaitAll);
  bar();
  if (nk > 2) issue(2, 2 * TK);
#pragma unroll
  for (int i = 0; i < FI; ++i) a[i] = read_a(0, i);
#pragma unroll
  for (int j = 0; j < FJ; ++j) b0[j] = read_b(0, j);
  int ks = 0;
  for (; ks + 4 < nk; ks += 2) {
    step(full_t{}, ks, b0, b1);
    step(full_t{}, ks + 1, b1, b0);
  }
  // the last one to four steps
  step(tail_t{}, ks, b0, b1);
  if (ks + 1 < nk) step(tail_t{}, ks + 1, b1, b0);
  if (ks + 2 < nk) step(tail_t{}, ks + 2, b0, b1);
  if (ks + 3 < nk) step(tail_t{}, ks + 3, b1, b0);
  }

  // epilogue: D[4G + r][l16] of MFMA tile (i, j) is token m0 + wm + 16i + l16,
  // weight row wn + 16j + 4G + r of the tile.
  if constexpr (OUT_BF16) {
    if (!eta_tile) {
      // bf16 q, k, v, gate: each wave stages one output (64 tokens x 64
      // features) at a time in its own LDS rows, then writes whole 128-byte
      // token rows with 16-byte stores (8 lanes per row, 8 rows per store)
      __syncthreads();   // every wave is done with the operand ring
      constexpr int SROW = 2 * D + 16;   // staged row: 64 bf16 + 16 bytes of padding
      char* const stage = reinterpret_cast<char*>(&sm) + wave * (FI * 16 * SROW);
      const int64_t mb = m0 + wm;        // this wave's first token
      const int64_t bb0 = mb / T, t0 = mb % T;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int kind = (wn >> 6) + p;   // 0 q, 1 k, 2 v, 3 gate
        uint16_t* const dst = static_cast<uint16_t*>(kind == 0 ? q : kind == 1 ? k : kind == 2 ? v : gate);
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int f0 = 16 * jj + 4 * G;
            float y[4] = {acc[i][4 * p + jj][0], acc[i][4 * p + jj][1], acc[i][4 * p + jj][2],
                          acc[i][4 * p + jj][3]};
            if (bias) {
#pragma unroll
              for (int r = 0; r < 4; ++r) y[r] += bias[int64_t(h) * R + 64 * kind + f0 + r];
            }
            uint2 pk;
            pk.x = uint32_t(to_bf16(y[0])) | (uint32_t(to_bf16(y[1])) << 16);
            pk.y = uint32_t(to_bf16(y[2])) | (uint32_t(to_bf16(y[3])) << 16);
            *reinterpret_cast<uint2*>(stage + (16 * i + l16) * SROW + 2 * f0) = pk;
          }
        // the same wave reads the rows back (its LDS accesses stay in order)
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const int row = (lane >> 3) + 8 * n, ch = lane & 7;
          const uint4 val = *reinterpret_cast<const uint4*>(stage + row * SROW + 16 * ch);
          if (mb + row >= M) continue;
          int64_t bb, t;
          if (T >= FI * 16) {   // at most one sequence boundary inside the wave's rows
            t = t0 + row;
            bb = bb0;
            if (t >= T) { t -= T; ++bb; }
          } else {
            bb = (mb + row) / T;
            t = (mb + row) % T;
          }
          *reinterpret_cast<uint4*>(dst + ((bb * H + h) * T + t) * D + 8 * ch) = val;
        }
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < FI; ++i) {
    const int64_t m = m0 + wm + 16 * i + l16;
    if (m >= M) continue;
    const int64_t bb = m / T, t = m % T;
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      const int col0 = wn + 16 * j + 4 * G;
      float y[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      if (!eta_tile) {
        if (bias) {
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] += bias[int64_t(h) * R + col0 + r];
        }
        // rows 0-63 q, 64-127 k, 128-191 v, 192-255 gate; one output per (wave, j)
        const int kind = (wn + 16 * j) >> 6;
        void* const dst = kind == 0 ? q : kind == 1 ? k : kind == 2 ? v : gate;
        const int64_t off = ((bb * H + h) * T + t) * D + (col0 & (D - 1));
        if constexpr (OUT_BF16) {
          uint2 pk;
          pk.x = uint32_t(to_bf16(y[0])) | (uint32_t(to_bf16(y[1])) << 16);
          pk.y = uint32_t(to_bf16(y[2])) | (uint32_t(to_bf16(y[3])) << 16);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(dst) + off) = pk;
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(dst) + off) = float4{y[0], y[1], y[2], y[3]};
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int hh = e0 + col0 + r;
          if (hh >= H) continue;
          float yy = y[r];
          if (bias) yy += bias[int64_t(hh) * R + 4 * D];
          const int64_t off = (bb * H + hh) * T + t;
          if constexpr (OUT_BF16)
            static_cast<uint16_t*>(eta)[off] = to_bf16(yy);
          else
            static_cast<float*>(eta)[off] = yy;
        }
      }
    }
  }
}

}  // namespace

// token tiles, and the blocks of a launch: one per (token tile, head), then
// one per (token tile, group of TN heads) for the eta rows
static int64_t proj_mtiles(int64_t B, int64_t T) { return (B * T + TM - 1) / TM; }
static int64_t proj_grid(int64_t B, int64_t T, int64_t H) {
  return proj_mtiles(B, T) * (H + (H + TN - 1) / TN);
}

bool proj_mfma_grid_fits(int64_t B, int64_t T, int64_t H) {
  return B <= INT32_MAX && T <= INT32_MAX && H <= INT32_MAX / 4 &&
         proj_grid(B, T, H) <= INT32_MAX;
}

bool proj_mfma_supports(const ProjArgs& a) {
  return a.d == D && a.hidden % TK == 0 && a.hidden <= kMaxHidden &&
         proj_mfma_grid_fits(a.B, a.T, a.H);
}

hipError_t launch_proj_mfma(const ProjArgs& a, hipStream_t s) {
  if (!proj_mfma_supports(a)) return hipErrorNotSupported;
  const int64_t M = a.B * a.T;
  if (M == 0) return hipSuccess;
  const int ne = static_cast<int>((a.H + TN - 1) / TN);
  const int64_t head_blocks = proj_mtiles(a.B, a.T) * a.H;
  const int64_t grid = proj_grid(a.B, a.T, a.H);
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* w = static_cast<const uint16_t*>(a.w);
  if (a.out_bf16)
    hipLaunchKernelGGL((proj_mfma_kernel<true>), dim3(static_cast<unsigned>(grid)), dim3(NT), 0, s,
                       x, w, a.bias, a.q, a.k, a.v, a.gate, a.eta, M, a.T,
                       static_cast<int>(a.hidden), static_cast<int>(a.H), ne, head_blocks);
  else
    hipLaunchKernelGGL((proj_mfma_kernel<false>), dim3(static_cast<unsigned>(grid)), dim3(NT), 0,
                       s, x, w, a.bias, a.q, a.k, a.v, a.gate, a.eta, M, a.T,
                       static_cast<int>(a.hidden), static_cast<int>(a.H), ne, head_blocks);
  return hipGetLastError();
}

}  // namespace ttt
