// Internal declarations shared by the host dispatcher and the scan kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

enum LnMode : int { kLnST = 0, kLnExact = 1, kLnNone = 2 };

// One validated call, as the kernels see it.
struct ScanArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* eta_logit;
  const void* gate_logit;
  const float* W0;
  const float* gamma;  // nullptr with kLnNone
  const float* beta;   // nullptr with kLnNone
  float* out;
  float* W_final;      // nullptr: not written
  int64_t B, H, T, d;
  int ln;              // LnMode
  bool dual;
  int64_t chunk;       // tokens per chunk when dual
  bool in_bf16;
  float eps;
  // record of a forward pass for the backward (per-token modes, d = 64):
  // delta_t [B,H,T,d] and W at the start of every tile [B,H,ntiles,d,d];
  // nullptr: not recorded
  float* rec_delta = nullptr;
  float* rec_W = nullptr;
  // dual form: one SKIP (0) / UPDATE (nonzero) decision per chunk,
  // [B,H,ceil(T/chunk)]; a skipped chunk's tokens take eta = 0.  nullptr: all update
  const uint8_t* upd_mask = nullptr;
  // the :mlp variant: SiLU applied to q and k before the inner model
  bool silu_qk = false;
  // run the vector-ALU kernel even where the matrix-core one applies
  bool force_valu = false;
  // two-layer inner model W2 silu(W1 x): W0 / W_final above are W1's, these W2's
  const float* W2_0 = nullptr;
  float* W2_final = nullptr;   // nullptr: not written
};

// One validated backward call (d = 64, per-token modes).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* eta_logit;
  const void* gate_logit;
  const float* gamma;  // nullptr with kLnNone
  const float* beta;
  const float* dout;
  const float* dW_final;     // nullptr: zero
  const float* rec_delta;    // [B,H,T,d]
  const float* rec_W;        // [B,H,ntiles,d,d]
  float* gb_part;            // [B,H,2,d] caller workspace: per-scan dgamma, dbeta
  float* dq;
  float* dk;
  float* dv;
  float* deta_logit;
  float* dgate_logit;
  float* dW0;
  float* dgamma;       // nullptr with kLnNone
  float* dbeta;
  int64_t B, H, T, d;
  int ln;
  bool dual;
  int64_t chunk;       // the dual form's chunk (must be kRecTile); 1 otherwise
  bool in_bf16;
  float eps;
  bool silu_qk = false;   // the :mlp variant (SiLU on q and k)
};

// Tokens per tile of the recorded W (and of the backward's reverse walk).
constexpr int64_t kRecTile = 16;

// Per-token VALU scan: one workgroup per (b,h), W in VGPRs, 4 lanes per row.
// Handles every mode (including dual) for d in {16, 32, 64, 128}.
hipError_t launch_scan_valu(const ScanArgs& a, hipStream_t stream);

// Scan with the two-layer inner model on the vector ALUs: one workgroup per
// (b,h), every mode (per-token and dual), d in {16, 32, 64}.
hipError_t launch_mlp_valu(const ScanArgs& a, hipStream_t stream);

// Matrix-core dual-form chunk scan with the two-layer inner model (d = 64,
// chunk 16, bf16 inputs); hipErrorNotSupported for anything else.
hipError_t launch_mlp_mfma(const ScanArgs& a, hipStream_t stream);
bool mlp_mfma_supports(const ScanArgs& a);

// MFMA chunk scan for d = 64: exact per-token modes through the chunked
// (lookahead-corrected) form, and the dual form.  Returns hipErrorNotSupported
// for an argument combination it does not cover.
hipError_t launch_scan_mfma(const ScanArgs& a, hipStream_t stream);
bool scan_mfma_supports(const ScanArgs& a);

// The layer's input projections: x [B,T,hidden] bf16 times the stacked
// weights w [H,4d+1,hidden] bf16 (+ bias [H,4d+1] fp32), into q, k, v, gate
// [B,H,T,d] and eta [B,H,T], bf16 or fp32.
struct ProjArgs {
  const void* x;
  const void* w;
  const float* bias;   // nullptr: none
  void* q;
  void* k;
  void* v;
  void* eta;
  void* gate;
  int64_t B, T, hidden, H, d;
  bool out_bf16;
};
// MFMA projection kernel for d = 64 and hidden a multiple of 32; its grid of
// one workgroup per output tile must fit a launch (B*T tokens, H heads).
bool proj_mfma_supports(const ProjArgs& a);
bool proj_mfma_grid_fits(int64_t B, int64_t T, int64_t H);
hipError_t launch_proj_mfma(const ProjArgs& a, hipStream_t stream);

// Backward of the per-token scan, and of the dual form with chunks of
// kRecTile tokens, for d = 64 from a record; hipErrorNotSupported for
// anything else.
hipError_t launch_bwd_mfma(const BwdArgs& a, hipStream_t stream);

}  // namespace ttt
