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
};

// Per-token VALU scan: one workgroup per (b,h), W in VGPRs, 4 lanes per row.
// Handles every mode (including dual) for d in {16, 32, 64, 128}.
hipError_t launch_scan_valu(const ScanArgs& a, hipStream_t stream);

// MFMA chunk scan for d = 64: exact per-token modes through the chunked
// (lookahead-corrected) form, and the dual form.  Returns hipErrorNotSupported
// for an argument combination it does not cover.
hipError_t launch_scan_mfma(const ScanArgs& a, hipStream_t stream);
bool scan_mfma_supports(const ScanArgs& a);

}  // namespace ttt
