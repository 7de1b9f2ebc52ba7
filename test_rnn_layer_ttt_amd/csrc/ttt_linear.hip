// C-ABI entry points of the TTT-Linear scan library: argument validation,
// alias checks, and dispatch to the gfx950 kernels.  Every check runs before
// the first HIP call, so the error paths are testable on a host without a GPU.
#include "ttt_linear.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "bwd_valu.h"
#include "scan_common.h"

namespace {

constexpr float kLnEps = 1e-6f;  // cortex_rust ttt.rs, TTT_NORM_EPS
constexpr uint32_t kKnownModes =
    TTT_DUAL | TTT_LN_EXACT | TTT_IN_BF16 | TTT_NO_LN | TTT_SILU_QK | TTT_FORCE_VALU;

// digest of the sources this library was built from (set by the build)
#ifndef TTT_SOURCE_DIGEST
#define TTT_SOURCE_DIGEST "unknown"
#endif

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range span(const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}

bool overlaps(const Range& a, const Range& b) {
  if (a.lo == 0 || b.lo == 0 || a.hi == a.lo || b.hi == b.lo) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, uintptr_t n) {
  return (reinterpret_cast<uintptr_t>(p) % n) == 0;
}

// a * b with overflow detection for non-negative operands
bool mul_ok(int64_t a, int64_t b, int64_t* r) {
  if (a != 0 && b > INT64_MAX / a) return false;
  *r = a * b;
  return true;
}

// Every argument check of ttt_linear_forward; fills *a on success.  Makes
// no HIP call.
int32_t validate(const void* q, const void* k, const void* v, const void* eta_logit,
                 const void* gate_logit, const float* W0, const float* gamma,
                 const float* beta, float* out, float* W_final, int64_t B, int64_t H,
                 int64_t T, int64_t d, uint32_t mode, int64_t chunk, ttt::ScanArgs* a) {
  // ---- mode ----
  if (mode & ~kKnownModes) return TTT_ERR_MODE;
  if ((mode & TTT_LN_EXACT) && (mode & TTT_NO_LN)) return TTT_ERR_MODE;
  const bool dual = (mode & TTT_DUAL) != 0;
  if (dual && chunk < 1) return TTT_ERR_MODE;
  const bool no_ln = (mode & TTT_NO_LN) != 0;
  const bool bf16 = (mode & TTT_IN_BF16) != 0;

  // ---- shapes ----
  if (B < 1 || H < 1 || d < 1 || T < 0) return TTT_ERR_SHAPE;
  int64_t BH, BHT, seq_elems, dd, w_elems;
  if (!mul_ok(B, H, &BH) || BH > INT32_MAX) return TTT_ERR_SHAPE;
  if (!mul_ok(BH, T, &BHT) || !mul_ok(BHT, d, &seq_elems)) return TTT_ERR_SHAPE;
  if (!mul_ok(d, d, &dd) || !mul_ok(BH, dd, &w_elems)) return TTT_ERR_SHAPE;
  if (w_elems > INT64_MAX / 4 || !mul_ok(H, d, &dd) || dd > INT64_MAX / 4) return TTT_ERR_SHAPE;
  if (seq_elems > INT64_MAX / 4) return TTT_ERR_SHAPE;

  // ---- pointers ----
  if (W0 == nullptr) return TTT_ERR_NULL;
  if (!no_ln && (gamma == nullptr || beta == nullptr)) return TTT_ERR_NULL;
  if (T > 0 && (q == nullptr || k == nullptr || v == nullptr || eta_logit == nullptr ||
                gate_logit == nullptr || out == nullptr))
    return TTT_ERR_NULL;

  // ---- supported sizes and alignment ----
  if (d != 16 && d != 32 && d != 64 && d != 128) return TTT_ERR_UNSUPPORTED;
  const int64_t in_size = bf16 ? 2 : 4;
  if (!aligned(W0, 16) || (W_final && !aligned(W_final, 16))) return TTT_ERR_UNSUPPORTED;
  if (!no_ln && (!aligned(gamma, 4) || !aligned(beta, 4))) return TTT_ERR_UNSUPPORTED;
  if (T > 0) {
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(gate_logit, 16) ||
        !aligned(out, 16) || !aligned(eta_logit, static_cast<uintptr_t>(in_size)))
      return TTT_ERR_UNSUPPORTED;
  }

  // ---- aliasing ----
  const Range r_out = span(out, T > 0 ? seq_elems * 4 : 0);
  const Range r_w0 = span(W0, w_elems * 4);
  const Range r_wf = span(W_final, W_final ? w_elems * 4 : 0);
  const Range inputs[] = {span(q, T > 0 ? seq_elems * in_size : 0),
                          span(k, T > 0 ? seq_elems * in_size : 0),
                          span(v, T > 0 ? seq_elems * in_size : 0),
                          span(gate_logit, T > 0 ? seq_elems * in_size : 0),
                          span(eta_logit, T > 0 ? BHT * in_size : 0),
                          span(gamma, no_ln ? 0 : H * d * 4),
                          span(beta, no_ln ? 0 : H * d * 4)};
  for (const Range& r : inputs) {
    if (overlaps(r_out, r) || overlaps(r_wf, r)) return TTT_ERR_ALIAS;
  }
  if (overlaps(r_out, r_w0) || overlaps(r_out, r_wf)) return TTT_ERR_ALIAS;
  if (W_final && W_final != W0 && overlaps(r_wf, r_w0)) return TTT_ERR_ALIAS;

  *a = ttt::ScanArgs{};
  a->q = q;
  a->k = k;
  a->v = v;
  a->eta_logit = eta_logit;
  a->gate_logit = gate_logit;
  a->W0 = W0;
  a->gamma = no_ln ? nullptr : gamma;
  a->beta = no_ln ? nullptr : beta;
  a->out = out;
  a->W_final = W_final;
  a->B = B;
  a->H = H;
  a->T = T;
  a->d = d;
  a->ln = no_ln ? ttt::kLnNone : ((mode & TTT_LN_EXACT) ? ttt::kLnExact : ttt::kLnST);
  a->dual = dual;
  a->chunk = dual ? chunk : 1;
  a->in_bf16 = bf16;
  a->eps = kLnEps;
  a->silu_qk = (mode & TTT_SILU_QK) != 0;
  a->force_valu = (mode & TTT_FORCE_VALU) != 0;
  return TTT_OK;
}

// the kernel a validated forward call runs
bool runs_mfma(const ttt::ScanArgs& a) { return !a.force_valu && ttt::scan_mfma_supports(a); }

// ---- the record of a forward pass for the backward ----
// layout, fp32: delta [B,H,T,d] | W at every tile start [B,H,ntiles,d,d]
struct RecordLayout {
  int64_t delta_off, w_off, bytes;
};

// Checks the mode and shapes of a recording forward or a backward and fills
// the layout.  Makes no HIP call.
int32_t record_layout(int64_t B, int64_t H, int64_t T, int64_t d, uint32_t mode,
                      RecordLayout* r) {
  if (mode & ~kKnownModes) return TTT_ERR_MODE;
  if ((mode & TTT_LN_EXACT) && (mode & TTT_NO_LN)) return TTT_ERR_MODE;
  if (B < 1 || H < 1 || d < 1 || T < 0) return TTT_ERR_SHAPE;
  if (d != 16 && d != 32 && d != 64 && d != 128) return TTT_ERR_UNSUPPORTED;
  const int64_t ntiles = (T + ttt::kRecTile - 1) / ttt::kRecTile;
  int64_t BH, per_scan, a, b;
  if (!mul_ok(B, H, &BH) || BH > INT32_MAX) return TTT_ERR_SHAPE;
  if (!mul_ok(T, d, &a) || !mul_ok(ntiles, d * d, &b) || a > INT64_MAX / 2 - b)
    return TTT_ERR_SHAPE;
  per_scan = a + b;
  int64_t elems;
  if (!mul_ok(BH, per_scan, &elems) || elems > INT64_MAX / 4) return TTT_ERR_SHAPE;
  r->delta_off = 0;
  r->w_off = BH * a * 4;
  r->bytes = elems * 4;
  return TTT_OK;
}

// the backward kernel of a validated call: the matrix-core one for d = 64, per
// token or with chunks of kRecTile tokens; the vector-ALU one otherwise
bool runs_bwd_mfma(int64_t d, uint32_t mode, int64_t chunk) {
  return d == 64 && !(mode & TTT_FORCE_VALU) && (!(mode & TTT_DUAL) || chunk == ttt::kRecTile);
}

hipError_t launch_backward(const ttt::BwdArgs& a, uint32_t mode, hipStream_t s) {
  return runs_bwd_mfma(a.d, mode, a.chunk) ? ttt::launch_bwd_mfma(a, s)
                                           : ttt::launch_bwd_valu(a, s);
}

// bytes of the backward's scratch: per-(b,h) dgamma, dbeta before the batch sum
int64_t backward_workspace(int64_t B, int64_t H, int64_t d, uint32_t mode) {
  return (mode & TTT_NO_LN) ? 0 : B * H * 2 * d * 4;
}

// the record's own checks, after the forward's
int32_t validate_record(const void* record, int64_t record_bytes, int64_t B, int64_t H,
                        int64_t T, int64_t d, uint32_t mode, RecordLayout* r) {
  const int32_t st = record_layout(B, H, T, d, mode, r);
  if (st != TTT_OK) return st;
  // an empty sequence has an empty record, which may be NULL
  if (T > 0 && record == nullptr) return TTT_ERR_NULL;
  if (!aligned(record, 16)) return TTT_ERR_UNSUPPORTED;
  if (record_bytes < r->bytes) return TTT_ERR_WORKSPACE;
  return TTT_OK;
}

int32_t validate_forward_record(const void* q, const void* k, const void* v,
                                const void* eta_logit, const void* gate_logit, const float* W0,
                                const float* gamma, const float* beta, float* out,
                                float* W_final, void* record, int64_t record_bytes, int64_t B,
                                int64_t H, int64_t T, int64_t d, uint32_t mode, int64_t chunk,
                                ttt::ScanArgs* a, RecordLayout* r) {
  int32_t st = validate(q, k, v, eta_logit, gate_logit, W0, gamma, beta, out, W_final, B, H, T,
                        d, mode, chunk, a);
  if (st != TTT_OK) return st;
  st = validate_record(record, record_bytes, B, H, T, d, mode, r);
  if (st != TTT_OK) return st;
  const int64_t in_size = (mode & TTT_IN_BF16) ? 2 : 4;
  const int64_t seq = B * H * T * d, w = B * H * d * d;
  const Range rec = span(record, r->bytes);
  const Range others[] = {span(q, T > 0 ? seq * in_size : 0),
                          span(k, T > 0 ? seq * in_size : 0),
                          span(v, T > 0 ? seq * in_size : 0),
                          span(gate_logit, T > 0 ? seq * in_size : 0),
                          span(eta_logit, T > 0 ? B * H * T * in_size : 0),
                          span(a->gamma, a->gamma ? H * d * 4 : 0),
                          span(a->beta, a->beta ? H * d * 4 : 0),
                          span(out, T > 0 ? seq * 4 : 0), span(W0, w * 4),
                          span(W_final, W_final ? w * 4 : 0)};
  for (const Range& o : others)
    if (overlaps(rec, o)) return TTT_ERR_ALIAS;
  char* base = static_cast<char*>(record);
  a->rec_delta = reinterpret_cast<float*>(base + r->delta_off);
  a->rec_W = reinterpret_cast<float*>(base + r->w_off);
  return TTT_OK;
}

int32_t validate_backward(const void* q, const void* k, const void* v, const void* eta_logit,
                          const void* gate_logit, const float* gamma, const float* beta,
                          const void* record, int64_t record_bytes, void* workspace,
                          int64_t workspace_bytes, const float* dout,
                          const float* dW_final, float* dq, float* dk, float* dv,
                          float* deta_logit, float* dgate_logit, float* dW0, float* dgamma,
                          float* dbeta, int64_t B, int64_t H, int64_t T, int64_t d,
                          uint32_t mode, int64_t chunk, ttt::BwdArgs* a,
                          bool internal_ws = false) {
  // internal_ws: the scratch is the library's static device array (its size
  // is workspace_bytes; the pointer is filled in later and overlaps nothing)
  // mode and shapes (the forward's rules, then the backward's coverage)
  if (mode & ~kKnownModes) return TTT_ERR_MODE;
  if ((mode & TTT_LN_EXACT) && (mode & TTT_NO_LN)) return TTT_ERR_MODE;
  if ((mode & TTT_DUAL) && chunk < 1) return TTT_ERR_MODE;
  RecordLayout r;
  int32_t st = record_layout(B, H, T, d, mode, &r);
  if (st != TTT_OK) return st;
  const bool dual = (mode & TTT_DUAL) != 0;
  const bool no_ln = (mode & TTT_NO_LN) != 0;
  const bool bf16 = (mode & TTT_IN_BF16) != 0;
  // pointers
  if ((T > 0 && record == nullptr) || dW0 == nullptr) return TTT_ERR_NULL;
  if (!no_ln && (gamma == nullptr || beta == nullptr || dgamma == nullptr || dbeta == nullptr))
    return TTT_ERR_NULL;
  if (T > 0 && (q == nullptr || k == nullptr || v == nullptr || eta_logit == nullptr ||
                gate_logit == nullptr || dout == nullptr || dq == nullptr || dk == nullptr ||
                dv == nullptr || deta_logit == nullptr || dgate_logit == nullptr))
    return TTT_ERR_NULL;
  // alignment
  const int64_t in_size = bf16 ? 2 : 4;
  if (!aligned(record, 16) || !aligned(dW0, 16) || (dW_final && !aligned(dW_final, 16)))
    return TTT_ERR_UNSUPPORTED;
  if (!no_ln && (!aligned(gamma, 4) || !aligned(beta, 4) || !aligned(dgamma, 4) ||
                 !aligned(dbeta, 4)))
    return TTT_ERR_UNSUPPORTED;
  if (T > 0) {
    const void* a16[] = {q, k, v, gate_logit, dout, dq, dk, dv, dgate_logit};
    for (const void* p : a16)
      if (!aligned(p, 16)) return TTT_ERR_UNSUPPORTED;
    if (!aligned(eta_logit, static_cast<uintptr_t>(in_size)) || !aligned(deta_logit, 4))
      return TTT_ERR_UNSUPPORTED;
  }
  const int64_t ws_bytes = backward_workspace(B, H, d, mode);
  if (internal_ws) workspace = nullptr;
  if (!internal_ws && ws_bytes > 0 && workspace == nullptr) return TTT_ERR_NULL;
  if (ws_bytes > 0 && !aligned(workspace, 16)) return TTT_ERR_UNSUPPORTED;
  if (record_bytes < r.bytes || workspace_bytes < ws_bytes) return TTT_ERR_WORKSPACE;
  // aliasing: outputs (and the workspace) against one another and every input
  const int64_t seq = B * H * T * d, w = B * H * d * d, hd = no_ln ? 0 : H * d * 4;
  const int64_t ts = T > 0 ? 1 : 0;
  const Range outs[] = {span(dq, ts * seq * 4),          span(dk, ts * seq * 4),
                        span(dv, ts * seq * 4),          span(dgate_logit, ts * seq * 4),
                        span(deta_logit, ts * B * H * T * 4), span(dW0, w * 4),
                        span(no_ln ? nullptr : dgamma, hd), span(no_ln ? nullptr : dbeta, hd),
                        span(ws_bytes > 0 ? workspace : nullptr, ws_bytes)};
  const Range ins[] = {span(q, ts * seq * in_size),      span(k, ts * seq * in_size),
                       span(v, ts * seq * in_size),      span(gate_logit, ts * seq * in_size),
                       span(eta_logit, ts * B * H * T * in_size), span(dout, ts * seq * 4),
                       span(no_ln ? nullptr : gamma, hd), span(no_ln ? nullptr : beta, hd),
                       span(record, r.bytes), span(dW_final, dW_final ? w * 4 : 0)};
  constexpr int kOuts = sizeof(outs) / sizeof(outs[0]);
  constexpr int kDW0 = 5;
  constexpr int kDWFinal = sizeof(ins) / sizeof(ins[0]) - 1;
  for (int i = 0; i < kOuts; ++i) {
    for (int j = i + 1; j < kOuts; ++j)
      if (overlaps(outs[i], outs[j])) return TTT_ERR_ALIAS;
    for (int j = 0; j < static_cast<int>(sizeof(ins) / sizeof(ins[0])); ++j) {
      if (i == kDW0 && j == kDWFinal && dW0 == dW_final) continue;   // in place
      if (overlaps(outs[i], ins[j])) return TTT_ERR_ALIAS;
    }
  }
  *a = ttt::BwdArgs{};
  const char* base = static_cast<const char*>(record);
  a->q = q;
  a->k = k;
  a->v = v;
  a->eta_logit = eta_logit;
  a->gate_logit = gate_logit;
  a->gamma = no_ln ? nullptr : gamma;
  a->beta = no_ln ? nullptr : beta;
  a->dout = dout;
  a->dW_final = dW_final;
  a->rec_delta = reinterpret_cast<const float*>(base + r.delta_off);
  a->rec_W = reinterpret_cast<const float*>(base + r.w_off);
  a->gb_part = ws_bytes > 0 ? static_cast<float*>(workspace) : nullptr;
  a->dq = dq;
  a->dk = dk;
  a->dv = dv;
  a->deta_logit = deta_logit;
  a->dgate_logit = dgate_logit;
  a->dW0 = dW0;
  a->dgamma = no_ln ? nullptr : dgamma;
  a->dbeta = no_ln ? nullptr : dbeta;
  a->B = B;
  a->H = H;
  a->T = T;
  a->d = d;
  a->ln = no_ln ? ttt::kLnNone : ((mode & TTT_LN_EXACT) ? ttt::kLnExact : ttt::kLnST);
  a->dual = dual;
  a->chunk = dual ? chunk : 1;
  a->in_bf16 = bf16;
  a->eps = kLnEps;
  a->silu_qk = (mode & TTT_SILU_QK) != 0;
  return TTT_OK;
}

// Every argument check of ttt_linear_project; fills *a.  Makes no HIP call.
int32_t validate_project(const void* x, const void* w_proj, const float* b_proj, void* q,
                         void* k, void* v, void* eta_logit, void* gate_logit, int64_t B,
                         int64_t T, int64_t hidden, int64_t H, int64_t d, uint32_t mode,
                         ttt::ProjArgs* a) {
  if (mode & ~kKnownModes) return TTT_ERR_MODE;
  if (B < 1 || H < 1 || d < 1 || hidden < 1 || T < 0) return TTT_ERR_SHAPE;
  int64_t BT, x_elems, per_head, rows, w_elems, BH, BHT, out_elems;
  if (!mul_ok(B, T, &BT) || !mul_ok(BT, hidden, &x_elems) || x_elems > INT64_MAX / 2)
    return TTT_ERR_SHAPE;
  // weight rows: 4d + 1 per head (q, k, v, gate, eta)
  if (!mul_ok(d, 4, &per_head) || !mul_ok(H, per_head + 1, &rows) ||
      !mul_ok(rows, hidden, &w_elems) || w_elems > INT64_MAX / 2)
    return TTT_ERR_SHAPE;
  if (!mul_ok(B, H, &BH) || !mul_ok(BH, T, &BHT) || !mul_ok(BHT, d, &out_elems) ||
      out_elems > INT64_MAX / 4 || hidden > INT32_MAX || H > INT32_MAX / 2)
    return TTT_ERR_SHAPE;
  // d = 64, hidden a multiple of 32 and at most 65536, a grid that fits a launch
  const bool bf16 = (mode & TTT_IN_BF16) != 0;
  const ttt::ProjArgs pa{x, w_proj, b_proj, q, k, v, eta_logit, gate_logit,
                         B, T, hidden, H, d, bf16};
  if (!ttt::proj_mfma_supports(pa)) return TTT_ERR_UNSUPPORTED;
  if (T > 0 && (x == nullptr || w_proj == nullptr || q == nullptr || k == nullptr ||
                v == nullptr || eta_logit == nullptr || gate_logit == nullptr))
    return TTT_ERR_NULL;
  const int64_t osz = bf16 ? 2 : 4;
  if (T > 0) {
    if (!aligned(x, 16) || !aligned(w_proj, 16) || (b_proj && !aligned(b_proj, 4)))
      return TTT_ERR_UNSUPPORTED;
    const void* outs16[] = {q, k, v, gate_logit};
    for (const void* p : outs16)
      if (!aligned(p, 16)) return TTT_ERR_UNSUPPORTED;
    if (!aligned(eta_logit, static_cast<uintptr_t>(osz))) return TTT_ERR_UNSUPPORTED;
    const Range outs[] = {span(q, out_elems * osz), span(k, out_elems * osz),
                          span(v, out_elems * osz), span(gate_logit, out_elems * osz),
                          span(eta_logit, BHT * osz)};
    const Range ins[] = {span(x, x_elems * 2), span(w_proj, w_elems * 2),
                         span(b_proj, b_proj ? rows * 4 : 0)};
    constexpr int kOuts = sizeof(outs) / sizeof(outs[0]);
    for (int i = 0; i < kOuts; ++i) {
      for (int j = i + 1; j < kOuts; ++j)
        if (overlaps(outs[i], outs[j])) return TTT_ERR_ALIAS;
      for (const Range& r : ins)
        if (overlaps(outs[i], r)) return TTT_ERR_ALIAS;
    }
  }
  *a = pa;
  return TTT_OK;
}

// Every argument check of ttt_mlp_forward; fills *a.  Makes no HIP call.
int32_t validate_mlp(const void* q, const void* k, const void* v, const void* eta_logit,
                     const void* gate_logit, const float* W1_0, const float* W2_0,
                     const float* gamma, const float* beta, float* out, float* W1_final,
                     float* W2_final, int64_t B, int64_t H, int64_t T, int64_t d, uint32_t mode,
                     int64_t chunk, ttt::ScanArgs* a) {
  // the linear scan's checks with W1 in the role of W
  int32_t st = validate(q, k, v, eta_logit, gate_logit, W1_0, gamma, beta, out, W1_final, B, H,
                        T, d, mode, chunk, a);
  if (st != TTT_OK) return st;
  if (W2_0 == nullptr) return TTT_ERR_NULL;
  if (d > 64 || a->silu_qk) return TTT_ERR_UNSUPPORTED;
  if (!aligned(W2_0, 16) || (W2_final && !aligned(W2_final, 16))) return TTT_ERR_UNSUPPORTED;
  const bool bf16 = a->in_bf16;
  const int64_t in_size = bf16 ? 2 : 4;
  const int64_t seq = B * H * T * d, w = B * H * d * d, hd = a->gamma ? H * d * 4 : 0;
  const int64_t ts = T > 0 ? 1 : 0;
  const Range r_w2 = span(W2_0, w * 4);
  const Range r_w2f = span(W2_final, W2_final ? w * 4 : 0);
  const Range r_w1 = span(W1_0, w * 4);
  const Range r_w1f = span(W1_final, W1_final ? w * 4 : 0);
  const Range r_out = span(out, ts * seq * 4);
  const Range ins[] = {span(q, ts * seq * in_size),        span(k, ts * seq * in_size),
                       span(v, ts * seq * in_size),        span(gate_logit, ts * seq * in_size),
                       span(eta_logit, ts * B * H * T * in_size), span(a->gamma, hd),
                       span(a->beta, hd),                  r_w1};
  for (const Range& r : ins)
    if (overlaps(r_w2f, r)) return TTT_ERR_ALIAS;
  if (overlaps(r_w2f, r_out) || overlaps(r_w2f, r_w1f)) return TTT_ERR_ALIAS;
  if (overlaps(r_w2, r_out) || overlaps(r_w2, r_w1f)) return TTT_ERR_ALIAS;
  if (W2_final && W2_final != W2_0 && overlaps(r_w2f, r_w2)) return TTT_ERR_ALIAS;
  a->W2_0 = W2_0;
  a->W2_final = W2_final;
  return TTT_OK;
}

// the kernel a validated two-layer call runs
bool runs_mlp_mfma(const ttt::ScanArgs& a) {
  return !a.force_valu && ttt::mlp_mfma_supports(a);
}

}  // namespace

extern "C" int32_t ttt_mlp_validate(const void* q, const void* k, const void* v,
                                    const void* eta_logit, const void* gate_logit,
                                    const float* W1_0, const float* W2_0, const float* gamma,
                                    const float* beta, float* out, float* W1_final,
                                    float* W2_final, int64_t B, int64_t H, int64_t T, int64_t d,
                                    uint32_t mode, int64_t chunk) {
  ttt::ScanArgs a;
  return validate_mlp(q, k, v, eta_logit, gate_logit, W1_0, W2_0, gamma, beta, out, W1_final,
                      W2_final, B, H, T, d, mode, chunk, &a);
}

extern "C" int32_t ttt_mlp_forward(const void* q, const void* k, const void* v,
                                   const void* eta_logit, const void* gate_logit,
                                   const float* W1_0, const float* W2_0, const float* gamma,
                                   const float* beta, float* out, float* W1_final,
                                   float* W2_final, int64_t B, int64_t H, int64_t T, int64_t d,
                                   uint32_t mode, int64_t chunk, void* stream) {
  ttt::ScanArgs a;
  const int32_t st = validate_mlp(q, k, v, eta_logit, gate_logit, W1_0, W2_0, gamma, beta, out,
                                  W1_final, W2_final, B, H, T, d, mode, chunk, &a);
  if (st != TTT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {
    const size_t bytes = static_cast<size_t>(B * H * d * d) * sizeof(float);
    if (W1_final && W1_final != W1_0 &&
        hipMemcpyAsync(W1_final, W1_0, bytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
      return TTT_ERR_HIP;
    if (W2_final && W2_final != W2_0 &&
        hipMemcpyAsync(W2_final, W2_0, bytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
      return TTT_ERR_HIP;
    return TTT_OK;
  }
  const hipError_t err = runs_mlp_mfma(a) ? ttt::launch_mlp_mfma(a, s) : ttt::launch_mlp_valu(a, s);
  return err == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

extern "C" const char* ttt_mlp_kernel(int64_t d, uint32_t mode, int64_t chunk) {
  alignas(16) static const float dummy[4] = {0, 0, 0, 0};
  const void* p = dummy;
  float* o = reinterpret_cast<float*>(0x100000);  // never dereferenced
  ttt::ScanArgs a;
  if (validate_mlp(p, p, p, p, p, dummy, dummy, dummy, dummy, o, nullptr, nullptr, 1, 1, 1, d,
                   mode, chunk, &a) != TTT_OK)
    return "none";
  return runs_mlp_mfma(a) ? "mlp_mfma" : "mlp_valu";
}

extern "C" int32_t ttt_linear_project(const void* x, const void* w_proj, const float* b_proj,
                                      void* q, void* k, void* v, void* eta_logit,
                                      void* gate_logit, int64_t B, int64_t T, int64_t hidden,
                                      int64_t H, int64_t d, uint32_t mode, void* stream) {
  ttt::ProjArgs a;
  const int32_t st = validate_project(x, w_proj, b_proj, q, k, v, eta_logit, gate_logit, B, T,
                                      hidden, H, d, mode, &a);
  if (st != TTT_OK) return st;
  if (T == 0) return TTT_OK;
  const hipError_t err = ttt::launch_proj_mfma(a, static_cast<hipStream_t>(stream));
  if (err == hipErrorNotSupported) return TTT_ERR_UNSUPPORTED;
  return err == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

extern "C" int32_t ttt_linear_validate(const void* q, const void* k, const void* v,
                                       const void* eta_logit, const void* gate_logit,
                                       const float* W0, const float* gamma, const float* beta,
                                       float* out, float* W_final, int64_t B, int64_t H,
                                       int64_t T, int64_t d, uint32_t mode, int64_t chunk) {
  ttt::ScanArgs a;
  return validate(q, k, v, eta_logit, gate_logit, W0, gamma, beta, out, W_final, B, H, T, d,
                  mode, chunk, &a);
}

extern "C" int32_t ttt_linear_forward(const void* q, const void* k, const void* v,
                                      const void* eta_logit, const void* gate_logit,
                                      const float* W0, const float* gamma, const float* beta,
                                      float* out, float* W_final, int64_t B, int64_t H,
                                      int64_t T, int64_t d, uint32_t mode, int64_t chunk,
                                      void* stream) {
  ttt::ScanArgs a;
  const int32_t st = validate(q, k, v, eta_logit, gate_logit, W0, gamma, beta, out, W_final,
                              B, H, T, d, mode, chunk, &a);
  if (st != TTT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {
    if (W_final && W_final != W0) {
      const size_t bytes = static_cast<size_t>(B * H * d * d) * sizeof(float);
      if (hipMemcpyAsync(W_final, W0, bytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
        return TTT_ERR_HIP;
    }
    return TTT_OK;
  }
  const hipError_t err = runs_mfma(a) ? ttt::launch_scan_mfma(a, s) : ttt::launch_scan_valu(a, s);
  return err == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

extern "C" int32_t ttt_linear_forward_masked(const void* q, const void* k, const void* v,
                                             const void* eta_logit, const void* gate_logit,
                                             const float* W0, const float* gamma,
                                             const float* beta, const uint8_t* update_mask,
                                             float* out, float* W_final, int64_t B, int64_t H,
                                             int64_t T, int64_t d, uint32_t mode, int64_t chunk,
                                             void* stream) {
  ttt::ScanArgs a;
  const int32_t st = validate(q, k, v, eta_logit, gate_logit, W0, gamma, beta, out, W_final,
                              B, H, T, d, mode, chunk, &a);
  if (st != TTT_OK) return st;
  if (!(mode & TTT_DUAL)) return TTT_ERR_MODE;
  if (T > 0 && update_mask == nullptr) return TTT_ERR_NULL;
  // validate() bounded B*H*T*d, so these products cannot overflow
  const int64_t mask_bytes = T > 0 ? B * H * ((T + chunk - 1) / chunk) : 0;
  const Range r_mask = span(update_mask, mask_bytes);
  if (overlaps(r_mask, span(out, T > 0 ? B * H * T * d * 4 : 0)) ||
      overlaps(r_mask, span(W_final, W_final ? B * H * d * d * 4 : 0)))
    return TTT_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {
    if (W_final && W_final != W0) {
      const size_t bytes = static_cast<size_t>(B * H * d * d) * sizeof(float);
      if (hipMemcpyAsync(W_final, W0, bytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
        return TTT_ERR_HIP;
    }
    return TTT_OK;
  }
  a.upd_mask = update_mask;
  const hipError_t err = runs_mfma(a) ? ttt::launch_scan_mfma(a, s) : ttt::launch_scan_valu(a, s);
  return err == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

extern "C" int32_t ttt_linear_record_bytes(int64_t B, int64_t H, int64_t T, int64_t d,
                                           uint32_t mode, int64_t* bytes) {
  if (bytes == nullptr) return TTT_ERR_NULL;
  RecordLayout r;
  const int32_t st = record_layout(B, H, T, d, mode, &r);
  if (st == TTT_OK) *bytes = r.bytes;
  return st;
}

// ---- the backward without a caller workspace ----
// Its scratch (the per-(b,h) dgamma, dbeta before their sum over the batch)
// is this static device array; every GPU the library runs on holds its own
// copy until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: the device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
constexpr int64_t kStaticScratchBytes = TTT_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kStaticScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The device address of the current device's scratch array.
hipError_t static_scratch(void** ptr) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  *ptr = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

extern "C" int32_t ttt_linear_backward_noalloc(
    const void* q, const void* k, const void* v, const void* eta_logit, const void* gate_logit,
    const float* gamma, const float* beta, const void* record, int64_t record_bytes,
    const float* dout, const float* dW_final, float* dq, float* dk, float* dv,
    float* deta_logit, float* dgate_logit, float* dW0, float* dgamma, float* dbeta, int64_t B,
    int64_t H, int64_t T, int64_t d, uint32_t mode, int64_t chunk, void* stream) {
  ttt::BwdArgs a;
  const int32_t st = validate_backward(q, k, v, eta_logit, gate_logit, gamma, beta, record,
                                       record_bytes, nullptr, kStaticScratchBytes, dout,
                                       dW_final, dq, dk, dv, deta_logit, dgate_logit, dW0,
                                       dgamma, dbeta, B, H, T, d, mode, chunk, &a,
                                       /*internal_ws=*/true);
  if (st != TTT_OK) return st;
  if (a.ln != ttt::kLnNone) {
    void* p = nullptr;
    if (static_scratch(&p) != hipSuccess || p == nullptr) return TTT_ERR_HIP;
    a.gb_part = static_cast<float*>(p);
  }
  const hipError_t err = launch_backward(a, mode, static_cast<hipStream_t>(stream));
  if (err == hipErrorNotSupported) return TTT_ERR_UNSUPPORTED;
  return err == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

extern "C" int32_t ttt_linear_backward_workspace_bytes(int64_t B, int64_t H, int64_t d,
                                                       uint32_t mode, int64_t* bytes) {
  if (bytes == nullptr) return TTT_ERR_NULL;
  RecordLayout r;
  const int32_t st = record_layout(B, H, 0, d, mode, &r);
  if (st == TTT_OK) *bytes = backward_workspace(B, H, d, mode);
  return st;
}

extern "C" int32_t ttt_linear_forward_record(const void* q, const void* k, const void* v,
                                             const void* eta_logit, const void* gate_logit,
                                             const float* W0, const float* gamma,
                                             const float* beta, float* out, float* W_final,
                                             void* record, int64_t record_bytes, int64_t B,
                                             int64_t H, int64_t T, int64_t d, uint32_t mode,
                                             int64_t chunk, void* stream) {
  ttt::ScanArgs a;
  RecordLayout r;
  const int32_t st = validate_forward_record(q, k, v, eta_logit, gate_logit, W0, gamma, beta,
                                             out, W_final, record, record_bytes, B, H, T, d,
                                             mode, chunk, &a, &r);
  if (st != TTT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) {
    if (W_final && W_final != W0) {
      const size_t bytes = static_cast<size_t>(B * H * d * d) * sizeof(float);
      if (hipMemcpyAsync(W_final, W0, bytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
        return TTT_ERR_HIP;
    }
    return TTT_OK;
  }
  // either kernel records the same quantities
  const hipError_t err = runs_mfma(a) ? ttt::launch_scan_mfma(a, s) : ttt::launch_scan_valu(a, s);
  return err == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

extern "C" int32_t ttt_linear_backward(const void* q, const void* k, const void* v,
                                       const void* eta_logit, const void* gate_logit,
                                       const float* gamma, const float* beta,
                                       const void* record, int64_t record_bytes,
                                       void* workspace, int64_t workspace_bytes,
                                       const float* dout,
                                       const float* dW_final, float* dq, float* dk, float* dv,
                                       float* deta_logit, float* dgate_logit, float* dW0,
                                       float* dgamma, float* dbeta, int64_t B, int64_t H,
                                       int64_t T, int64_t d, uint32_t mode, int64_t chunk,
                                       void* stream) {
  ttt::BwdArgs a;
  const int32_t st = validate_backward(q, k, v, eta_logit, gate_logit, gamma, beta, record,
                                       record_bytes, workspace, workspace_bytes, dout, dW_final,
                                       dq, dk, dv, deta_logit, dgate_logit, dW0, dgamma, dbeta,
                                       B, H, T, d, mode, chunk, &a);
  if (st != TTT_OK) return st;
  const hipError_t err = launch_backward(a, mode, static_cast<hipStream_t>(stream));
  if (err == hipErrorNotSupported) return TTT_ERR_UNSUPPORTED;
  return err == hipSuccess ? TTT_OK : TTT_ERR_HIP;
}

extern "C" const char* ttt_linear_backward_kernel(int64_t d, uint32_t mode, int64_t chunk) {
  RecordLayout r;
  if (record_layout(1, 1, 1, d, mode, &r) != TTT_OK || ((mode & TTT_DUAL) && chunk < 1))
    return "none";
  return runs_bwd_mfma(d, mode, chunk) ? "bwd_mfma" : "bwd_valu";
}

extern "C" const char* ttt_linear_kernel(int64_t d, uint32_t mode, int64_t chunk) {
  // a 16-byte aligned stand-in for every pointer: only the mode and sizes matter here
  alignas(16) static const float dummy[4] = {0, 0, 0, 0};
  const void* p = dummy;
  float* o = reinterpret_cast<float*>(0x100000);  // never dereferenced
  ttt::ScanArgs a;
  if (validate(p, p, p, p, p, dummy, dummy, dummy, o, nullptr, 1, 1, 1, d, mode, chunk, &a) !=
      TTT_OK)
    return "none";
  return runs_mfma(a) ? "scan_mfma" : "scan_valu";
}

extern "C" const char* ttt_status_string(int32_t status) {
  switch (status) {
    case TTT_OK: return "ok";
    case TTT_ERR_NULL: return "a required pointer is NULL";
    case TTT_ERR_SHAPE: return "invalid shape (B, H, d must be >= 1, T >= 0, sizes must not overflow)";
    case TTT_ERR_MODE: return "invalid mode (unknown bit, LN_EXACT with NO_LN, or DUAL with chunk < 1)";
    case TTT_ERR_UNSUPPORTED: return "unsupported (d must be 16, 32, 64 or 128; pointers must be aligned)";
    case TTT_ERR_ALIAS: return "out or W_final overlaps another argument";
    case TTT_ERR_HIP: return "HIP runtime error at launch";
    case TTT_ERR_WORKSPACE:
      return "record or workspace smaller than ttt_linear_record_bytes / "
             "ttt_linear_backward_workspace_bytes";
    default: return "unknown status";
  }
}

extern "C" const char* ttt_version(void) {
  return "ttt_linear 0.2.0 (gfx950) src=" TTT_SOURCE_DIGEST;
}
