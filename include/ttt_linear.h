/*
 * ttt_linear.h -- C ABI of the TTT-Linear fast-weight scan on gfx950 (MI355X).
 *
 * The operation ("Edifice.Recurrent.TTT", sections "Equations (TTT-Linear)",
 * "Architecture" and "Paper-Faithful Implementation"): for every
 * (batch b, head h) an inner weight W (d x d, fp32) starts at W0[b,h] and, for
 * t = 0 .. T-1,
 *
 *     eta_t   = sigmoid(eta_logit[b,h,t]) / d
 *     z_t     = P k_t                        (z_i = sum_j P[i][j] k_t[j])
 *     pred_t  = gamma[h] * (z_t - mean) / sqrt(var + 1e-6) + beta[h]
 *                                            (biased variance over the d entries)
 *     e_t     = pred_t - v_t
 *     delta_t = e_t                          (default: the page's grad_W = e_t k_t^T)
 *             | J_LN(z_t)^T e_t              (TTT_LN_EXACT: exact gradient of
 *                                             0.5*||LN(z)-v||^2, "Error Correction in
 *                                             Trained TTT Layers", abstract)
 *             | z_t - v_t                    (TTT_NO_LN: LayerNorm removed; the
 *                                             delta rule of linear attention)
 *     W       = W - eta_t * delta_t k_t^T
 *     out[b,h,t] = (W q_t) * sigmoid(gate_logit[b,h,t])   (updated W; elementwise gate)
 *
 * P is the current W (per-token mode) or, with TTT_DUAL, the weight at the
 * start of t's chunk of `chunk` tokens (the dual-form / mini-batch update of
 * "PonderTTT", "Technical Architecture", with the chunking of cortex_rust's
 * forward_chunkwise: a final chunk may be shorter).  W_final receives W after
 * the last token, so a scan can be resumed by passing it back as W0.
 *
 * Layout: every array is dense, row-major, C-contiguous, in device memory
 * (hipMalloc'd or equivalent):
 *     q, k, v, gate_logit   [B,H,T,d]  fp32, or bf16 when TTT_IN_BF16
 *     eta_logit             [B,H,T]    same element type as q
 *     W0, W_final           [B,H,d,d]  fp32
 *     gamma, beta           [H,d]      fp32 (unused, may be NULL, with TTT_NO_LN)
 *     out                   [B,H,T,d]  fp32
 *
 * Ownership: the caller owns every buffer.  The library allocates nothing,
 * keeps no pointer after returning and holds no mutable global state; calls
 * are reentrant.  Inputs are read-only and may alias one another (q == k is
 * fine).  `out` must not overlap any other argument.  W_final may be NULL (not
 * written), may equal W0 exactly (in-place state update), and must not
 * overlap anything else.
 *
 * Errors: every argument check below runs before any HIP call, so all of them
 * can be exercised on a host without a GPU.  The kernel is launched
 * asynchronously on `stream` (a hipStream_t; NULL = the default stream); a
 * device fault surfaces at the caller's next synchronisation.  No exception
 * crosses this boundary.
 */
#ifndef TTT_LINEAR_H_
#define TTT_LINEAR_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* mode bits */
#define TTT_DUAL      1u  /* chunk-start gradients (dual form); needs chunk >= 1 */
#define TTT_LN_EXACT  2u  /* LayerNorm Jacobian applied to the error */
#define TTT_IN_BF16   4u  /* q, k, v, eta_logit, gate_logit are bf16 */
#define TTT_NO_LN     8u  /* inner LayerNorm removed (delta rule); excludes TTT_LN_EXACT */
#define TTT_SILU_QK  16u  /* the :mlp variant of "Edifice.Recurrent.TTT" (Options,
                             :variant): SiLU on k and q before the inner model, so
                             z_t = P silu(k_t), the update uses silu(k_t) and
                             out = (W silu(q_t)) * sigmoid(gate); gradients are
                             with respect to the raw q and k.  On the bf16-input
                             matrix-core path silu(q), silu(k) are rounded to bf16 */
#define TTT_FORCE_VALU 32u /* run the vector-ALU per-token kernel even where the
                             matrix-core kernel applies (d = 64): the kernel the
                             scan's specification names for the per-token mode,
                             kept callable for comparison; same results within
                             rounding.  Given to the recording forward and the
                             backward, it selects their vector-ALU kernels too */

/* status codes */
#define TTT_OK               0
#define TTT_ERR_NULL         1  /* a required pointer is NULL */
#define TTT_ERR_SHAPE        2  /* B, H or d < 1, T < 0, or a size overflows */
#define TTT_ERR_MODE         3  /* unknown mode bit, EXACT|NO_LN, or DUAL with chunk < 1 */
#define TTT_ERR_UNSUPPORTED  4  /* d not in {16, 32, 64, 128}, or a misaligned pointer */
#define TTT_ERR_ALIAS        5  /* out overlaps an argument, or W_final partially overlaps */
#define TTT_ERR_HIP          6  /* the HIP runtime reported an error at launch */
#define TTT_ERR_WORKSPACE    7  /* record_bytes or workspace_bytes below the size query's value */

/*
 * Run the scan over all B*H (batch, head) pairs.
 *
 * d must be 16, 32, 64 or 128.  Pointers to the [.,d]- and [.,d,d]-shaped
 * arrays must be 16-byte aligned; eta_logit, gamma and beta need only their
 * element alignment.  `chunk` is read only when TTT_DUAL is set.  The
 * LayerNorm epsilon is fixed at 1e-6 (inside the square root).
 * T == 0 writes nothing to `out` and copies W0 to W_final (if distinct and
 * non-NULL); q, k, v, eta_logit, gate_logit and out may then be NULL.
 *
 * Returns TTT_OK or one of the TTT_ERR_* codes above.
 */
int32_t ttt_linear_forward(const void* q, const void* k, const void* v,
                           const void* eta_logit, const void* gate_logit,
                           const float* W0, const float* gamma, const float* beta,
                           float* out, float* W_final,
                           int64_t B, int64_t H, int64_t T, int64_t d,
                           uint32_t mode, int64_t chunk, void* stream);

/*
 * Run only the argument checks of ttt_linear_forward (same arguments, no
 * stream) and return the status it would return before launching.  Makes no
 * HIP call and touches no memory behind the pointers.
 */
int32_t ttt_linear_validate(const void* q, const void* k, const void* v,
                            const void* eta_logit, const void* gate_logit,
                            const float* W0, const float* gamma, const float* beta,
                            float* out, float* W_final,
                            int64_t B, int64_t H, int64_t T, int64_t d,
                            uint32_t mode, int64_t chunk);

/*
 * The kernel family a valid call with this d, mode and chunk launches:
 * "scan_mfma" (matrix-core chunk scan) or "scan_valu" (vector-ALU scan), or
 * "none" if the combination is not supported.  For profiling and reporting.
 */
const char* ttt_linear_kernel(int64_t d, uint32_t mode, int64_t chunk);

/*
 * The dual-form scan with one SKIP/UPDATE decision per chunk ("PonderTTT",
 * "Core Idea" and "Technical Architecture": instead of updating on every
 * chunk, learned SKIP/UPDATE decisions pick the chunks that update).
 * update_mask is [B,H,ceil(T/chunk)] uint8 in device memory: 0 = SKIP, any
 * other value = UPDATE.  A skipped chunk applies no update: its tokens take
 * eta = 0 (exactly what eta_logit = -inf gives), so W passes the chunk
 * unchanged and its outputs are (W_c q_t) * sigmoid(gate).  Every other
 * argument is as in ttt_linear_forward.  mode must include TTT_DUAL
 * (TTT_ERR_MODE otherwise); update_mask may be NULL only when T == 0 and must
 * not overlap out or W_final (TTT_ERR_ALIAS).  update_mask is read-only.
 */
int32_t ttt_linear_forward_masked(const void* q, const void* k, const void* v,
                                  const void* eta_logit, const void* gate_logit,
                                  const float* W0, const float* gamma, const float* beta,
                                  const uint8_t* update_mask, float* out, float* W_final,
                                  int64_t B, int64_t H, int64_t T, int64_t d,
                                  uint32_t mode, int64_t chunk, void* stream);

/*
 * ---- Training: a recording forward and the backward pass ----
 *
 * The backward gives the gradients of a scalar loss L with respect to every
 * input of the scan, from dL/dout and dL/dW_final: reverse-mode
 * differentiation through each step of the recurrence above (the models of
 * "Edifice.Recurrent.TTT" and "PonderTTT" train the layer end to end).  It
 * walks the sequence backwards in tiles of 16 tokens, from a record that the
 * forward leaves behind: delta_t for every token and the running W before
 * every 16th token (16 KiB per tile and (b,h) at d = 64; in the dual form this
 * W includes the updates of the chunk's tokens so far).
 *
 * Supported: every d and mode of ttt_linear_forward (d = 16, 32, 64, 128; the
 * per-token modes straight-through, TTT_LN_EXACT and TTT_NO_LN, and the dual
 * form with any chunk >= 1, where every z of a chunk is taken at the chunk's
 * first W, "PonderTTT", dual-form updates), fp32 or bf16 inputs, with or
 * without TTT_SILU_QK.  d = 64, per token or with chunk == 16, runs on the
 * matrix cores, the rest on the vector ALUs (ttt_linear_backward_kernel says
 * which); both record the same quantities, so a record of either forward
 * serves either backward.  A chunk that ttt_linear_forward_masked would skip
 * is trained by giving its tokens eta_logit = -inf in both calls: the step
 * size sigmoid(-inf) = 0 makes the forward identical, and its deta_logit is 0.
 *
 * The record is one caller-owned device buffer of ttt_linear_record_bytes()
 * bytes, 16-byte aligned; its contents are private to the library.  The
 * backward only reads it, so any number of backward calls may use one record,
 * also at the same time on different streams.  The backward's own scratch (the
 * per-(b,h) LayerNorm parameter gradients before their sum over the batch)
 * lives in a separate caller-owned workspace of
 * ttt_linear_backward_workspace_bytes() bytes.
 */

/*
 * The record size for these sizes and mode, in *bytes:
 * 4 * B*H * (T*d + ceil(T/16)*d*d), the same with or without TTT_DUAL.
 * Checks the shapes and mode as ttt_linear_forward_record does (the chunk of
 * the dual form is checked by the two calls that take it).  Makes no HIP call.
 */
int32_t ttt_linear_record_bytes(int64_t B, int64_t H, int64_t T, int64_t d, uint32_t mode,
                                int64_t* bytes);

/*
 * ttt_linear_forward (same arguments, same results: out and W_final are
 * identical to its, for the same mode) that also fills `record` for
 * ttt_linear_backward.
 * `record` is written, so it must not overlap any other argument.  T == 0
 * writes no record (its size is then 0 and it may be NULL) and copies W0 to
 * W_final as the forward does.
 */
int32_t ttt_linear_forward_record(const void* q, const void* k, const void* v,
                                  const void* eta_logit, const void* gate_logit,
                                  const float* W0, const float* gamma, const float* beta,
                                  float* out, float* W_final, void* record, int64_t record_bytes,
                                  int64_t B, int64_t H, int64_t T, int64_t d,
                                  uint32_t mode, int64_t chunk, void* stream);

/*
 * Gradients of L from dout = dL/dout [B,H,T,d] fp32 and dW_final = dL/dW_final
 * [B,H,d,d] fp32 (NULL: zero).  q, k, v, eta_logit, gate_logit, gamma, beta and
 * mode must be those of the recording forward, and `record` what it wrote.
 * Outputs, all fp32 whatever the input type:
 *     dq, dk, dv, dgate_logit   [B,H,T,d]
 *     deta_logit                [B,H,T]
 *     dW0                       [B,H,d,d]   may equal dW_final exactly (in place)
 *     dgamma, dbeta             [H,d]       summed over the batch and the tokens;
 *                                           unused, may be NULL, with TTT_NO_LN
 * Every output is overwritten, not accumulated into.  Outputs must not overlap
 * one another, the inputs, the record or the workspace (except dW0 ==
 * dW_final).  `workspace` is caller-owned device scratch of at least
 * ttt_linear_backward_workspace_bytes() bytes, 16-byte aligned (it may be NULL
 * when that size is 0); its contents on entry do not matter and on return are
 * unspecified, and two calls that overlap in time need two workspaces.  Pointer
 * alignment as in ttt_linear_forward; deta_logit, dgamma and dbeta need 4
 * bytes.  With T == 0 only dW0 (= dW_final, or zero), dgamma and dbeta (zero)
 * are written, and the per-token pointers may be NULL.  Runs asynchronously on
 * `stream`; dgamma and dbeta are reduced over the batch by a second kernel on
 * the same stream, in a fixed order, so repeated calls give identical bits.
 */
int32_t ttt_linear_backward(const void* q, const void* k, const void* v,
                            const void* eta_logit, const void* gate_logit,
                            const float* gamma, const float* beta,
                            const void* record, int64_t record_bytes,
                            void* workspace, int64_t workspace_bytes,
                            const float* dout, const float* dW_final,
                            float* dq, float* dk, float* dv, float* deta_logit,
                            float* dgate_logit, float* dW0, float* dgamma, float* dbeta,
                            int64_t B, int64_t H, int64_t T, int64_t d,
                            uint32_t mode, int64_t chunk, void* stream);

/*
 * The workspace size of ttt_linear_backward for these sizes and mode, in
 * *bytes: 4 * B*H * 2*d with the LayerNorm (per-(b,h) dgamma, dbeta before the
 * batch sum), 0 with TTT_NO_LN.  Checks the shapes and mode as
 * ttt_linear_record_bytes does.  Makes no HIP call.
 */
int32_t ttt_linear_backward_workspace_bytes(int64_t B, int64_t H, int64_t d, uint32_t mode,
                                            int64_t* bytes);

/*
 * Which kernel ttt_linear_backward runs for this d, mode and chunk:
 * "bwd_mfma" (matrix cores), "bwd_valu" (vector ALUs), or "none" when the
 * combination is rejected.  A static string; makes no HIP call.
 */
const char* ttt_linear_backward_kernel(int64_t d, uint32_t mode, int64_t chunk);

/*
 * ttt_linear_backward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and results, without the workspace.  The
 * scratch is instead a static device array inside the library, of
 * TTT_STATIC_SCRATCH_BYTES, that each GPU holds for the life of the process;
 * its device address is looked up once per device, on the first call made with
 * that device current.  Sizes whose workspace
 * (ttt_linear_backward_workspace_bytes) exceeds it return TTT_ERR_WORKSPACE
 * before any HIP call: at d = 64, B*H <= 4096.  The call allocates nothing.
 * Every call on one GPU shares that GPU's array, so calls that overlap in time
 * on one GPU (two streams, two threads) race and must be serialised by the
 * caller; sequential calls are safe (nothing in the array needs clearing
 * between calls).  Call it with the device of `stream` current.
 */
#define TTT_STATIC_SCRATCH_BYTES 2097152   /* 2 MiB */
int32_t ttt_linear_backward_noalloc(const void* q, const void* k, const void* v,
                                    const void* eta_logit, const void* gate_logit,
                                    const float* gamma, const float* beta,
                                    const void* record, int64_t record_bytes,
                                    const float* dout, const float* dW_final,
                                    float* dq, float* dk, float* dv, float* deta_logit,
                                    float* dgate_logit, float* dW0, float* dgamma, float* dbeta,
                                    int64_t B, int64_t H, int64_t T, int64_t d,
                                    uint32_t mode, int64_t chunk, void* stream);

/*
 * ---- The layer's input projections ----
 *
 * q_t = W_q x_t, k_t = W_k x_t, v_t = W_v x_t, and the learning-rate and gate
 * logits W_eta x_t, W_gate x_t of every head ("Edifice.Recurrent.TTT",
 * "Equations (TTT-Linear)" and "Architecture": the layer projects its input
 * to Q, K, V, eta and gate before the scan), in one launch that reads x once
 * and writes the five results in the layouts ttt_linear_forward reads.
 *
 *   x          [B,T,hidden]   bf16
 *   w_proj     [H,4d+1,hidden] bf16; the 4d+1 rows of head h are W_q (d rows),
 *                             W_k (d), W_v (d), W_gate (d), W_eta (1)
 *   b_proj     [H,4d+1] fp32, added to the products, or NULL (no bias, as the
 *                             pages write the projections)
 *   q, k, v, gate_logit [B,H,T,d] and eta_logit [B,H,T]: outputs, bf16 when
 *              mode has TTT_IN_BF16 (rounded to nearest even from the fp32
 *              sums), else fp32
 *
 * mode is the scan's mode word (only TTT_IN_BF16 is read here), so one mode
 * serves both calls.  Supported: d = 64, hidden a multiple of 32 and at most
 * 65536 (otherwise TTT_ERR_UNSUPPORTED).  x, w_proj and q, k, v, gate_logit 16-byte aligned,
 * eta_logit and b_proj element-aligned.  The outputs must not overlap one
 * another or the inputs.  T == 0 writes nothing.  Runs asynchronously on
 * `stream`; the accumulation order is fixed, so repeated calls give
 * identical bits.
 */
int32_t ttt_linear_project(const void* x, const void* w_proj, const float* b_proj,
                           void* q, void* k, void* v, void* eta_logit, void* gate_logit,
                           int64_t B, int64_t T, int64_t hidden, int64_t H, int64_t d,
                           uint32_t mode, void* stream);

/*
 * ---- TTT-MLP: the scan with a two-layer inner model ----
 *
 * The inner model of every (batch, head) is f(x) = W2 silu(W1 x), with W1 and
 * W2 both d x d fast weights and no biases ("Edifice.Recurrent.TTT", Options,
 * `:variant`: the `:mlp` variant makes the hidden state a two-layer MLP with
 * SiLU; "Error Correction in Trained TTT Layers", abstract: TTT-MLP is
 * trained under the same LayerNorm squared-error objective as TTT-Linear).
 * Per token t, with P1, P2 the weights the gradient is taken at (the current
 * ones, or the chunk-start ones with TTT_DUAL):
 *
 *   h = P1 k_t,  a = silu(h),  z = P2 a
 *   delta = LN(z) - v_t  (default),  J^T (LN(z) - v_t)  (TTT_LN_EXACT),
 *           z - v_t  (TTT_NO_LN)
 *   W1 -= (sigmoid(eta_logit_t)/d) ((P2^T delta) * silu'(h)) k_t^T
 *   W2 -= (sigmoid(eta_logit_t)/d) delta a^T
 *   out_t = (W2 silu(W1 q_t)) * sigmoid(gate_logit_t)      (updated weights)
 *
 * Arguments are those of ttt_linear_forward with W0 / W_final replaced by
 * the two weights:
 *   W1_0, W2_0           [B,H,d,d] fp32, row-major (h = W1 k, z = W2 a), read-only
 *   W1_final, W2_final   [B,H,d,d] fp32 outputs, each NULL = not written; each
 *                        may equal its own initial weight exactly (in place)
 * Modes: TTT_DUAL, TTT_LN_EXACT, TTT_NO_LN, TTT_IN_BF16, TTT_FORCE_VALU as for
 * the linear scan; TTT_SILU_QK (the other reading of `:mlp`) does not combine
 * with this call (TTT_ERR_UNSUPPORTED).  d must be 16, 32 or 64.  Every check
 * of ttt_linear_forward applies (W1 in the role of W), then: W2_0 non-NULL
 * (TTT_ERR_NULL), W2_0 / W2_final 16-byte aligned (TTT_ERR_UNSUPPORTED), and
 * no output overlapping another output or an input other than its own
 * initial weight (TTT_ERR_ALIAS).  T == 0 copies W1_0 and W2_0 to the finals.
 * Runs asynchronously on `stream`.
 */
int32_t ttt_mlp_forward(const void* q, const void* k, const void* v,
                        const void* eta_logit, const void* gate_logit,
                        const float* W1_0, const float* W2_0,
                        const float* gamma, const float* beta,
                        float* out, float* W1_final, float* W2_final,
                        int64_t B, int64_t H, int64_t T, int64_t d,
                        uint32_t mode, int64_t chunk, void* stream);

/* The argument checks of ttt_mlp_forward alone (no HIP call, no memory read). */
int32_t ttt_mlp_validate(const void* q, const void* k, const void* v,
                         const void* eta_logit, const void* gate_logit,
                         const float* W1_0, const float* W2_0,
                         const float* gamma, const float* beta,
                         float* out, float* W1_final, float* W2_final,
                         int64_t B, int64_t H, int64_t T, int64_t d,
                         uint32_t mode, int64_t chunk);

/* The kernel a valid ttt_mlp_forward call with this d, mode and chunk runs:
 * "mlp_mfma", "mlp_valu", or "none" if the combination is not supported. */
const char* ttt_mlp_kernel(int64_t d, uint32_t mode, int64_t chunk);

/* A static, human-readable description of a status code (never NULL). */
const char* ttt_status_string(int32_t status);

/* A static version string of the library (never NULL).  It ends with
 * "src=<16 hex digits>", a digest of the sources the library was built from,
 * so a caller can tell a stale build from a current one. */
const char* ttt_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TTT_LINEAR_H_ */
