/*
 * adaflash.h -- C ABI of the MI355X (gfx950) verify-and-supervise library.
 *
 * One speculative-decoding round hands the verifier, per request b, the
 * target model's logits for the verified positions plus one extra row, the
 * drafter's logits and its sampled draft tokens, and the verify length the
 * adaptive length head predicted.  The library
 *   1. accepts draft x_i when u_i * q_i(x_i) < p_i(x_i) (acceptance
 *      probability min(1, p/q): AdaFlash review, "Speculative Decoding: The
 *      Basic Idea", step 3; DFlash reading notes, section 5.2, eq. 6), or, in
 *      greedy mode (T == 0), when x_i is the target argmax (DFlash reading
 *      notes, section 5.1);
 *   2. stops at the first rejection inside the request's verify length
 *      (AdaFlash review, step 4; adaptive length head, "Method Part 2");
 *   3. draws the correction token from norm(max(0, p - q)) at the rejected
 *      position, or a bonus token from the target row after the last verified
 *      position when every draft is accepted (DFlash reading notes, section
 *      5.2, eqs. 7-8, and Algorithm 1 step 9);
 *   4. optionally, in the same read of the logits, computes the on-policy
 *      distillation supervision of every verified row at temperature 1: the
 *      hard-label cross entropy on the target's top-1 token plus lambda times
 *      the entry-wise clipped reverse KL(q || p) (AdaFlash review, "The
 *      Reverse-KL + Hard-Label Mixture Loss, Derived" and "Entry-Wise
 *      Divergence Clipping, Derived", Algorithm 2), and its gradient with
 *      respect to the draft logits.
 *
 * Conventions shared by every entry point
 *  - All array arguments are DEVICE pointers owned by the caller; the library
 *    allocates nothing and keeps no state between calls (the measurement
 *    hook adaflash_timing_enable aside, which owns its HIP events; a
 *    workspace carries only its call counter from one call to the next).  Calls are enqueued
 *    on `stream` (a hipStream_t; NULL = the null stream) and return without
 *    synchronising.  Concurrent calls must use distinct workspaces.
 *  - Logits are row-major, contiguous; `dtype` selects fp32 or bf16 (raw
 *    16-bit patterns).  The fast path needs V to be a multiple of 8 (bf16) or
 *    4 (fp32) and 16-byte aligned base pointers; other shapes take a slower
 *    element-wise path.
 *  - Host-detectable argument errors return a negative status before anything
 *    is enqueued; nothing is written.  adaflash_last_error() then describes
 *    the error (thread-local string).
 *  - Data errors only the device can see are repaired and reported in
 *    *status_flags (see ADAFLASH_FLAG_*): verify lengths outside [1, k] are
 *    clamped (the packed-logits forms instead read nothing, see below),
 *    draft tokens outside [0, V) are clamped, non-finite row
 *    statistics are flagged.  Read the flags after synchronising the stream.
 *  - Sizes: 1 <= k <= 64, 1 <= V <= 2^20, 0 <= B and B * (k + 1) < 2^24.
 *    B == 0 is a valid empty call (row_offsets[0] is set to 0).
 *  - Logit value -inf means probability 0.  +inf and NaN logits are caller
 *    errors (flagged when they reach a row statistic; outputs undefined).
 */
#ifndef ADAFLASH_H
#define ADAFLASH_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define ADAFLASH_API __attribute__((visibility("default")))
#else
#define ADAFLASH_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ADAFLASH_OK = 0,
  ADAFLASH_E_INVALID = -1,     /* bad argument (NULL pointer, size, T, c, lambda) */
  ADAFLASH_E_WORKSPACE = -2,   /* workspace NULL or smaller than adaflash_workspace_bytes() */
  ADAFLASH_E_HIP = -3,         /* a HIP runtime call failed; see adaflash_last_error() */
  ADAFLASH_E_UNSUPPORTED = -4  /* valid but unsupported configuration */
} adaflash_status;

typedef enum { ADAFLASH_F32 = 0, ADAFLASH_BF16 = 1 } adaflash_dtype;

/* Bits OR-ed into *status_flags by the device. */
#define ADAFLASH_FLAG_BAD_VERIFY_LEN 1 /* some verify_len outside [1, k]; clamped */
#define ADAFLASH_FLAG_BAD_TOKEN 2      /* some draft token outside [0, V); clamped */
#define ADAFLASH_FLAG_NONFINITE 4      /* a row maximum was +inf/NaN or a row had no mass */
#define ADAFLASH_FLAG_SYNC_TIMEOUT 8   /* a cross-workgroup wait hit its bound; outputs invalid */

/* Library version, as major*10000 + minor*100 + patch. */
ADAFLASH_API int adaflash_version(void);

/* Bytes of device workspace either entry point needs for these sizes
 * (0 on invalid sizes).  The workspace needs no initialisation: its first
 * word is a call counter that each call advances on the device (any initial
 * value works), so that cross-workgroup records left by earlier calls are
 * never mistaken for the current call's. */
ADAFLASH_API size_t adaflash_workspace_bytes(int B, int k, int V);

/* Description of the last error returned on this thread ("" if none). */
ADAFLASH_API const char* adaflash_last_error(void);

/*
 * Measurement hook, for benchmarks; no part of the method.  While enabled on
 * the calling thread, every call of the verify / supervision / loss-variant
 * entry points launches its dominant kernel (the row kernel: the
 * supervision kernel, the statistics kernel of sampled verification, or the
 * greedy row kernel) with a pair of HIP events attached to that dispatch,
 * which take the kernel's own start and end times, for up to max_records
 * calls.  The events belong to the device current at
 * adaflash_timing_enable; time calls on that device only.
 * adaflash_timing_enable(0) disables the hook and
 * destroys the events.  adaflash_timing_read waits for the recorded events,
 * writes up to cap durations in milliseconds (call order) and starts a new
 * series; it returns the count written, or a negative adaflash_status.
 * adaflash_timing_every(n), n >= 1, attaches the events to every n-th call
 * only (the first one included; 1 = every call, the default, which
 * adaflash_timing_enable restores): attached events add a few microseconds
 * to a call, so a benchmark samples its calls.
 */
ADAFLASH_API int adaflash_timing_enable(int max_records);
ADAFLASH_API int adaflash_timing_read(float* ms, int cap);
ADAFLASH_API int adaflash_timing_every(int n);

/*
 * adaflash_verify -- speculative verification of a batch of B requests, with
 * optional fused supervision of the verified rows.
 *
 *   target_logits [B, k+1, V]  z_p.  Row i of request b is the target's
 *                              distribution for position i given the accepted
 *                              prefix x_0..x_{i-1}; row L_b is the bonus row.
 *   draft_logits  [B, k, V]    z_q, the proposal the drafter sampled from.
 *                              May be NULL only when T == 0 and no supervision
 *                              output is requested.
 *   draft_tokens  [B, k]       x_i in [0, V).
 *   verify_len    [B]          L_b in [1, k]: the verify length from the
 *                              adaptive length head (AdaFlash review,
 *                              Algorithm 3, k_hat = clamp(floor(gamma a k), 1, k)).
 *   uniforms      [B, k+1]     in [0, 1): uniforms[b][i] (i < k) drives accept
 *                              test i; uniforms[b][k] drives the single
 *                              correction-or-bonus draw.  Ignored when T == 0.
 *   T                          verification temperature; 0 = greedy.
 *   accept_len    [B]    out   A_b: drafts accepted before the first rejection.
 *   out_tokens    [B, k+1] out x_0..x_{A-1}, then the correction (A < L) or
 *                              bonus (A == L) token, then -1.
 *   margins       [B, k+1] out or NULL.  T > 0: margins[b][i] = p_i(x_i) -
 *                              u_i q_i(x_i) for i < L_b (every test is
 *                              evaluated); margins[b][k] = distance of the
 *                              draw's threshold to the nearest boundary of the
 *                              chosen token's CDF interval, divided by the
 *                              total mass.  NaN elsewhere and when T == 0.
 *   clip_c, lambda             supervision: clip threshold c > 0 and weight
 *                              lambda >= 0 (ignored when every supervision
 *                              output is NULL).
 *   row_offsets   [B+1]  out   exclusive prefix sum of the clamped verify
 *                              lengths: packed row n = row_offsets[b] + i
 *                              holds request b, position i < L_b.  Required.
 *   loss_ce       [N]    out or NULL  per-row hard-label cross entropy
 *                              -log q_i(x*_i), x*_i = argmax z_p (lowest index).
 *   loss_rkl      [N]    out or NULL  per-row clipped reverse KL
 *                              sum_v min(q log(q/p), c) at temperature 1.
 *   grad_draft    [N, V] out or NULL  d(ce + lambda * rkl)/d z_q per row, in the
 *                              logits' dtype (bf16 rounded to nearest even).
 *                              N = row_offsets[B]; N <= B*k, so a [B*k, V]
 *                              buffer always suffices.  Only N rows are written.
 *   status_flags  [1]    out or NULL  ADAFLASH_FLAG_* bits.
 *   workspace, workspace_bytes     device scratch, >= adaflash_workspace_bytes.
 *   stream                     hipStream_t.
 * Returns ADAFLASH_OK or a negative adaflash_status.
 */
ADAFLASH_API int adaflash_verify(adaflash_dtype dtype, const void* target_logits, const void* draft_logits,
                    const int32_t* draft_tokens, const int32_t* verify_len, const float* uniforms,
                    int B, int k, int V, float T, int32_t* accept_len, int32_t* out_tokens,
                    float* margins, float clip_c, float lambda, int32_t* row_offsets,
                    float* loss_ce, float* loss_rkl, void* grad_draft, int32_t* status_flags,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * adaflash_verify_noalloc -- adaflash_verify for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, outputs and errors as
 * adaflash_verify (padded logits layout), without the workspace: the call
 * uses a device array of the library, ADAFLASH_NOALLOC_WORKSPACE_BYTES per
 * GPU (every GPU the library runs on holds one until the process ends), whose
 * address is looked up on the first call on each device; it calls no
 * allocating routine.  Returns ADAFLASH_E_UNSUPPORTED, with nothing enqueued,
 * when adaflash_workspace_bytes(B, k, V) exceeds that size (at V = 151936 and
 * k = 16 up to about 460 requests fit).  Every call on one GPU shares the
 * array and initialises what it reads: calls that overlap on one GPU (other
 * streams or host threads) race, and the caller must order them.
 */
#define ADAFLASH_NOALLOC_WORKSPACE_BYTES ((size_t)16 << 20)
ADAFLASH_API int adaflash_verify_noalloc(adaflash_dtype dtype, const void* target_logits, const void* draft_logits,
                    const int32_t* draft_tokens, const int32_t* verify_len, const float* uniforms,
                    int B, int k, int V, float T, int32_t* accept_len, int32_t* out_tokens,
                    float* margins, float clip_c, float lambda, int32_t* row_offsets,
                    float* loss_ce, float* loss_rkl, void* grad_draft, int32_t* status_flags,
                    void* stream);

/*
 * adaflash_opd_loss_fwd_bwd -- supervision only (no verification) for the
 * verified rows of a replay batch (AdaFlash review, Algorithm 1 steps 4-6 and
 * Algorithm 2, at temperature 1).
 *
 *   target_logits [B, k+1, V]  z_p; row k of each request is not read.
 *   draft_logits  [B, k, V]    z_q.
 *   verify_len    [B] or NULL  rows i < L_b are supervised (NULL: L_b = k).
 *   clip_c > 0, lambda >= 0, and the outputs row_offsets (required),
 *   loss_ce, loss_rkl, grad_draft (each may be NULL), status_flags, workspace
 *   and stream exactly as in adaflash_verify.
 */
ADAFLASH_API int adaflash_opd_loss_fwd_bwd(adaflash_dtype dtype, const void* target_logits,
                              const void* draft_logits, const int32_t* verify_len, int B, int k,
                              int V, float clip_c, float lambda, int32_t* row_offsets,
                              float* loss_ce, float* loss_rkl, void* grad_draft,
                              int32_t* status_flags, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * Packed-logits forms of adaflash_verify and adaflash_opd_loss_fwd_bwd.
 *
 * AdaFlash review (ZH), section 2.3, and AdaFlash review (EN), "Adaptive
 * request scheduling for variable verification lengths": the target's verify
 * pass runs over only the real verify tokens of each request, sum_b k_hat_b
 * positions instead of B x k, so its logits arrive packed request after
 * request.  These entry points read them in place, with no scatter into the
 * padded [B, k+1, V] form:
 *
 *   target_logits [sum_b (L_b + 1), V]  request b's rows i = 0..L_b (the last
 *                              one is its bonus row) start at row
 *                              row_offsets[b] + b.  (For the supervision-only
 *                              form the bonus rows are present but not read.)
 *   draft_logits  [sum_b L_b, V]  request b's rows i = 0..L_b-1 start at row
 *                              row_offsets[b] -- the same order as the packed
 *                              supervision outputs.
 *
 * Every other argument, output and error is as in the padded form (draft
 * tokens, uniforms and margins stay [B, k] / [B, k+1]).  L_b must lie in
 * [1, k]: the packed rows are found through the lengths themselves, so when
 * one of them is outside that range (ADAFLASH_FLAG_BAD_VERIFY_LEN) no logits
 * row is read and the outputs other than row_offsets and status_flags are
 * left unwritten.  verify_len == NULL (supervision only) means L_b = k.
 * The workspace is the padded form's (adaflash_workspace_bytes).
 */
ADAFLASH_API int adaflash_verify_packed(adaflash_dtype dtype, const void* target_logits, const void* draft_logits,
                    const int32_t* draft_tokens, const int32_t* verify_len, const float* uniforms,
                    int B, int k, int V, float T, int32_t* accept_len, int32_t* out_tokens,
                    float* margins, float clip_c, float lambda, int32_t* row_offsets,
                    float* loss_ce, float* loss_rkl, void* grad_draft, int32_t* status_flags,
                    void* workspace, size_t workspace_bytes, void* stream);

ADAFLASH_API int adaflash_opd_loss_fwd_bwd_packed(adaflash_dtype dtype, const void* target_logits,
                              const void* draft_logits, const int32_t* verify_len, int B, int k,
                              int V, float clip_c, float lambda, int32_t* row_offsets,
                              float* loss_ce, float* loss_rkl, void* grad_draft,
                              int32_t* status_flags, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * Supervision loss variants the pages compare, on the same fused row pass as
 * adaflash_opd_loss_fwd_bwd (temperature 1; p = softmax(z_p), q = softmax(z_q),
 * x* = argmax z_p, lowest index on ties; CE = -log q(x*); R_c = sum_v
 * min(q log(q/p), c); FKL = sum_v p log(p/q)):
 *   ADAFLASH_LOSS_RKL       R_inf: plain reverse KL (AdaFlash review (EN),
 *                           ablation Table 2, first row)
 *   ADAFLASH_LOSS_RKL_CLIP  R_delta, p1 = delta > 0 (Table 2, second row;
 *                           "Entry-Wise Divergence Clipping, Derived")
 *   ADAFLASH_LOSS_MIXTURE   alpha CE + (1 - alpha) R_delta, p1 = alpha in
 *                           [0, 1], p2 = delta > 0 (Table 2, third row;
 *                           AdaFlash review (ZH) section 2.1: alpha = 0.8,
 *                           delta = 0.01)
 *   ADAFLASH_LOSS_FKL       FKL: forward KL, the OSD baseline's objective
 *                           (AdaFlash review (EN), "Forward KL vs. Reverse KL")
 *   ADAFLASH_LOSS_WCE       exp(-i / p1) CE for draft position i (DFlash
 *                           reading notes, section 7.3, eq. 12; p1 = 7 at
 *                           block size 16)
 */
typedef enum {
  ADAFLASH_LOSS_RKL = 1,
  ADAFLASH_LOSS_RKL_CLIP = 2,
  ADAFLASH_LOSS_MIXTURE = 3,
  ADAFLASH_LOSS_FKL = 4,
  ADAFLASH_LOSS_WCE = 5
} adaflash_loss_variant;

/*
 * adaflash_loss_variant_fwd_bwd -- one loss variant and its gradient with
 * respect to the draft logits for the verified rows (i < L_b) of a batch.
 *   target_logits, draft_logits, verify_len, B, k, V, row_offsets,
 *   status_flags, workspace, stream   as in adaflash_opd_loss_fwd_bwd.
 *   variant, p1, p2                   see adaflash_loss_variant.
 *   loss          [N]    out or NULL  the variant's per-row loss.
 *   grad_draft    [N, V] out or NULL  its gradient in the logits' dtype.
 * Returns ADAFLASH_OK or a negative adaflash_status.
 */
ADAFLASH_API int adaflash_loss_variant_fwd_bwd(adaflash_dtype dtype, const void* target_logits,
                                  const void* draft_logits, const int32_t* verify_len, int B, int k,
                                  int V, int variant, float p1, float p2, int32_t* row_offsets,
                                  float* loss, void* grad_draft, int32_t* status_flags, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Adaptive length head: the step before verification (it produces the verify
 * lengths) and after it (it learns from the accept lengths).  AdaFlash review
 * (ZH), section 2.2 "Adaptive Length Head", and AdaFlash review (EN),
 * Algorithm 3 and "Online Update of the Length Head, Derived":
 *   z[b,i]  = W1 h[b,i] + b1            per draft position i < k
 *   hbar[b] = (1/k) sum_i SiLU(z[b,i])  mean over the block
 *   a_hat[b] = sigmoid(w2 . hbar[b] + b2)   predicted accept rate
 *   k_hat[b] = clamp(floor(gamma a_hat[b] k), 1, k)
 *   loss[b] = (a_hat[b] - A_b / L_b)^2 with A_b accepted of the L_b verified
 *   drafts; the gradient reaches the head's parameters only (the hidden
 *   states are detached from the drafter).
 * Shapes: hidden [B, k, H] bf16 (row-major, 16-byte aligned, H a multiple of
 * 16, 16 <= H <= 65536), W1 [H', H] bf16 (16-byte aligned, 1 <= H' <= 8192),
 * b1 [H'] fp32, w2 [H'] fp32, b2 a float, 1 <= k <= 64, B*k < 2^24.  The two
 * dense products run on the matrix cores with fp32 accumulation.
 */

/* Bytes of device workspace the length-head entry points need (0 on invalid
 * sizes).  The workspace needs no initialisation. */
ADAFLASH_API size_t adaflash_length_head_workspace_bytes(int B, int k, int H, int Hp);

/*
 * adaflash_length_head_forward -- predicted accept rate and verify length.
 *   a_hat [B] fp32 out or NULL   sigmoid output (before gamma).
 *   k_hat [B] int32 out or NULL  clamp(floor(gamma a_hat k), 1, k), computed
 *                                in fp32 from a_hat; usable as verify_len.
 *   gamma > 0, finite            load scale (1 by default on the pages).
 * At least one of a_hat, k_hat must be non-NULL.  Returns ADAFLASH_OK or a
 * negative adaflash_status (nothing enqueued on error).
 */
ADAFLASH_API int adaflash_length_head_forward(const void* hidden, const void* W1, const float* b1,
                                 const float* w2, float b2, int B, int k, int H, int Hp, float gamma,
                                 float* a_hat, int32_t* k_hat, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * adaflash_length_head_backward -- loss and head gradients for one round.
 *   accept_len [B] int32   A_b from adaflash_verify (clamped to [0, L_b]).
 *   verify_len [B] int32   L_b, the verify length used (clamped to [1, k]).
 *   loss [B] fp32 out      (a_hat - A/L)^2 per request.
 *   dW1 [H', H], db1 [H'], dw2 [H'], db2 [1]  fp32 out: gradients of the SUM
 *                          of the losses over the batch (overwritten).
 * The forward pass is recomputed (same arithmetic as the forward entry
 * point).  Returns ADAFLASH_OK or a negative adaflash_status.
 */
ADAFLASH_API int adaflash_length_head_backward(const void* hidden, const void* W1, const float* b1,
                                  const float* w2, float b2, int B, int k, int H, int Hp,
                                  const int32_t* accept_len, const int32_t* verify_len, float* loss,
                                  float* dW1, float* db1, float* dw2, float* db2, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * The same two calls with the projection kept between them.  In a serving
 * round the forward runs before verification and the backward after it, on
 * the same hidden states and weights; the backward then needs the forward's
 * projection again.
 *   z1_cache [B k, H'] fp32   forward: out, the projection h W1^T (before
 *                             the bias); backward: in, that same array
 *                             (not recomputed).  Caller-owned device memory;
 *                             must not be NULL when B > 0.  The backward's
 *                             results equal those of
 *                             adaflash_length_head_backward only if z1_cache
 *                             holds the forward's output for the same hidden
 *                             states and W1.
 * Every other argument is as in the plain forms above.
 */
ADAFLASH_API int adaflash_length_head_forward_cached(const void* hidden, const void* W1, const float* b1,
                                 const float* w2, float b2, int B, int k, int H, int Hp, float gamma,
                                 float* a_hat, int32_t* k_hat, float* z1_cache, void* workspace,
                                 size_t workspace_bytes, void* stream);
ADAFLASH_API int adaflash_length_head_backward_cached(const void* hidden, const void* W1, const float* b1,
                                  const float* w2, float b2, int B, int k, int H, int Hp,
                                  const int32_t* accept_len, const int32_t* verify_len, float* loss,
                                  float* dW1, float* db1, float* dw2, float* db2, const float* z1_cache,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Verification-batch admission controller (host only; no GPU call).
 * AdaFlash review (ZH), section 2.3, and AdaFlash review (EN), "Adaptive
 * request scheduling for variable verification lengths": with per-request
 * verify lengths the verify batch is packed to sum_i k_hat_i tokens, so the
 * scheduler smooths the number of requests a round actually advanced,
 * N_hat <- (1 - beta) N_hat + beta N, admits up to that many next round, and
 * returns requests that still overflow the budget to the pending queue.
 * One round:
 *   n = adaflash_admission_propose(h, ids, cap)   running requests, then
 *       pending ones in arrival order until the batch holds
 *       max(1, floor(N_hat + 0.5)); the caller computes k_hat for them
 *       (adaflash_length_head_forward);
 *   m = adaflash_admission_commit(h, k_hat, n, ids)   while sum k_hat exceeds
 *       budget_tokens (and m > 1) the most recently placed request goes back
 *       to the front of the pending queue, order kept; N = m updates N_hat;
 *       ids[0..m) is the batch to verify;
 *   adaflash_admission_finish(h, done, nd)   after verification, drops the
 *       requests that completed.
 * Request ids are the caller's (int64); host pointers; the handle is not
 * thread-safe.  Functions return ADAFLASH_OK / a count, or ADAFLASH_E_INVALID
 * (nothing changed) on a NULL handle, a negative count, a too small `cap`, or
 * a k_hat count different from the proposed batch.
 */
ADAFLASH_API void* adaflash_admission_create(double beta, double n_hat0, int64_t budget_tokens);  /* NULL if
                                      beta not in (0, 1], n_hat0 < 0 or not finite, budget < 1 */
ADAFLASH_API void adaflash_admission_destroy(void* h);
ADAFLASH_API int adaflash_admission_enqueue(void* h, const int64_t* ids, int n);
ADAFLASH_API int adaflash_admission_propose(void* h, int64_t* out_ids, int cap);
ADAFLASH_API int adaflash_admission_commit(void* h, const int32_t* k_hat, int n, int64_t* out_ids);
ADAFLASH_API int adaflash_admission_finish(void* h, const int64_t* done_ids, int n);
ADAFLASH_API double adaflash_admission_estimate(const void* h);   /* N_hat (NaN for NULL) */
ADAFLASH_API int adaflash_admission_pending(const void* h);       /* pending queue length */

#ifdef __cplusplus
}
#endif

#endif /* ADAFLASH_H */
