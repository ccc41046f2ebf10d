/*
 * lik.h -- C ABI of the MI355X (gfx950) fused MaxSim late-interaction scorer.
 *
 * What is computed (README "Late Interaction Kernels", section "What does it
 * compute?"):
 *
 *     score(q, d) = sum over valid query tokens i of
 *                   max over valid document tokens j of  Q[q,i,:] . D[d,j,:]
 *
 * with the rules of the README's "Scoring interface" section:
 *   - masks are bytes, nonzero = valid token; a NULL mask means every token
 *     is valid;
 *   - a query mask removes tokens from the sum, a document mask removes
 *     tokens from the max (a masked token never wins, whatever its value);
 *   - a document with no valid token scores exactly -1e9 for every query;
 *   - raw dot products, no normalisation inside; scores are float32.
 * The "Precision and compatibility" section fixes the input types: float16,
 * bfloat16 and float32, with float32 accumulation.
 *
 * The [Nq, Nd, Lq, Ld] similarity grid is never written to device memory
 * (social thread, post (4/N): stream document tiles through on-chip memory,
 * keep a running max in registers).  The backward is fused as well (post
 * (5/N)) and produces only the input gradients (colpali pull request,
 * section "Results").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.  Every pointer is a DEVICE pointer on the current HIP device.
 *   Tensors are dense, row-major, embedding dim innermost.  The caller owns
 *   all memory; the library never allocates or frees device memory, never
 *   synchronises, and keeps no pointer after returning.  Q, D, the outputs
 *   and the workspace must be 16-byte aligned.
 * Stream.  `stream` is a hipStream_t (NULL = the legacy default stream).
 *   All work is enqueued on it; results are valid once it has drained.
 * Workspace.  Scratch memory comes only from `workspace`, whose size must be
 *   at least lik_workspace_bytes(...) for the same operation and shapes.
 * Outputs.  Every output element is written, so outputs need no clearing.
 *   Gradients are float32 and OVERWRITTEN (not accumulated).
 * Argmax.  int32, the document-token index j that reached the max for each
 *   (pair, query token), ties to the lowest j; -1 for masked query tokens
 *   and for documents with no valid token.
 * Errors.  Arguments are checked on the host before any device work; on an
 *   error nothing is enqueued, no output is touched and a status is
 *   returned (lik_last_error() gives the detail, per host thread).
 *   LIK_ERR_INVALID_ARG   null required pointer, negative or overflowing
 *                         size, unknown dtype, misaligned pointer, workspace
 *                         too small;
 *   LIK_ERR_UNSUPPORTED   a valid request the library does not implement
 *                         (see lik_supported_dim; all-pairs with
 *                         Nd >= 2^23, Ld > 261120 or Nq * Lq > 2^30;
 *                         LIK_F32_BF16X3 where the all-pairs forward's
 *                         split copies, (Nq*Lq + Nd*Ld) * dim * 4 bytes,
 *                         exceed 1 GiB; no gfx950 device);
 *   LIK_ERR_HIP           a HIP launch error, reported as it happens.
 *   Zero-sized batches (Nq, Nd, B or N of 0) are a successful no-op.
 * Determinism.  For identical inputs and shapes the results are bitwise
 *   identical run to run: no floating-point atomics are used anywhere.
 * Reentrancy.  Calls may be made from several host threads; calls that share
 *   a workspace on overlapping streams race on it.
 */
#ifndef LIK_H_
#define LIK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: adds LIK_F32_BF16X3 (version 1 callers are unaffected). */
#define LIK_ABI_VERSION 2

/*
 * Input element types.  LIK_F16, LIK_BF16 and LIK_F32 are the input types of
 * the README's "Precision and compatibility" section, multiplied exactly
 * (every product of two inputs is exact) with float32 accumulation.
 *
 * LIK_F32_BF16X3 takes the same float32 inputs and buffers as LIK_F32 and
 * trades a bounded error for speed in the one place where float32 is slow:
 * the all-pairs forward at dim 64 and 128 (also when a backward recomputes
 * the argmax).  There every value x is split into two bfloat16 parts,
 * hi = bf16(x) and lo = bf16(x - hi) (rounded to nearest even), in copies of
 * Q and D kept in the workspace, and each product q*d is taken as
 * hi_q*hi_d + hi_q*lo_d + lo_q*hi_d on the bfloat16 matrix cores with float32
 * accumulation.  The dropped terms bound a similarity's error by about
 * 3 * 2^-16 * sum_k |q_k d_k| beyond float32 accumulation (4.6e-5 for unit
 * vectors); a score, a sum of Lq maxima, by Lq times that.  Values whose
 * bfloat16 rounding overflows become infinite.  Every other call with
 * LIK_F32_BF16X3 (pairwise and kd, dim 256, the gradient sums) computes
 * exactly as LIK_F32: those kernels are bound by memory, not multiplies.
 */
typedef enum { LIK_F16 = 0, LIK_BF16 = 1, LIK_F32 = 2, LIK_F32_BF16X3 = 3 } lik_dtype;

typedef enum {
  LIK_OK = 0,
  LIK_ERR_INVALID_ARG = 1,
  LIK_ERR_UNSUPPORTED = 2,
  LIK_ERR_HIP = 3
} lik_status;

/* Operation codes for lik_workspace_bytes. */
typedef enum {
  LIK_OP_FWD = 0,          /* all-pairs forward  */
  LIK_OP_BWD = 1,          /* all-pairs backward */
  LIK_OP_PAIRWISE_FWD = 2,
  LIK_OP_PAIRWISE_BWD = 3,
  LIK_OP_KD_FWD = 4,
  LIK_OP_KD_BWD = 5
} lik_op;

/* LIK_ABI_VERSION of the loaded library. */
int lik_abi_version(void);

/* Static description of a status code. */
const char* lik_status_string(lik_status s);

/* Detail of the last non-OK status returned on this host thread ("" if none). */
const char* lik_last_error(void);

/* 1 if the embedding dim `dim` has kernels in the library, else 0. */
int lik_supported_dim(int64_t dim);

/*
 * Profiling hook (not needed for scoring).  After this call, every forward
 * entry point called from the same host thread attaches `start_event` and
 * `stop_event` to the launch of its main scoring kernel (hipExtLaunchKernel:
 * they take the kernel's own start and end; the mask preparation and
 * split-merge kernels fall outside), so that the main kernel's duration can
 * be read with hipEventElapsedTime.
 * Both are hipEvent_t handles owned by the caller, created on the current
 * device; pass NULL, NULL to stop.  Returns LIK_ERR_INVALID_ARG when exactly
 * one of them is NULL.
 */
lik_status lik_set_profile_events(void* start_event, void* stop_event);

/*
 * Workspace bytes needed by one call.  Arguments mirror the entry point:
 *   all-pairs : nq_or_b = Nq, nd_or_n = Nd;
 *   pairwise  : nq_or_b = B,  nd_or_n = 1 (ignored);
 *   kd        : nq_or_b = B,  nd_or_n = N.
 * flags bit 0: forward -- the caller passes an argmax buffer;
 *              backward -- the caller passes the forward's argmax (if 0, the
 *              backward recomputes it into the workspace).
 * flags bit 1: a document mask will be passed.
 * flags bit 2: a query mask will be passed (all-pairs: only valid query
 *              tokens are scored, packed through a token list kept in the
 *              workspace).
 * A call whose masks or argmax differ from the flags the workspace was sized
 * with may need more bytes; it then returns LIK_ERR_INVALID_ARG.
 * Returns 0 for zero-sized problems; never fails (returns SIZE_MAX for sizes
 * that overflow).
 */
size_t lik_workspace_bytes(lik_op op, int64_t nq_or_b, int64_t lq,
                           int64_t nd_or_n, int64_t ld, int64_t dim,
                           lik_dtype dtype, int flags);

/*
 * Launch-plan introspection (not needed for scoring): one value of the plan
 * the library would use for a call with these shapes and flags (same
 * arguments as lik_workspace_bytes), so that tests can show they exercise
 * the same kernels and work split as a given workload.  `key` is a NUL-
 * terminated name:
 *   forward  "nb" (32-column MFMA blocks per wave), "upw" (document units per
 *            all-pairs workgroup), "n_groups", "n_sb" (query slot blocks),
 *            "nchunks" (pieces a document is split into), "tpc" (32-row
 *            tiles per piece), "compact" (query tokens compacted), "partial"
 *            (per-piece partials merged by a second kernel), "qpw" (whole
 *            queries per wave, 0 = flattened), "n_units" (pairwise/kd waves),
 *            "split" (1 when LIK_F32_BF16X3 scores through split rows);
 *   backward every forward key (the plan of the recomputing forward) and
 *            "gd_mode" (grad_D kernel: 0 workspace sort, 1 sorted in LDS
 *            per all-pairs document, 2 pairwise/kd streaming), "gd_parts",
 *            "gs_split", "gs_sw", "gs_lds", "gq_ap" (all-pairs grad_Q by
 *            document rounds), "gq_slices", "recompute", "sort_batch"
 *            (workspace sort: documents per batch, 0 when not used);
 *   both     "workspace" (the same as lik_workspace_bytes).
 * Returns -1 for an unknown key, a key of the other direction, or sizes
 * lik_workspace_bytes rejects.  Host only; no device is touched.
 */
int64_t lik_plan_value(lik_op op, int64_t nq_or_b, int64_t lq, int64_t nd_or_n,
                       int64_t ld, int64_t dim, lik_dtype dtype, int flags,
                       const char* key);

/*
 * All-pairs forward (README "Scoring interface", layer MaxSim):
 *   Q [Nq, Lq, dim] x D [Nd, Ld, dim] -> scores [Nq, Nd] float32.
 * q_mask [Nq, Lq] bytes or NULL; d_mask [Nd, Ld] bytes or NULL.
 * argmax [Nq, Nd, Lq] int32, or NULL to not keep it.
 */
lik_status lik_maxsim_fwd(const void* Q, const void* D, lik_dtype dtype,
                          int64_t Nq, int64_t Lq, int64_t Nd, int64_t Ld,
                          int64_t dim, const uint8_t* q_mask,
                          const uint8_t* d_mask, float* scores,
                          int32_t* argmax, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * All-pairs forward that allocates nothing, for callers that cannot allocate
 * device memory or size a workspace at call time: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, kernels and results as lik_maxsim_fwd (bitwise), but no
 * workspace: scratch comes from a fixed array the library holds on every
 * device it runs on (64 MiB per device, held until the process ends; its
 * address is resolved once per device, at the first call on that device).
 * A call whose scratch (lik_workspace_bytes(LIK_OP_FWD, ...) with the same
 * shapes and flags) exceeds 64 MiB returns LIK_ERR_UNSUPPORTED before any
 * device work.  Calls that overlap on one device (other streams, other host
 * threads) share that array and race: serialise them.  Nothing in the
 * scratch has to start at zero, and nothing is kept between calls.
 */
lik_status lik_maxsim_fwd_noalloc(const void* Q, const void* D, lik_dtype dtype,
                                  int64_t Nq, int64_t Lq, int64_t Nd, int64_t Ld,
                                  int64_t dim, const uint8_t* q_mask,
                                  const uint8_t* d_mask, float* scores,
                                  int32_t* argmax, void* stream);

/*
 * All-pairs backward: gradients of sum(grad_scores * scores).
 *   grad_Q[q,i,:] = sum over non-empty d of grad_scores[q,d] * D[d, a(q,d,i), :]
 *   grad_D[d,j,:] = sum over (q, valid i) with a(q,d,i) = j of
 *                   grad_scores[q,d] * Q[q,i,:]
 * (all other rows exactly 0).  grad_scores [Nq, Nd] float32.  argmax is the
 * forward's output for the same inputs, or NULL to recompute it.  grad_Q
 * [Nq, Lq, dim] and grad_D [Nd, Ld, dim] are float32; either may be NULL to
 * skip it.  grad_D's rows are each summed by one owner in a fixed order.
 */
lik_status lik_maxsim_bwd(const void* Q, const void* D, lik_dtype dtype,
                          int64_t Nq, int64_t Lq, int64_t Nd, int64_t Ld,
                          int64_t dim, const uint8_t* q_mask,
                          const uint8_t* d_mask, const float* grad_scores,
                          const int32_t* argmax, float* grad_Q, float* grad_D,
                          void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * Pairwise forward (README "Scoring interface", layer MaxSimPairwise):
 *   Q [B, Lq, dim] x D [B, Ld, dim] -> scores [B]; query b meets document b
 *   only.  q_mask [B, Lq], d_mask [B, Ld] or NULL; argmax [B, Lq] or NULL.
 */
lik_status lik_maxsim_pairwise_fwd(const void* Q, const void* D,
                                   lik_dtype dtype, int64_t B, int64_t Lq,
                                   int64_t Ld, int64_t dim,
                                   const uint8_t* q_mask,
                                   const uint8_t* d_mask, float* scores,
                                   int32_t* argmax, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Pairwise backward: grad_scores [B]; grad_Q [B, Lq, dim]; grad_D [B, Ld, dim]. */
lik_status lik_maxsim_pairwise_bwd(const void* Q, const void* D,
                                   lik_dtype dtype, int64_t B, int64_t Lq,
                                   int64_t Ld, int64_t dim,
                                   const uint8_t* q_mask,
                                   const uint8_t* d_mask,
                                   const float* grad_scores,
                                   const int32_t* argmax, float* grad_Q,
                                   float* grad_D, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * kd (per-query candidate) forward (colpali pull request, section "Design":
 * the [B, N, Ld, d] candidate layout of the negative-document losses):
 *   Q [B, Lq, dim] x D [B, N, Ld, dim] -> scores [B, N]; query b meets its
 *   own N candidates.  q_mask [B, Lq], d_mask [B, N, Ld] or NULL;
 *   argmax [B, N, Lq] or NULL.
 */
lik_status lik_maxsim_kd_fwd(const void* Q, const void* D, lik_dtype dtype,
                             int64_t B, int64_t Lq, int64_t N, int64_t Ld,
                             int64_t dim, const uint8_t* q_mask,
                             const uint8_t* d_mask, float* scores,
                             int32_t* argmax, void* workspace,
                             size_t workspace_bytes, void* stream);

/* kd backward: grad_scores [B, N]; grad_Q [B, Lq, dim]; grad_D [B, N, Ld, dim]. */
lik_status lik_maxsim_kd_bwd(const void* Q, const void* D, lik_dtype dtype,
                             int64_t B, int64_t Lq, int64_t N, int64_t Ld,
                             int64_t dim, const uint8_t* q_mask,
                             const uint8_t* d_mask, const float* grad_scores,
                             const int32_t* argmax, float* grad_Q,
                             float* grad_D, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Loss head: softmax cross-entropy over the rows of a score matrix.
 *
 * The colpali pull request ("What this PR adds") routes its in-batch ColBERT
 * loss and its negative-doc losses (over kd scores) through MaxSim, and its
 * "Results" benchmark this loss head together with the operator.  The pages
 * do not define the losses; the reading implemented is the row
 * cross-entropy with one target column t_r per row, mean over rows, logits
 * scaled by `scale`:
 *   row_loss[r] = logsumexp_c(scale*S[r,c]) - scale*S[r,t_r]
 *   *loss       = mean_r row_loss[r]
 *   grad[r,c]   = scale/R * (softmax_c(scale*S[r,:]) - [c == t_r])
 * In-batch loss: labels NULL (t_r = r, needs C >= R).  Negative-doc loss over
 * kd scores [B, N] with the positive as candidate 0: labels all 0.
 *
 * scores      [R, C] float32, row-major, device.
 * labels      [R] int32 target columns, device, or NULL for the diagonal.
 *             A label outside [0, C) makes that row's loss NaN (so the mean
 *             is NaN) and leaves the -1 term out of its gradient row.
 * scale       logit multiplier, finite and non-zero (1 = no temperature).
 * row_loss    [R] float32 output, device (also the reduction buffer).
 * loss        [1] float32 output, device: the mean, summed in a fixed order
 *             in float64, so bitwise reproducible.
 * grad_scores [R, C] float32 output (overwritten), or NULL to skip; it is the
 *             grad_scores input of the backward entry points.
 * R == 0 is a successful no-op.  Pointers 4-byte aligned.  Asynchronous on
 * `stream`; nothing is allocated.
 * ------------------------------------------------------------------------ */
lik_status lik_ce_rows(const float* scores, int64_t R, int64_t C,
                       const int32_t* labels, float scale, float* row_loss,
                       float* loss, float* grad_scores, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIK_H_ */
