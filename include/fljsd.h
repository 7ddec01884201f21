/*
 * fljsd.h - C ABI of the fused-linear generalized Jensen-Shannon distillation
 * pass for AMD Instinct MI355X (gfx950).
 *
 * The operation (Liger-Kernel PR #1352 "Fuse log-softmax into
 * fused_linear_jsd kernel", Summary and Details; PR #1429 "write the
 * weight-gradient product directly into grad_weight", Summary):
 *
 *   Z_s = X_s W_s^T,  Z_t = X_t W_t^T                 (lm_head products)
 *   Q = softmax(Z_s / T),  P = softmax(Z_t / T)        (student, teacher)
 *   JSD_beta = beta KL(P||M) + (1-beta) KL(Q||M),  M = beta P + (1-beta) Q
 *     beta == 0 is forward KL(P||Q), beta == 1 is reverse KL(Q||P)
 *     (PR #1352, Testing Done: the four beta branches)
 *   loss = scale * sum over rows and vocabulary of the per-element terms
 *   dZ_s = d loss / d Z_s  (log-softmax chain rule, 1/T factor, dX_sum term)
 *   grad_X_s = dZ_s W_s,   grad_W_s = dZ_s^T X_s
 *
 * Temperature divides both logits once; there is no T^2 factor (PR #1352,
 * Open question 2). Exact ties p == q contribute zero (PR #1374 "Fix TVD
 * gradient at p == q", Summary). The teacher receives no gradient.
 *
 * Conventions shared by every entry point:
 *  - All tensors are dense, row-major, in device memory, and 16-byte aligned.
 *  - Floating-point inputs and outputs use `dtype` (FLJSD_F32 or FLJSD_BF16);
 *    losses are always fp32. All logit-to-loss arithmetic is fp32; GEMMs
 *    accumulate in fp32 and round once to `dtype`.
 *  - The caller allocates and owns every buffer, including the workspace.
 *    The library never allocates device memory, never synchronizes, and
 *    enqueues work only on `stream` (a hipStream_t; NULL is the null stream).
 *    Calls return as soon as the work is enqueued.
 *  - Every argument is checked before anything is enqueued; on error the
 *    call returns a negative code and leaves every output untouched.
 *    fljsd_last_error() then describes the failure. NaN or Inf inside the
 *    data is not checked and propagates.
 *  - Calls on one stream are ordered. Concurrent calls on different streams
 *    are safe when their workspaces and outputs do not overlap.
 */
#ifndef FLJSD_H
#define FLJSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of inputs, logits, gradients and weights. */
typedef enum fljsd_dtype {
  FLJSD_F32 = 0,
  FLJSD_BF16 = 1
} fljsd_dtype;

/* Reduction of the per-element loss terms; `scale` is what multiplies both
 * the summed loss and the gradient. batchmean divides by the number of rows
 * (PR #1374's tie table: -0.0625 = -0.5 * 1/8 at 8 rows).
 *   BATCHMEAN: loss = sum / rows          scale = 1/rows
 *   SUM:       loss = sum                 scale = 1
 *   MEAN:      loss = sum / (rows * V)    scale = 1/(rows*V)
 *   NONE:      loss[r] = row r's sum      scale = 1 (gradient as for SUM) */
typedef enum fljsd_reduction {
  FLJSD_BATCHMEAN = 0,
  FLJSD_SUM = 1,
  FLJSD_MEAN = 2,
  FLJSD_NONE = 3
} fljsd_reduction;

/* Status codes. The pages give no error convention for this op; negative
 * C status codes checked before any work is enqueued are this library's
 * reading. */
#define FLJSD_OK 0
#define FLJSD_EINVAL (-1)      /* null required pointer, size <= 0, beta outside [0,1],
                                  temperature <= 0 or not finite, ld < V, num_chunks < 0 */
#define FLJSD_EDTYPE (-2)      /* dtype or reduction value not in the enums */
#define FLJSD_EWORKSPACE (-3)  /* workspace smaller than the plan needs */
#define FLJSD_EALIGN (-4)      /* pointer not 16-byte aligned, or H_s / H_t not a multiple
                                  of 8 elements (bf16) or 4 elements (fp32) */
#define FLJSD_EHIP (-5)        /* a HIP call or kernel launch failed */
#define FLJSD_EDEVICE (-6)     /* the current device is not a gfx950 GPU */

/*
 * fljsd_forward_backward - the whole fused-linear JSD pass, forward and
 * backward (PR #1352 Details; PR #1429 Summary).
 *
 * Inputs (read only):
 *   X_s [BT, H_s], W_s [V, H_s]   student hidden states and lm_head weight
 *   X_t [BT, H_t], W_t [V, H_t]   teacher hidden states and lm_head weight
 *   beta in [0, 1], temperature > 0, reduction (fljsd_reduction).
 *   num_chunks >= 1: rows are processed in chunks of C = ceil(BT/num_chunks)
 *     rows, exactly as asked (the last chunk may be shorter, and there may be
 *     fewer than num_chunks chunks). num_chunks == 0: the library picks the
 *     smallest count whose workspace fits in workspace_bytes
 *     (fljsd_plan_num_chunks). Results do not depend on the chunk count
 *     beyond rounding.
 * Outputs (every element written; may be uninitialized on entry):
 *   loss      fp32: 1 value, or BT values for FLJSD_NONE.
 *   grad_X_s  [BT, H_s] in dtype, or NULL to skip the grad_input product.
 *   grad_W_s  [V, H_s] in dtype, or NULL to skip the grad_weight product.
 *             The first chunk overwrites it; later chunks add to it with one
 *             fp32 add and one rounding per chunk (PR #1429 Summary).
 * Workspace: device scratch of at least
 *   fljsd_workspace_size(BT, H_s, H_t, V, dtype, num_chunks) bytes (for
 *   num_chunks == 0, at least the size for one chunk's worth of rows that
 *   fits). It holds both logits chunks (the student chunk becomes dZ in
 *   place, PR #1352 Details), per-row loss, row statistics (for bf16, per-tile
 *   partials written by the logits products), split-K partial sums, and for
 *   bf16 the transposed dZ and X_s chunk the weight-gradient product reads.
 *   For bf16 with V a multiple of 256, H_s a multiple of 64, BT above 4096
 *   and chunks of at least 512 rows, the size also counts W_s^T (V * H_s * 2
 *   bytes), which the first chunk's student logits product writes so that
 *   grad_input reads both of its operands along the reduction index (the
 *   write costs a fixed time, the faster grad_input gains per row). A workspace that is short of
 *   exactly that region still runs, with grad_input reading W_s as given
 *   (same results, a slower product); the region is also unused when
 *   grad_X_s is NULL. Its contents on entry do not matter.
 * Errors: FLJSD_EINVAL, FLJSD_EDTYPE, FLJSD_EALIGN, FLJSD_EWORKSPACE (all
 *   before any work is enqueued), FLJSD_EDEVICE, FLJSD_EHIP.
 */
int fljsd_forward_backward(const void* X_s, const void* W_s,
                           const void* X_t, const void* W_t,
                           int64_t BT, int64_t H_s, int64_t H_t, int64_t V,
                           int dtype, float beta, float temperature,
                           int reduction, int num_chunks,
                           float* loss, void* grad_X_s, void* grad_W_s,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

/* Flag bits of fljsd_forward_backward_ex. */
#define FLJSD_ACCUMULATE_GRAD_W 1u  /* add this call's weight gradient to the
                                       values grad_W_s already holds */
#define FLJSD_TEMPERATURE_SQUARED 2u /* multiply the loss, and so every gradient,
                                        by temperature^2 (PR #1352, Open question 2:
                                        the soft-target convention of Hinton et al.) */

/*
 * fljsd_forward_backward_ex - fljsd_forward_backward with a choice of
 * weight-gradient accumulation (PR #1429 Details: the accum_dtype=float32
 * path, where the per-chunk products add up in fp32).
 *
 * Same arguments, outputs, workspace and errors as fljsd_forward_backward,
 * plus:
 *   grad_w_dtype  element type of grad_W_s: `dtype`, or FLJSD_F32 with
 *                 FLJSD_BF16 inputs. With FLJSD_F32 the bf16 products
 *                 (fp32-accumulated inside each GEMM) are stored and summed
 *                 over chunks in fp32 with no rounding in between, so the
 *                 result does not carry one bf16 rounding per chunk. Any
 *                 other value is FLJSD_EDTYPE.
 *   flags         bitwise OR of:
 *                 FLJSD_ACCUMULATE_GRAD_W: the first chunk adds to grad_W_s
 *                 instead of overwriting it, so grad_W_s must hold
 *                 initialized values on entry (for summing gradients over
 *                 several calls, e.g. micro-batches of one optimizer step);
 *                 FLJSD_TEMPERATURE_SQUARED: loss (also each per-row loss of
 *                 FLJSD_NONE) and gradients carry an extra factor T^2.
 *                 Unknown bits are FLJSD_EINVAL.
 * fljsd_forward_backward(...) is fljsd_forward_backward_ex(..., dtype, 0, ...).
 * The workspace size does not depend on these two arguments.
 */
int fljsd_forward_backward_ex(const void* X_s, const void* W_s,
                              const void* X_t, const void* W_t,
                              int64_t BT, int64_t H_s, int64_t H_t, int64_t V,
                              int dtype, float beta, float temperature,
                              int reduction, int num_chunks,
                              float* loss, void* grad_X_s, void* grad_W_s,
                              int grad_w_dtype, unsigned flags,
                              void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * fljsd_generalized_jsd - the loss step alone over given logits: the three
 * online-softmax passes (PR #1352 Details: statistics m/d for both
 * distributions; then loss and dX_sum; then dX), without the GEMMs.
 *
 *   logits_s, logits_t [BT, ld] in dtype, the first V columns used.
 *   loss      fp32: 1 value, or BT values for FLJSD_NONE.
 *   grad_logits_s [BT, ld] in dtype, or NULL for the loss only. It receives
 *             d loss / d logits_s, including 1/T and the reduction scale. It
 *             may equal logits_s (in place: the student logits are
 *             overwritten by their gradient); any other overlap is an error
 *             the library does not detect.
 *   Columns V..ld-1 are neither read nor written. Any ld >= V works; rows
 *             whose stride is a multiple of 16 bytes take the vector path.
 * Workspace: at least fljsd_generalized_jsd_workspace_size(BT, V, dtype).
 */
int fljsd_generalized_jsd(const void* logits_s, const void* logits_t,
                          int64_t BT, int64_t V, int64_t ld, int dtype,
                          float beta, float temperature, int reduction,
                          float* loss, void* grad_logits_s,
                          void* workspace, size_t workspace_bytes,
                          void* stream);

/* Bytes of the device scratch array behind fljsd_generalized_jsd_noalloc
 * (8 MiB per GPU the library runs on, held until the process ends). */
#define FLJSD_NOALLOC_SCRATCH_BYTES (8u << 20)

/*
 * fljsd_generalized_jsd_noalloc - fljsd_generalized_jsd without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Arguments, outputs and results are those of fljsd_generalized_jsd. The
 * workspace is a file-scope device array of FLJSD_NOALLOC_SCRATCH_BYTES inside
 * the library, one per GPU, whose address is looked up on the first call on
 * each device (with that device current). The call allocates nothing (no
 * hipMalloc, no allocating library routine) and clears nothing: the loss
 * passes write every scratch byte before they read it.
 * Every call on one GPU shares that GPU's array and leaves the last call's
 * contents in it: calls that overlap on one GPU (on different streams, or
 * from different threads without ordering) race and give wrong results.
 * Order them on one stream.
 * Errors: as fljsd_generalized_jsd; FLJSD_EWORKSPACE (before any HIP call)
 * when fljsd_generalized_jsd_workspace_size(BT, V, dtype) exceeds
 * FLJSD_NOALLOC_SCRATCH_BYTES (about 174,000 rows at any V); FLJSD_EHIP when
 * the scratch address cannot be looked up.
 */
int fljsd_generalized_jsd_noalloc(const void* logits_s, const void* logits_t,
                                  int64_t BT, int64_t V, int64_t ld, int dtype,
                                  float beta, float temperature, int reduction,
                                  float* loss, void* grad_logits_s, void* stream);

/*
 * fljsd_jsd_logprob - generalized JSD over given log-probabilities, the
 * log-space contract of the public JSD op (PR #1352, Open question 3), in
 * one pass.
 *
 *   logq_s, logp_t [BT, ld] in dtype: student and teacher log-probabilities
 *             (natural log), first V columns used; -inf means probability 0.
 *             They are taken as given: nothing renormalizes them.
 *   beta in [0, 1]: 0 is KL(P||Q) (P = exp(logp_t), Q = exp(logq_s)),
 *             1 is KL(Q||P), between them beta KL(P||M) + (1-beta) KL(Q||M).
 *   loss      fp32: 1 value, or BT per-row sums for FLJSD_NONE.
 *   grad_logq_s [BT, ld] in dtype, or NULL: d loss / d logq_s elementwise
 *             (each input element is an independent variable; no softmax
 *             chain rule), including the reduction scale. May equal logq_s.
 *   Exact ties P == Q contribute no loss and, for 0 < beta < 1, no
 *   gradient (PR #1374); in the KL branches the tie gradient is the true
 *   derivative (-P for beta 0, Q for beta 1).
 * Workspace: at least fljsd_generalized_jsd_workspace_size(BT, V, dtype).
 * Errors: as fljsd_generalized_jsd.
 */
int fljsd_jsd_logprob(const void* logq_s, const void* logp_t,
                      int64_t BT, int64_t V, int64_t ld, int dtype,
                      float beta, int reduction, float* loss, void* grad_logq_s,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * fljsd_tvd - total variation distance between given distributions, with the
 * gradient fix at ties (PR #1374 "Fix TVD gradient at p == q", Summary).
 *
 *   p, q   [BT, ld] in dtype, first V columns used.
 *   loss   fp32: 1 value, or for FLJSD_NONE the BT x V elementwise losses
 *          |p - q| / 2, dense with row stride V.
 *   grad_p [BT, ld] in dtype, or NULL: d loss / d p = scale/2 * sign(p - q),
 *          exactly 0 where p == q. May equal p.
 * Workspace: at least fljsd_generalized_jsd_workspace_size(BT, V, dtype).
 * Errors: as fljsd_generalized_jsd (beta and temperature do not apply).
 */
int fljsd_tvd(const void* p, const void* q, int64_t BT, int64_t V, int64_t ld,
              int dtype, int reduction, float* loss, void* grad_p,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * fljsd_flce_forward_backward - fused-linear cross-entropy with hard labels,
 * forward and backward: the pattern the JSD pass follows (PR #1352, Details:
 * lm_head GEMM, online softmax in two passes, gradient written over the
 * logits in place; PR #1429: grad_weight written straight from the product,
 * first chunk overwriting).
 *
 *   X [BT, H], W [V, H] in dtype (16-byte aligned, H a multiple of 8 bf16 /
 *             4 fp32 elements); labels [BT] int64 (8-byte aligned).
 *   A row counts unless its label is ignore_index or lies outside [0, V);
 *   a row that does not count has loss 0 and gradient 0.
 *   label_smoothing eps in [0, 1]: row loss
 *             lse - (1 - eps) z_y - (eps / V) sum_v z_v, with lse the row's
 *             log-sum-exp of the logits z = X W^T (eps = 0: -log softmax(z)_y).
 *   reduction FLJSD_MEAN: sum over counted rows / number of counted rows
 *             (nan loss and zero gradients when none counts); FLJSD_BATCHMEAN:
 *             / BT; FLJSD_SUM; FLJSD_NONE: loss[r] per row.
 *   num_chunks as for fljsd_forward_backward (0: fljsd_flce_plan_num_chunks
 *             for the workspace size).
 * Outputs (every element written): loss fp32 (1 or BT values); grad_X
 *   [BT, H] and grad_W [V, H] in dtype, each optional (NULL skips it).
 * Workspace: at least fljsd_flce_workspace_size(BT, H, V, dtype, num_chunks),
 *   which counts, for the shapes named under fljsd_forward_backward, a W^T
 *   region (V * H * 2 bytes) for grad_X; a workspace short of exactly that
 *   region runs grad_X on W as given (same results).
 * Errors: FLJSD_EINVAL (NULL required pointer, sizes <= 0, label_smoothing
 *   outside [0, 1] or nan, num_chunks < 0), FLJSD_EDTYPE, FLJSD_EALIGN,
 *   FLJSD_EWORKSPACE, FLJSD_EDEVICE, FLJSD_EHIP.
 */
int fljsd_flce_forward_backward(const void* X, const void* W, const int64_t* labels,
                                int64_t BT, int64_t H, int64_t V, int dtype,
                                int64_t ignore_index, float label_smoothing,
                                int reduction, int num_chunks, float* loss,
                                void* grad_X, void* grad_W,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * fljsd_flce_forward_backward_ex - fljsd_flce_forward_backward with the
 * weight-gradient options of fljsd_forward_backward_ex (PR #1429, Details:
 * the accum_dtype=float32 path, where the per-chunk products of grad_weight
 * add up in fp32):
 *   grad_w_dtype  `dtype`, or FLJSD_F32 with FLJSD_BF16 inputs (grad_W [V, H]
 *                 in fp32: the bf16 products stored and summed over chunks in
 *                 fp32, no rounding in between); anything else FLJSD_EDTYPE.
 *   flags         0 or FLJSD_ACCUMULATE_GRAD_W (the first chunk adds to the
 *                 grad_W the caller passes); other bits FLJSD_EINVAL.
 * fljsd_flce_forward_backward(...) is this call with (dtype, 0). The
 * workspace size does not depend on either argument.
 */
int fljsd_flce_forward_backward_ex(const void* X, const void* W, const int64_t* labels,
                                   int64_t BT, int64_t H, int64_t V, int dtype,
                                   int64_t ignore_index, float label_smoothing,
                                   int reduction, int num_chunks, float* loss,
                                   void* grad_X, void* grad_W, int grad_w_dtype,
                                   unsigned flags, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Workspace bytes of fljsd_flce_forward_backward (0 for invalid arguments),
 * and the smallest chunk count whose workspace, less the optional W^T
 * region, fits `budget_bytes` (or a negative status code). Host-only. */
size_t fljsd_flce_workspace_size(int64_t BT, int64_t H, int64_t V, int dtype, int num_chunks);
int fljsd_flce_plan_num_chunks(int64_t BT, int64_t H, int64_t V, int dtype,
                               size_t budget_bytes);

/* Workspace bytes fljsd_forward_backward needs for this shape with
 * num_chunks >= 1 chunks, after the pages' per-chunk memory model (PR #1352,
 * Details, memory table: a chunk of C rows holds both logits tensors, and only
 * the per-row loss grows with BT): for bf16 about 3 * C * V * 2 bytes (student
 * logits / dZ, teacher logits, dZ^T) plus C * H_s * 2 (X_s^T) and small
 * per-row arrays (and W_s^T, V * H_s * 2, for the shapes named under
 * fljsd_forward_backward); for fp32 2 * C * V * 4 plus the per-row arrays. Pure host
 * arithmetic; no device is touched. Returns 0 for invalid arguments (sizes
 * <= 0, num_chunks < 1, bad dtype). */
size_t fljsd_workspace_size(int64_t BT, int64_t H_s, int64_t H_t, int64_t V,
                            int dtype, int num_chunks);

/* Workspace bytes fljsd_generalized_jsd needs. Pure host arithmetic. */
size_t fljsd_generalized_jsd_workspace_size(int64_t BT, int64_t V, int dtype);

/* Chunk policy (a replacement for the cdiv(V, H) heuristic that PR #1352,
 * Open question 4, calls mis-tuned for JSD): the smallest num_chunks >= 1
 * whose workspace, less the optional W_s^T region, fits in budget_bytes (that
 * region never costs a chunk; it is used when the budget also holds it).
 * Larger chunks keep the GEMMs
 * compute-bound, and the pages' sweep shows speed rising with chunk size.
 * Pure host arithmetic. Returns the count, or FLJSD_EINVAL for invalid sizes,
 * or FLJSD_EWORKSPACE when even one-row chunks do not fit. */
int fljsd_plan_num_chunks(int64_t BT, int64_t H_s, int64_t H_t, int64_t V,
                          int dtype, size_t budget_bytes);

/* Static description of a status code (the codes are this library's reading;
 * the pages define none). */
const char* fljsd_strerror(int code);

/* Details of the calling thread's most recent failure ("" if none). */
const char* fljsd_last_error(void);

/*
 * Kernel timing for measurement. While enabled, the library brackets every
 * kernel launch with a pair of HIP events on the launch stream and adds the
 * elapsed time, the launch count and the launch's algorithmic work to a
 * per-kernel-class tally. fljsd_profile_read() waits for the recorded events
 * and fills up to `n` classes (see FLJSD_KCLASS_*): total milliseconds,
 * launches, algorithmic floating-point operations and algorithmic HBM bytes.
 * Enabling clears the tally. Not thread safe; intended for a benchmark that
 * drives one stream. Returns FLJSD_OK or FLJSD_EHIP.
 */
#define FLJSD_KCLASS_GEMM_LOGITS 0      /* Z = X W^T (student and teacher) */
#define FLJSD_KCLASS_JSD_STATS 1        /* pass 1: row max / denominator */
#define FLJSD_KCLASS_JSD_LOSS 2         /* pass 2: loss and G (bf16 with grad_W: G alone) */
#define FLJSD_KCLASS_JSD_GRAD 3         /* pass 3: dZ in place (and dZ^T, loss partials) */
#define FLJSD_KCLASS_GEMM_GRAD_INPUT 4  /* grad_X = dZ W_s */
#define FLJSD_KCLASS_SPLITK_REDUCE 5    /* split-K partial sums -> grad_X */
#define FLJSD_KCLASS_GEMM_GRAD_WEIGHT 6 /* grad_W (=|+=) dZ^T X_s */
#define FLJSD_KCLASS_LOSS_REDUCE 7      /* scalar loss; row losses from pass 3's partials */
#define FLJSD_KCLASS_TRANSPOSE 8        /* dZ^T and X_s^T for the grad_W product */
#define FLJSD_KCLASS_ELEM_LOSS 9        /* fljsd_jsd_logprob / fljsd_tvd element pass */
#define FLJSD_KCLASS_CE_STATS 10        /* cross-entropy pass 1: row max / denominator */
#define FLJSD_KCLASS_CE_GRAD 11         /* cross-entropy pass 2: dZ in place, row loss */
#define FLJSD_KCLASS_COUNT 12

int fljsd_profile_enable(int enable);
int fljsd_profile_read(double* total_ms, int64_t* launches, double* flops,
                       double* hbm_bytes, int n);

#ifdef __cplusplus
}
#endif

#endif /* FLJSD_H */
