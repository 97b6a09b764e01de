/*
 * mhc_coeff_bwd.h - C ABI of the MI355X (gfx950) mHC coefficient backward
 * epilogue: the step after the Sinkhorn backward that turns the upstream
 * gradients of the pre / post gates and of the residual-mixing logits into
 * the gradient of the coefficient projection and the bias and gain
 * gradients.
 *
 * Operation (page "perf: fuse mHC coefficient backward epilogue",
 * Liger-Kernel pull request 1402, section Summary: the pre/post sigmoid
 * derivatives, grad_mix and fp32 partial sums for grad_b and the alpha
 * gradients, then a deterministic reducer for the bias columns and the three
 * scalar alpha gradients; section Risks and Limitations: a fixed two-stage
 * reduction order). The page prints no formulas; this library implements
 * the following reading of it.
 *
 * Expansion n in {2, 4, 8}; m = 2n + n*n coefficient columns (24 at n = 4):
 * columns [0, n) are the pre gates, [n, 2n) the post gates, [2n, m) the
 * n x n residual-mixing logits in row-major order. Column j belongs to group
 * k(j) = 0, 1, 2 respectively. The forward being differentiated is
 *     z[r,j] = alpha[k(j)] * mix[r,j] + b[j]
 *     pre    = sigmoid(z[:, 0:n])
 *     post   = c * sigmoid(z[:, n:2n])           (c = post_scale)
 *     z[:, 2n:m] -> Sinkhorn normalisation (its backward supplies grad_res)
 * and, per row r (R rows; every row is one token of one batch entry):
 *     d[r,j] = grad_pre[r,j]  * (pre[r,j]  * (1 - pre[r,j]))                j <  n
 *     d[r,j] = grad_post[r,i] * (post[r,i] * (1 - post[r,i] / c))           i = j - n
 *     d[r,j] = grad_res[r,j-2n]                                             j >= 2n
 *     grad_mix[r,j] = alpha[k(j)] * d[r,j]
 *     e[r,k]        = sum over j of group k, ascending, from +0.0, of d[r,j] * mix[r,j]
 *     grad_b[j]     = row_sum of d[:,j]
 *     grad_alpha[k] = row_sum of e[:,k]
 * post[r,i] / c is the post gate's sigmoid, so the post derivative is
 * c * s * (1 - s) written in the saved output. Every product, quotient, sum
 * and difference is one fp32 operation rounded to nearest even (the
 * quotient correctly rounded) in exactly the nesting written; products and
 * sums are never fused.
 *
 * row_sum (fixed; depends only on R):
 *   1. rows are cut into chunks of 64 consecutive rows (rows past R count as
 *      +0.0); each chunk is summed by the halving tree: for off = 32, 16, 8,
 *      4, 2, 1 in that order, x[i] += x[i+off] for all i < off; the chunk
 *      sum is x[0];
 *   2. 64 accumulators start at +0.0; chunk sum c is added to accumulator
 *      c mod 64, in ascending c; the 64 accumulators are summed by the same
 *      halving tree.
 * With R = 0 both sums are +0.0.
 *
 * Tensors (fp32, contiguous, row-major; DEVICE pointers on the current HIP
 * device, owned by the caller):
 *     mix [R, m], pre [R, n], post [R, n], grad_pre [R, n], grad_post [R, n],
 *     grad_res [R, n*n], alpha [3]                                  (inputs)
 *     grad_mix [R, m], grad_b [m], grad_alpha [3]                   (outputs)
 *     workspace: mhc_coeff_bwd_workspace_bytes(R, n) bytes of device memory
 *     (0 when R = 0; NULL is then allowed). Its first 4 bytes are an arrival
 *     counter: they must be zero before the first call that uses the
 *     workspace, and every call that completes leaves them zero, so a
 *     workspace zeroed once when it is allocated serves any sequence of
 *     calls. The rest holds the per-chunk sums; its contents before and
 *     after a call mean nothing to the caller. Calls that share a workspace
 *     must not run concurrently (they are safe one after another on one
 *     stream).
 *
 * Launches: the second stage of row_sum runs either in the same launch as
 * the first (the block that finishes its chunks last does it) or in a second
 * launch. Both give the same bits. The policy (`launches` = 0) takes one
 * launch at n = 2 or 4 up to 256 chunks (16384 rows), two otherwise;
 * `launches` = 1 or 2 forces a form. R = 0 always takes the second form (it
 * only writes the +0.0 sums).
 *
 * Rules: calls enqueue one or two kernels on `stream` (a hipStream_t cast to
 * void*, NULL = null stream) and never synchronise; inputs must stay valid
 * until the stream reaches them. The library allocates no memory at run time
 * (mhc_coeff_bwd_noalloc's fixed array is part of the loaded device code).
 * n not in {2,4,8},
 * R < 0, R > MHC_COEFF_MAX_ROWS, c not finite and positive, a NULL or
 * non-4-byte-aligned pointer that the call needs (the row tensors, alpha and
 * the workspace when R > 0; grad_b and grad_alpha always), or a workspace
 * smaller than required give MHC_ERROR_INVALID_VALUE; any overlap between an
 * output (the workspace counts as one) and an input or another output gives
 * MHC_ERROR_ALIASING. On either error nothing is launched and nothing is
 * written. A failed launch gives MHC_ERROR_HIP (the status of that launch;
 * the thread's HIP last-error state is neither read nor cleared).
 * mhc_coeff_last_error_message describes the most recent failure on the
 * calling thread. The status codes are those of mhc_h_aggregate.h.
 */
#ifndef MHC_COEFF_BWD_H
#define MHC_COEFF_BWD_H

#include <stdint.h>

#include "mhc_h_aggregate.h"

#ifdef __cplusplus
extern "C" {
#endif

#define MHC_COEFF_ABI_VERSION 4

/* Rows per first-stage chunk of row_sum. */
#define MHC_COEFF_CHUNK 64

/* Most rows one call accepts (2^28: keeps every workspace byte offset and
 * buffer range within 31 bits at every expansion rate). */
#define MHC_COEFF_MAX_ROWS (1LL << 28)

/* Storage formats of the six row tensors and grad_mix (mhc_coeff_bwd_ex). */
#define MHC_COEFF_F32 0
#define MHC_COEFF_BF16 1
#define MHC_COEFF_F16 2

/* Bytes of the fixed device array that mhc_coeff_bwd_noalloc uses as its
 * workspace (one array per GPU the library runs on). */
#define MHC_COEFF_SCRATCH_BYTES (2LL << 20)

int mhc_coeff_abi_version(void);

const char* mhc_coeff_last_error_message(void);

/* Bytes of workspace a call with R rows at expansion n needs:
 * 256 + (m + 3) * ceil(R / 64) * 4, or 0 when R = 0. Returns -1 for an
 * invalid n or R. */
int64_t mhc_coeff_bwd_workspace_bytes(int64_t rows, int32_t n);

/* Number of launches a call with these arguments makes (1 or 2; see
 * Launches above), on the host only. Returns -1 for an invalid n, R or
 * launches value. */
int32_t mhc_coeff_bwd_plan(int64_t rows, int32_t n, int32_t launches);

/* Checks the arguments exactly as mhc_coeff_bwd does, on the host only:
 * touches no device memory and launches nothing. */
mhc_status mhc_coeff_bwd_validate(const float* mix, const float* pre, const float* post,
                                  const float* grad_pre, const float* grad_post,
                                  const float* grad_res, const float* alpha, float post_scale,
                                  const float* grad_mix, const float* grad_b,
                                  const float* grad_alpha, const void* workspace,
                                  int64_t workspace_bytes, int64_t rows, int32_t n);

/* The epilogue described above. launches: 0 (policy), 1 or 2; any other
 * value gives MHC_ERROR_INVALID_VALUE. start_event / stop_event (hipEvent_t
 * cast to void*, each may be NULL) are recorded when the first of the
 * call's kernels starts and when the last one ends. */
mhc_status mhc_coeff_bwd(const float* mix, const float* pre, const float* post,
                         const float* grad_pre, const float* grad_post, const float* grad_res,
                         const float* alpha, float post_scale, float* grad_mix, float* grad_b,
                         float* grad_alpha, void* workspace, int64_t workspace_bytes,
                         int64_t rows, int32_t n, int32_t launches, void* stream,
                         void* start_event, void* stop_event);

/*
 * The epilogue on 16-bit (or fp32) inputs (page Testing Done: FP16, BF16
 * and FP32 inputs; Performance Method: BF16 is the primary case).
 * dtype = MHC_COEFF_F32, MHC_COEFF_BF16 or MHC_COEFF_F16 is the storage
 * format of mix, pre, post, grad_pre, grad_post, grad_res and grad_mix (raw
 * bit patterns for the 16-bit formats; 2-byte alignment). Every stored
 * input value is widened to fp32 exactly, the computation above runs in
 * fp32 unchanged, and grad_mix is rounded once to the format (nearest even,
 * subnormals kept, overflow to infinity). alpha, grad_b and grad_alpha
 * stay fp32, and so do the row sums, which add the fp32 values of d and e
 * (never the rounded grad_mix). Everything else as in mhc_coeff_bwd, which
 * is this call with MHC_COEFF_F32; an unknown dtype gives
 * MHC_ERROR_INVALID_VALUE.
 */
mhc_status mhc_coeff_bwd_ex(const void* mix, const void* pre, const void* post,
                            const void* grad_pre, const void* grad_post, const void* grad_res,
                            const float* alpha, float post_scale, void* grad_mix, float* grad_b,
                            float* grad_alpha, void* workspace, int64_t workspace_bytes,
                            int64_t rows, int32_t n, int32_t dtype, int32_t launches,
                            void* stream, void* start_event, void* stop_event);

/* The argument checks of mhc_coeff_bwd_ex, on the host only. */
mhc_status mhc_coeff_bwd_validate_ex(const void* mix, const void* pre, const void* post,
                                     const void* grad_pre, const void* grad_post,
                                     const void* grad_res, const float* alpha, float post_scale,
                                     const void* grad_mix, const float* grad_b,
                                     const float* grad_alpha, const void* workspace,
                                     int64_t workspace_bytes, int64_t rows, int32_t n,
                                     int32_t dtype);

/*
 * No-allocation variant of mhc_coeff_bwd, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same operation, arguments and results as
 * mhc_coeff_bwd, except that the workspace is a fixed array of
 * MHC_COEFF_SCRATCH_BYTES (2 MiB) inside the library's device code, one per
 * GPU, held until the process ends; the caller still passes every input
 * and output. The call allocates nothing (no hipMalloc, no hipFree).
 *   - Limit: mhc_coeff_bwd_workspace_bytes(R, n) must not exceed
 *     MHC_COEFF_SCRATCH_BYTES, i.e. at most 47,656 chunks of 64 rows at
 *     n = 2 (3,049,984 rows), 19,415 at n = 4 (1,242,560 rows) and 6,315 at
 *     n = 8 (404,160 rows); larger calls give MHC_ERROR_INVALID_VALUE before
 *     anything else is touched.
 *   - Sharing: every call on one GPU uses that GPU's array, which keeps the
 *     last call's contents. Calls that overlap in time on one GPU (other
 *     streams, other threads) race and give undefined results; calls one
 *     after another on one stream are safe.
 *   - Set-up: the first call on a device looks up the array's address there
 *     (hipGetSymbolAddress) and enqueues, ahead of its own kernels, a
 *     one-wave kernel that zeroes the array's arrival counter; every
 *     completed call leaves the counter at zero. start_event / stop_event
 *     time the operation's kernels, not that set-up kernel.
 *   - R == 0 touches no scratch (it only writes the +0.0 sums).
 */
mhc_status mhc_coeff_bwd_noalloc(const float* mix, const float* pre, const float* post,
                                 const float* grad_pre, const float* grad_post,
                                 const float* grad_res, const float* alpha, float post_scale,
                                 float* grad_mix, float* grad_b, float* grad_alpha, int64_t rows,
                                 int32_t n, int32_t launches, void* stream, void* start_event,
                                 void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* MHC_COEFF_BWD_H */
