/*
 * mhc_h_aggregate.h - C ABI of the MI355X (gfx950) mHC pre / H-aggregate
 * library: the forward collapse of the hyper-connection residual stream and
 * its backward.
 *
 * Operation (page "Add batch-invariant h_aggregate kernel", RL-Kernel pull
 * request 366, section Summary):
 *
 *     residual [T, 4, H]  bf16      (hyper-connection expansion 4)
 *     pre      [T, 4]     fp32
 *     out      [T, H]     bf16
 *     out[t,h] = bf16( (pre[t,0]*r0 + pre[t,1]*r1) + (pre[t,2]*r2 + pre[t,3]*r3) ),
 *     r_i = residual[t,i,h]
 *
 * Arithmetic contract (same page, section Batch invariance): every product
 * and sum is one fp32 operation rounded to nearest even, never fused into a
 * multiply-add; the association is the fixed tree (0+1)+(2+3); bf16 inputs
 * are widened exactly and the result is rounded to bf16 (nearest even) once.
 * Denormals are kept. Each output element is produced by one thread with no
 * atomics, so the bytes of out[t,:] depend only on residual[t], pre[t] and H:
 * never on T, on the batch partition, or on the launch configuration.
 *
 * Backward (asked for in the same page's review comments so that training
 * can converge; the formulas are the derivative of the forward):
 *
 *     grad_residual[t,i,h] = bf16( pre[t,i] * grad_out[t,h] )       (written)
 *     grad_pre[t,i]        = sum over h of grad_out[t,h] * residual[t,i,h]
 *
 * Each grad_out*residual product is one fp32 round-to-nearest multiply; it
 * is exact (two 8-bit significands) unless it falls below fp32's normal range.
 * The sum over h follows one fixed order that depends only on H, so
 * grad_pre is batch invariant:
 *   1. 256 fp32 accumulator lanes start at +0.0;
 *   2. group k holds the 8 consecutive elements h = 8k..8k+7 (the last group
 *      may be short); groups are visited in ascending k and group k is
 *      added, element by element in ascending h, to lane (k mod 256);
 *   3. lanes form 4 waves of 64; in each wave, for off = 32,16,8,4,2,1 in
 *      that order, x[j] += x[j+off] for all j < off; the wave result is x[0];
 *   4. grad_pre = (y0 + y2) + (y1 + y3) over the four wave results.
 * Every addition is one fp32 round-to-nearest-even operation.
 *
 * Common rules for every entry point below
 *   - All tensor pointers are DEVICE pointers on the current HIP device; the
 *     caller owns every buffer. bf16 tensors are passed as raw uint16_t bit
 *     patterns. Tensors are contiguous and row-major in the shapes above.
 *   - `stream` is a hipStream_t cast to void*; NULL means the null stream.
 *     Calls only enqueue work: they never synchronise, and inputs must stay
 *     valid until the stream reaches the call. The library allocates no
 *     memory and keeps no mutable global state; it is reentrant.
 *   - T == 0 is a successful no-op (pointers may then be NULL). T < 0,
 *     H < 1, H > MHC_MAX_H, a NULL pointer when T > 0, a pointer that is not
 *     aligned to its element size, or sizes whose byte counts overflow
 *     int64 give MHC_ERROR_INVALID_VALUE. Any overlap between an output and
 *     an input, or between the two backward outputs, gives
 *     MHC_ERROR_ALIASING. On either error nothing is launched and no output
 *     is touched. A failed kernel launch gives MHC_ERROR_HIP (with the
 *     status of that launch itself; the library never reads or clears the
 *     thread's HIP last-error state, so an error the caller had pending is
 *     still pending after the call).
 *   - A misaligned or odd-H buffer is not an error: it only narrows the
 *     vector width, which never changes a result bit.
 *   - mhc_last_error_message() returns a text describing the most recent
 *     failure on the calling thread.
 */
#ifndef MHC_H_AGGREGATE_H
#define MHC_H_AGGREGATE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MHC_ABI_VERSION 5

/* Hyper-connection expansion rate of the page's operation (Summary: residual
 * [T, 4, H]). The *_n entry points below also take 2 and 8. */
#define MHC_HC 4

/* Largest hidden size accepted. */
#define MHC_MAX_H (1LL << 26)

typedef enum mhc_status {
  MHC_SUCCESS = 0,
  MHC_ERROR_INVALID_VALUE = 1,
  MHC_ERROR_ALIASING = 2,
  MHC_ERROR_HIP = 3
} mhc_status;

/*
 * Launch shape. Passed to the *_ex entry points as an override (a field of
 * 0 means "let the launch policy choose") and returned by the plan queries
 * with every field filled in. No field changes any result bit: they exist so
 * that tests can prove that and benchmarks can sweep shapes.
 *   block_threads     forward: threads per block, a multiple of 64 in
 *                     [64, 1024]. Backward, split layout: 0 or 256 (one
 *                     block of 4 waves owns a token's reduction); row
 *                     layout: 64, 128, 256 or 512 (1, 2, 4 or 8 rows per
 *                     block; default 256).
 *   vec_width         bf16 elements per vector access: 1, 2, 4 or 8. It must
 *                     divide H and match the alignment of every bf16 buffer.
 *   units_per_thread  forward: vector units each thread handles (1, 2 or
 *                     4; default 1). Backward: 8-element groups each lane
 *                     keeps in flight, a ring of loads whose slots are
 *                     refilled with the lane's next group once consumed -
 *                     1, 2 or 4 in the split layout (default: the most the
 *                     register budget allows), 4, 8 or 12 in the row layout
 *                     (default 12 for rows the library compiles for their
 *                     exact chunk count, 8 otherwise, fewer where the
 *                     budget requires). More
 *                     than the register budget allows for the vec_width,
 *                     layout, expansion rate and streams_per_block gives
 *                     MHC_ERROR_INVALID_VALUE; the plan query reports the
 *                     value a call would use.
 *   tokens_per_block  backward split layout only: tokens one block handles
 *                     in sequence, 1..4096.
 *   streams_per_block backward split layout only: residual streams one
 *                     block handles, 1, 2 or 4. The summation order is
 *                     defined per (token, stream), so a token's streams may
 *                     be spread over blocks without any change in the
 *                     result.
 *   layout            backward only: MHC_BWD_SPLIT (a token's 256
 *                     accumulator lanes are the 256 threads of one block)
 *                     or MHC_BWD_ROWS (one wave streams one (token, stream)
 *                     row; each of its 64 lanes holds accumulator lanes
 *                     j, j+64, j+128, j+192 and the 64-lane trees run inside
 *                     the wave). The policy takes the row layout from
 *                     T * n = 544 rows on, unless a split-layout field is set or
 *                     the row layout does not fit the register budget
 *                     (scalar-width accumulating calls). Same summation
 *                     order, same bits.
 *   wave_priority     backward only: MHC_PRIO_FLAT (every wave at one issue
 *                     priority; a CU then serves its waves oldest first) or
 *                     MHC_PRIO_PROGRESS (row layout, rows of at most 16
 *                     chunks of 16-byte accesses, i.e. vec_width 8 and
 *                     H <= 8192: each wave starts at the highest priority
 *                     and steps down as it consumes each quarter of its row,
 *                     so the waves of a launch progress together). The
 *                     policy takes MHC_PRIO_PROGRESS for the written (not
 *                     the accumulating) backward when every row of the
 *                     call has a wave slot from the start (T * n <= 16 x
 *                     the device's compute units: T <= 1024 at n = 4 on
 *                     256 CUs; 256 CUs are assumed when no device can be
 *                     queried), MHC_PRIO_FLAT otherwise. Issue order only:
 *                     same bits. The policy assumes the call has the GPU
 *                     to itself; alongside other kernels that hold CUs,
 *                     MHC_PRIO_FLAT may be the faster choice.
 * Forward calls reject non-zero backward-only fields.
 */
typedef struct mhc_launch {
  int32_t block_threads;
  int32_t vec_width;
  int32_t units_per_thread;
  int32_t tokens_per_block;
  int32_t streams_per_block;
  int32_t layout;
  int32_t wave_priority;
} mhc_launch;

/* Backward layouts (mhc_launch.layout); both compute the same bits. */
#define MHC_BWD_SPLIT 1 /* a token's 256 accumulator lanes over a block's 4 waves */
#define MHC_BWD_ROWS 2  /* one wave per (token, stream) row, 4 lanes per wave lane */

/* Backward issue priorities (mhc_launch.wave_priority); same bits. */
#define MHC_PRIO_FLAT 1     /* one priority for every wave */
#define MHC_PRIO_PROGRESS 2 /* row layout: priority steps down with the row's progress */

/* Version of this ABI (MHC_ABI_VERSION of the built library). */
int mhc_abi_version(void);

/* Static name of a status code ("MHC_SUCCESS", ...). Never NULL. */
const char* mhc_status_string(mhc_status status);

/* Text describing the last failure on the calling thread ("" if none).
 * Valid until the next call into this library on that thread. */
const char* mhc_last_error_message(void);

/*
 * Forward (Summary and Batch invariance of "Add batch-invariant h_aggregate
 * kernel").
 *   residual  [T,4,H] bf16 bits, read
 *   pre       [T,4]   fp32, read
 *   out       [T,H]   bf16 bits, written (every element, once)
 */
mhc_status mhc_h_aggregate_fwd(const uint16_t* residual, const float* pre,
                               uint16_t* out, int64_t T, int64_t H,
                               void* stream);

/* Forward with a launch-shape override (NULL = same as mhc_h_aggregate_fwd).
 * An override the buffers cannot honour gives MHC_ERROR_INVALID_VALUE. */
mhc_status mhc_h_aggregate_fwd_ex(const uint16_t* residual, const float* pre,
                                  uint16_t* out, int64_t T, int64_t H,
                                  void* stream, const mhc_launch* launch);

/*
 * Backward (review comments of "Add batch-invariant h_aggregate kernel":
 * the gradient of the forward formula).
 *   residual       [T,4,H] bf16 bits, read
 *   pre            [T,4]   fp32, read
 *   grad_out       [T,H]   bf16 bits, read
 *   grad_residual  [T,4,H] bf16 bits, written: bf16(pre[t,i]*grad_out[t,h])
 *   grad_pre       [T,4]   fp32, written: the fixed-order sum above
 * Both gradients are overwritten, never accumulated into.
 */
mhc_status mhc_h_aggregate_bwd(const uint16_t* residual, const float* pre,
                               const uint16_t* grad_out,
                               uint16_t* grad_residual, float* grad_pre,
                               int64_t T, int64_t H, void* stream);

/* Backward with a launch-shape override (NULL = same as the plain call). */
mhc_status mhc_h_aggregate_bwd_ex(const uint16_t* residual, const float* pre,
                                  const uint16_t* grad_out,
                                  uint16_t* grad_residual, float* grad_pre,
                                  int64_t T, int64_t H, void* stream,
                                  const mhc_launch* launch);

/*
 * Timed variants: identical to the *_ex calls, plus two caller-created HIP
 * events (hipEvent_t cast to void*, created with timing enabled; either may
 * be NULL). start_event takes the start timestamp of the call's first kernel
 * dispatch and stop_event the end timestamp of its last, taken by the
 * dispatch itself (hipExtLaunchKernel), so hipEventElapsedTime between them
 * is the kernels' own execution time with no marker packets in the stream.
 * With T == 0 both events are recorded on the stream with nothing between
 * them. The events stay owned by the caller.
 */
mhc_status mhc_h_aggregate_fwd_timed(const uint16_t* residual, const float* pre,
                                     uint16_t* out, int64_t T, int64_t H,
                                     void* stream, const mhc_launch* launch,
                                     void* start_event, void* stop_event);
mhc_status mhc_h_aggregate_bwd_timed(const uint16_t* residual, const float* pre,
                                     const uint16_t* grad_out,
                                     uint16_t* grad_residual, float* grad_pre,
                                     int64_t T, int64_t H, void* stream,
                                     const mhc_launch* launch,
                                     void* start_event, void* stop_event);

/*
 * Accumulating backward (for training, where the residual stream's gradient
 * also receives contributions from other branches):
 *   grad_residual[t,i,h] = bf16( fp32(grad_residual[t,i,h]) + RN32(pre[t,i] *
 *                                grad_out[t,h]) )
 * i.e. the stored bf16 gradient is widened exactly, the fp32-rounded product
 * is added in fp32 and the sum is rounded to bf16 once. grad_residual is
 * read and written in place (it must still not overlap any input or
 * grad_pre); grad_pre is written as in mhc_h_aggregate_bwd. `launch`,
 * `start_event` and `stop_event` may each be NULL (same meaning as in the
 * *_ex and *_timed calls). Moves 26H + 32 bytes per token.
 */
mhc_status mhc_h_aggregate_bwd_acc(const uint16_t* residual, const float* pre,
                                   const uint16_t* grad_out,
                                   uint16_t* grad_residual, float* grad_pre,
                                   int64_t T, int64_t H, void* stream,
                                   const mhc_launch* launch, void* start_event,
                                   void* stop_event);

/*
 * Any supported expansion rate n in {2, 4, 8} (the second page's sibling
 * implementation covers HC in {2, 4, 8}; the first page fixes 4):
 *   residual [T, n, H] bf16, pre [T, n] fp32, out [T, H] bf16,
 *   grad_residual [T, n, H] bf16, grad_pre [T, n] fp32.
 * Forward: the n products are summed as a balanced pairwise tree, adjacent
 * pairs first, then pairs of pairs - (0+1)+(2+3) at n = 4 (identical to
 * mhc_h_aggregate_fwd), p0+p1 at n = 2, ((0+1)+(2+3))+((4+5)+(6+7)) at n = 8;
 * every product and sum one fp32 round-to-nearest-even operation, one bf16
 * rounding at the end. Backward: per stream exactly as above (the fixed
 * grad_pre order is per (token, stream)); accumulate = 1 selects the
 * accumulating form of mhc_h_aggregate_bwd_acc, 0 the written form. launch,
 * start_event and stop_event may each be NULL. An n outside {2, 4, 8} gives
 * MHC_ERROR_INVALID_VALUE; streams_per_block must not exceed n.
 */
mhc_status mhc_h_aggregate_fwd_n(const uint16_t* residual, const float* pre,
                                 uint16_t* out, int64_t T, int32_t n, int64_t H,
                                 void* stream, const mhc_launch* launch,
                                 void* start_event, void* stop_event);
mhc_status mhc_h_aggregate_bwd_n(const uint16_t* residual, const float* pre,
                                 const uint16_t* grad_out,
                                 uint16_t* grad_residual, float* grad_pre,
                                 int64_t T, int32_t n, int64_t H,
                                 int32_t accumulate, void* stream,
                                 const mhc_launch* launch, void* start_event,
                                 void* stop_event);

/*
 * Host-only checks and plan queries. They touch no device and no memory
 * behind the pointers (the pointers are used only as numbers for alignment
 * and overlap tests), so they run without a GPU.
 *
 * validate_*: the status the matching compute call would return before any
 * launch (argument, alignment and aliasing rules above).
 * plan_*: validates like the compute call, then writes the launch shape it
 * would use into *plan and the number of blocks it would launch in total
 * into *grid_blocks (either output pointer may be NULL).
 */
mhc_status mhc_h_aggregate_validate_fwd(const uint16_t* residual,
                                        const float* pre, const uint16_t* out,
                                        int64_t T, int64_t H);
mhc_status mhc_h_aggregate_validate_bwd(const uint16_t* residual,
                                        const float* pre,
                                        const uint16_t* grad_out,
                                        const uint16_t* grad_residual,
                                        const float* grad_pre, int64_t T,
                                        int64_t H);
mhc_status mhc_h_aggregate_plan_fwd(const uint16_t* residual, const float* pre,
                                    const uint16_t* out, int64_t T, int64_t H,
                                    const mhc_launch* launch, mhc_launch* plan,
                                    int64_t* grid_blocks);
mhc_status mhc_h_aggregate_plan_bwd(const uint16_t* residual, const float* pre,
                                    const uint16_t* grad_out,
                                    const uint16_t* grad_residual,
                                    const float* grad_pre, int64_t T,
                                    int64_t H, const mhc_launch* launch,
                                    mhc_launch* plan, int64_t* grid_blocks);
mhc_status mhc_h_aggregate_plan_fwd_n(const uint16_t* residual, const float* pre,
                                      const uint16_t* out, int64_t T, int32_t n,
                                      int64_t H, const mhc_launch* launch,
                                      mhc_launch* plan, int64_t* grid_blocks);
mhc_status mhc_h_aggregate_plan_bwd_n(const uint16_t* residual, const float* pre,
                                      const uint16_t* grad_out,
                                      const uint16_t* grad_residual,
                                      const float* grad_pre, int64_t T, int32_t n,
                                      int64_t H, int32_t accumulate,
                                      const mhc_launch* launch, mhc_launch* plan,
                                      int64_t* grid_blocks);
mhc_status mhc_h_aggregate_plan_bwd_acc(const uint16_t* residual,
                                        const float* pre,
                                        const uint16_t* grad_out,
                                        const uint16_t* grad_residual,
                                        const float* grad_pre, int64_t T,
                                        int64_t H, const mhc_launch* launch,
                                        mhc_launch* plan, int64_t* grid_blocks);

#ifdef __cplusplus
}
#endif

#endif /* MHC_H_AGGREGATE_H */
