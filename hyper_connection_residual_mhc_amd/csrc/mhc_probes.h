/*
 * mhc_probes.h - C ABI of the measurement library libmhc_probes.so, which
 * sits beside the operation's libraries and is used only by the tests and
 * the benchmark. Nothing here is part of the mHC operation.
 *
 * Rules as in mhc_h_aggregate.h: device pointers on the current HIP device,
 * owned by the caller; `stream` is a hipStream_t cast to void* (NULL = null
 * stream); calls only enqueue work; the library allocates nothing. Invalid
 * arguments give MHC_ERROR_INVALID_VALUE (nothing launched), overlapping
 * buffers MHC_ERROR_ALIASING, a failed launch MHC_ERROR_HIP;
 * mhc_probe_last_error_message() describes the most recent failure on the
 * calling thread.
 */
#ifndef MHC_PROBES_H
#define MHC_PROBES_H

#include <stdint.h>

#include "mhc_h_aggregate.h"

#ifdef __cplusplus
extern "C" {
#endif

#define MHC_PROBE_ABI_VERSION 2

int mhc_probe_abi_version(void);

const char* mhc_probe_last_error_message(void);

/*
 * Conversion probe: out[k] = bf16 bits of the fp32 value whose bit pattern
 * is (first_bits + k) mod 2^32, for k in [0, n), rounded by the device
 * routine every bf16 result of the h_aggregate kernels goes through (round
 * to nearest even; both libraries compile the same routine). Lets tests
 * compare the device rounding with an independent one over any range of
 * fp32 patterns, including all 2^32. out: [n] uint16, 2-byte aligned.
 * 0 <= n <= 2^32; n == 0 launches nothing.
 */
mhc_status mhc_bf16_rne_probe(uint32_t first_bits, int64_t n, uint16_t* out, void* stream);

/*
 * Streaming probe: a kernel that only moves bytes, with a given read:write
 * mix and no arithmetic, so that the operation's kernels can be compared
 * with what a plain stream of the same bytes takes on this GPU. One 64-lane
 * block per unit; a unit reads `reads` consecutive KiB of src and writes
 * `writes` consecutive KiB of dst (each access instruction covers 1 KiB:
 * 64 lanes x 16 bytes), all loads before the first store. Each written
 * 16-byte vector is the XOR of the unit's loaded vectors at that lane,
 * repeated `writes` times (a write-only unit writes its unit index in every
 * word). Cache policy: nontemporal loads; write-through stores for the 4:1
 * mix (the forward's policy), nontemporal stores otherwise.
 *   reads:writes  1:1 (copy), 4:1 (forward: 8H read, 2H written),
 *                 5:4 (backward: 10H read, 8H written),
 *                 9:4 (accumulating backward: 18H read, 8H written),
 *                 8:0 (read only), 0:8 (write only).
 *   With reads > 0: src_bytes is a non-negative multiple of reads KiB and
 *   dst_bytes is exactly (src_bytes / reads KiB) * writes KiB.
 *   With reads == 0: src_bytes is 0 (src may be NULL) and dst_bytes a
 *   multiple of writes KiB.
 *   src and dst are 16-byte aligned and disjoint. start_event / stop_event
 *   (hipEvent_t or NULL) are attached to the dispatch itself. Zero units
 *   launch nothing and record the events.
 */
mhc_status mhc_stream_probe(const void* src, int64_t src_bytes, void* dst, int64_t dst_bytes,
                            int32_t reads, int32_t writes, void* stream, void* start_event,
                            void* stop_event);

/*
 * Clock probe: the streaming probe's units and mixes (same byte layout,
 * cache policies and stored values), launched with `waves_per_block` units
 * per block (1, 4 or 16: blocks of 64, 256 or 1024 threads), where every
 * wave also stamps when it ran and where. Shows how a launch's waves are
 * spread over the accelerator complexes (XCDs) and over time, for any
 * launch shape, with no arithmetic in the way.
 *   stamps: [4 * units] uint64, 8-byte aligned, disjoint from src and dst;
 *   stamps_len is its element count (at least 4 * units). For unit u:
 *     stamps[4u + 0]  device wall clock as the wave starts,
 *     stamps[4u + 1]  ... once all its loads have returned,
 *     stamps[4u + 2]  ... once all its stores have completed,
 *     stamps[4u + 3]  XCC_ID (the XCD the wave ran on) in the low 32 bits,
 *                     the wave's HW_ID register in the high 32 bits.
 *   The wall clock is the device's constant-rate real-time counter (read
 *   with s_memrealtime); mhc_probe_wall_clock_khz gives its rate.
 *   start_event / stop_event as for mhc_stream_probe. Zero units launch
 *   nothing and record the events.
 */
mhc_status mhc_clock_probe(const void* src, int64_t src_bytes, void* dst, int64_t dst_bytes,
                           int32_t reads, int32_t writes, int32_t waves_per_block,
                           uint64_t* stamps, int64_t stamps_len, void* stream,
                           void* start_event, void* stop_event);

/* Rate of the wall clock the clock probe reads, in kHz, for the current device. */
mhc_status mhc_probe_wall_clock_khz(int32_t* khz);

#ifdef __cplusplus
}
#endif

#endif /* MHC_PROBES_H */
