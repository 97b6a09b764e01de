// mhc_probes.hip - the measurement library (libmhc_probes.so): the bf16
// rounding probe, the streaming probe and the clock probe described in
// mhc_probes.h. Used by the tests and the benchmark only; it is not part of
// the operation.

#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "mhc_convert.h"
#include "mhc_lanes.h"
#include "mhc_launch.h"
#include "mhc_probes.h"

#if defined(__FAST_MATH__)
#error "mhc_probes must not be built with fast-math: the rounding probe is compared bit for bit"
#endif

#pragma clang fp contract(off)

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void bf16_probe_kernel(uint32_t first_bits, int64_t n,
                                                         uint16_t* __restrict__ out) {
  const int64_t k = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (k >= n) return;
  const uint32_t bits = first_bits + static_cast<uint32_t>(k);
  out[k] = to_bf16(__uint_as_float(bits));
}

constexpr int kProbeChunk = 1024;  // bytes per access instruction of a wave

// One 64-lane block per unit: R KiB read from src, W KiB written to dst.
// A read-only unit (W == 0) keeps its loads alive with an empty asm that
// takes the XOR of its vectors as an operand (so each load must complete);
// a write-only unit (R == 0) stores its unit index.
template <int R, int W, int POL>
__global__ __launch_bounds__(64) void stream_probe_kernel(const uint8_t* __restrict__ src,
                                                          uint8_t* __restrict__ dst) {
  const int64_t u = blockIdx.x;
  const uint32_t lane = threadIdx.x;
  u32x4 acc = {static_cast<uint32_t>(u), static_cast<uint32_t>(u), static_cast<uint32_t>(u),
               static_cast<uint32_t>(u)};
  if constexpr (R > 0) {
    const Rsrc rs = make_rsrc(src + u * (R * kProbeChunk), R * kProbeChunk);
    u32x4 x[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
      x[r] = __builtin_amdgcn_raw_buffer_load_b128(rs, r * kProbeChunk + lane * 16, 0,
                                                   kNontemporal);
    acc = x[0];
#pragma unroll
    for (int r = 1; r < R; ++r) acc ^= x[r];
  }
  if constexpr (W > 0) {
    const Rsrc rd = make_rsrc(dst + u * (W * kProbeChunk), W * kProbeChunk);
#pragma unroll
    for (int w = 0; w < W; ++w)
      __builtin_amdgcn_raw_buffer_store_b128(acc, rd, w * kProbeChunk + lane * 16, 0, POL);
  } else {
    __asm__ volatile("" : : "v"(acc));
  }
}

// s_getreg operands (size 32, offset 0): HW_ID (register 4) and XCC_ID
// (register 20, the XCD a wave runs on).
constexpr int kHwRegHwId = (31 << 11) | 4;
constexpr int kHwRegXccId = (31 << 11) | 20;

// The streaming probe's unit with `blockDim.x / 64` units per block and
// per-wave stamps: wall clock at the start, once the loads have returned and
// once the stores have completed, then the XCD and HW_ID (written by lane 0
// with vector stores).
template <int R, int W, int POL>
__global__ __launch_bounds__(1024) void clock_probe_kernel(const uint8_t* __restrict__ src,
                                                           uint8_t* __restrict__ dst,
                                                           int64_t units,
                                                           uint64_t* __restrict__ stamps) {
  const int64_t u =
      static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (u >= units) return;  // the whole wave
  const uint32_t lane = threadIdx.x & 63;
  const uint64_t t_start = wall_clock64();
  u32x4 acc = {static_cast<uint32_t>(u), static_cast<uint32_t>(u), static_cast<uint32_t>(u),
               static_cast<uint32_t>(u)};
  if constexpr (R > 0) {
    const Rsrc rs = make_rsrc(src + u * (R * kProbeChunk), R * kProbeChunk);
    u32x4 x[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
      x[r] = __builtin_amdgcn_raw_buffer_load_b128(rs, r * kProbeChunk + lane * 16, 0,
                                                   kNontemporal);
    acc = x[0];
#pragma unroll
    for (int r = 1; r < R; ++r) acc ^= x[r];
  }
  __asm__ volatile("s_waitcnt vmcnt(0)" : : "v"(acc) : "memory");
  const uint64_t t_loaded = wall_clock64();
  if constexpr (W > 0) {
    const Rsrc rd = make_rsrc(dst + u * (W * kProbeChunk), W * kProbeChunk);
#pragma unroll
    for (int w = 0; w < W; ++w)
      __builtin_amdgcn_raw_buffer_store_b128(acc, rd, w * kProbeChunk + lane * 16, 0, POL);
  }
  __asm__ volatile("s_waitcnt vmcnt(0)" : : : "memory");
  const uint64_t t_stored = wall_clock64();
  if (lane == 0) {
    const uint32_t xcc = __builtin_amdgcn_s_getreg(kHwRegXccId);
    const uint32_t hw = __builtin_amdgcn_s_getreg(kHwRegHwId);
    stamps[4 * u + 0] = t_start;
    stamps[4 * u + 1] = t_loaded;
    stamps[4 * u + 2] = t_stored;
    stamps[4 * u + 3] = (static_cast<uint64_t>(hw) << 32) | xcc;
  }
}

thread_local char g_msg[256] = "";

mhc_status fail(mhc_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
mhc_status fail(mhc_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return s;
}

mhc_status ok() {
  g_msg[0] = '\0';
  return MHC_SUCCESS;
}

mhc_status launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(MHC_ERROR_HIP, "%s launch failed: %s (%s)", what, hipGetErrorName(e),
                hipGetErrorString(e));
  return ok();
}

mhc_status aligned(const void* p, uintptr_t align, const char* name) {
  if (p == nullptr) return fail(MHC_ERROR_INVALID_VALUE, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % align != 0)
    return fail(MHC_ERROR_INVALID_VALUE, "%s is not %u-byte aligned", name,
                static_cast<unsigned>(align));
  return ok();
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range(const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}

bool overlaps(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

// Validates a streaming probe's buffers and mix and gives its unit count.
mhc_status probe_units(const void* src, int64_t src_bytes, const void* dst, int64_t dst_bytes,
                       int32_t reads, int32_t writes, int64_t* units_out) {
  const int mix = reads * 100 + writes;
  if (reads < 0 || writes < 0 ||
      (mix != 101 && mix != 401 && mix != 504 && mix != 904 && mix != 800 && mix != 8))
    return fail(MHC_ERROR_INVALID_VALUE,
                "reads:writes must be 1:1, 4:1, 5:4, 9:4, 8:0 or 0:8 (got %d:%d)", reads, writes);
  if (src_bytes < 0 || dst_bytes < 0)
    return fail(MHC_ERROR_INVALID_VALUE, "byte counts must be non-negative");
  int64_t units;
  if (reads > 0) {
    if (src_bytes % (int64_t(reads) * kProbeChunk) != 0)
      return fail(MHC_ERROR_INVALID_VALUE,
                  "src_bytes must be a multiple of reads KiB (got %lld)", (long long)src_bytes);
    units = src_bytes / (int64_t(reads) * kProbeChunk);
    if (dst_bytes != units * writes * kProbeChunk)
      return fail(MHC_ERROR_INVALID_VALUE,
                  "dst_bytes must be writes KiB per unit of src (want %lld, got %lld)",
                  (long long)(units * writes * kProbeChunk), (long long)dst_bytes);
  } else {
    if (src_bytes != 0)
      return fail(MHC_ERROR_INVALID_VALUE, "a write-only probe reads nothing (src_bytes %lld)",
                  (long long)src_bytes);
    if (dst_bytes % (int64_t(writes) * kProbeChunk) != 0)
      return fail(MHC_ERROR_INVALID_VALUE,
                  "dst_bytes must be a multiple of writes KiB (got %lld)", (long long)dst_bytes);
    units = dst_bytes / (int64_t(writes) * kProbeChunk);
  }
  if (units > 0x7FFFFFFF)
    return fail(MHC_ERROR_INVALID_VALUE, "too many units (%lld)", (long long)units);
  mhc_status st;
  if (units > 0) {
    if (reads > 0 && (st = aligned(src, 16, "src")) != MHC_SUCCESS) return st;
    if (writes > 0 && (st = aligned(dst, 16, "dst")) != MHC_SUCCESS) return st;
    if (reads > 0 && writes > 0 && overlaps(range(src, src_bytes), range(dst, dst_bytes)))
      return fail(MHC_ERROR_ALIASING, "dst overlaps src");
  }
  *units_out = units;
  return ok();
}

// Zero units: nothing to launch, the events are still recorded.
mhc_status record_only(hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  if (start && hipEventRecord(start, s) != hipSuccess)
    return fail(MHC_ERROR_HIP, "hipEventRecord(start) failed");
  if (stop && hipEventRecord(stop, s) != hipSuccess)
    return fail(MHC_ERROR_HIP, "hipEventRecord(stop) failed");
  return ok();
}

}  // namespace

extern "C" {

int mhc_probe_abi_version(void) { return MHC_PROBE_ABI_VERSION; }

const char* mhc_probe_last_error_message(void) { return g_msg; }

mhc_status mhc_bf16_rne_probe(uint32_t first_bits, int64_t n, uint16_t* out, void* stream) {
  if (n < 0 || n > (int64_t(1) << 32))
    return fail(MHC_ERROR_INVALID_VALUE, "n must be in [0, 2^32]");
  if (n == 0) return ok();
  mhc_status st = aligned(out, 2, "out");
  if (st != MHC_SUCCESS) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t per_launch = int64_t(1) << 30;  // work-items per dispatch
  for (int64_t k0 = 0; k0 < n; k0 += per_launch) {
    const int64_t m = (n - k0 < per_launch) ? n - k0 : per_launch;
    const uint32_t blocks = static_cast<uint32_t>((m + 255) / 256);
    const hipError_t e = launch_kernel(bf16_probe_kernel, dim3(blocks), dim3(256), s, nullptr,
                                       nullptr, first_bits + static_cast<uint32_t>(k0), m,
                                       out + k0);
    if ((st = launch_status(e, "bf16 probe")) != MHC_SUCCESS) return st;
  }
  return ok();
}

mhc_status mhc_stream_probe(const void* src, int64_t src_bytes, void* dst, int64_t dst_bytes,
                            int32_t reads, int32_t writes, void* stream, void* start_event,
                            void* stop_event) {
  int64_t units;
  mhc_status st = probe_units(src, src_bytes, dst, dst_bytes, reads, writes, &units);
  if (st != MHC_SUCCESS) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipEvent_t start = static_cast<hipEvent_t>(start_event);
  const hipEvent_t stop = static_cast<hipEvent_t>(stop_event);
  if (units == 0) return record_only(s, start, stop);
  const dim3 grid(static_cast<uint32_t>(units));
  const auto* sp = static_cast<const uint8_t*>(src);
  auto* dp = static_cast<uint8_t*>(dst);
  hipError_t e;
  switch (reads * 100 + writes) {
    case 101: e = launch_kernel(stream_probe_kernel<1, 1, kNontemporal>, grid, dim3(64), s, start, stop, sp, dp); break;
    case 401: e = launch_kernel(stream_probe_kernel<4, 1, kWriteThrough>, grid, dim3(64), s, start, stop, sp, dp); break;
    case 504: e = launch_kernel(stream_probe_kernel<5, 4, kNontemporal>, grid, dim3(64), s, start, stop, sp, dp); break;
    case 904: e = launch_kernel(stream_probe_kernel<9, 4, kNontemporal>, grid, dim3(64), s, start, stop, sp, dp); break;
    case 800: e = launch_kernel(stream_probe_kernel<8, 0, kNontemporal>, grid, dim3(64), s, start, stop, sp, dp); break;
    default: e = launch_kernel(stream_probe_kernel<0, 8, kNontemporal>, grid, dim3(64), s, start, stop, sp, dp); break;
  }
  return launch_status(e, "stream probe");
}

mhc_status mhc_clock_probe(const void* src, int64_t src_bytes, void* dst, int64_t dst_bytes,
                           int32_t reads, int32_t writes, int32_t waves_per_block,
                           uint64_t* stamps, int64_t stamps_len, void* stream,
                           void* start_event, void* stop_event) {
  if (waves_per_block != 1 && waves_per_block != 4 && waves_per_block != 16)
    return fail(MHC_ERROR_INVALID_VALUE, "waves_per_block must be 1, 4 or 16 (got %d)",
                waves_per_block);
  int64_t units;
  mhc_status st = probe_units(src, src_bytes, dst, dst_bytes, reads, writes, &units);
  if (st != MHC_SUCCESS) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipEvent_t start = static_cast<hipEvent_t>(start_event);
  const hipEvent_t stop = static_cast<hipEvent_t>(stop_event);
  if (units == 0) return record_only(s, start, stop);
  if (stamps_len < 4 * units)
    return fail(MHC_ERROR_INVALID_VALUE, "stamps holds %lld values, %lld needed",
                (long long)stamps_len, (long long)(4 * units));
  if ((st = aligned(stamps, 8, "stamps")) != MHC_SUCCESS) return st;
  const Range rs = range(stamps, 32 * units);
  if ((reads > 0 && overlaps(rs, range(src, src_bytes))) ||
      (writes > 0 && overlaps(rs, range(dst, dst_bytes))))
    return fail(MHC_ERROR_ALIASING, "stamps overlap src or dst");
  const dim3 grid(static_cast<uint32_t>((units + waves_per_block - 1) / waves_per_block));
  const dim3 block(64 * waves_per_block);
  const auto* sp = static_cast<const uint8_t*>(src);
  auto* dp = static_cast<uint8_t*>(dst);
  hipError_t e;
  switch (reads * 100 + writes) {
    case 101: e = launch_kernel(clock_probe_kernel<1, 1, kNontemporal>, grid, block, s, start, stop, sp, dp, units, stamps); break;
    case 401: e = launch_kernel(clock_probe_kernel<4, 1, kWriteThrough>, grid, block, s, start, stop, sp, dp, units, stamps); break;
    case 504: e = launch_kernel(clock_probe_kernel<5, 4, kNontemporal>, grid, block, s, start, stop, sp, dp, units, stamps); break;
    case 904: e = launch_kernel(clock_probe_kernel<9, 4, kNontemporal>, grid, block, s, start, stop, sp, dp, units, stamps); break;
    case 800: e = launch_kernel(clock_probe_kernel<8, 0, kNontemporal>, grid, block, s, start, stop, sp, dp, units, stamps); break;
    default: e = launch_kernel(clock_probe_kernel<0, 8, kNontemporal>, grid, block, s, start, stop, sp, dp, units, stamps); break;
  }
  return launch_status(e, "clock probe");
}

mhc_status mhc_probe_wall_clock_khz(int32_t* khz) {
  if (khz == nullptr) return fail(MHC_ERROR_INVALID_VALUE, "khz is NULL");
  int dev = 0, rate = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&rate, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess)
    return fail(MHC_ERROR_HIP, "wall clock rate: %s (%s)", hipGetErrorName(e),
                hipGetErrorString(e));
  *khz = rate;
  return ok();
}

}  // extern "C"
