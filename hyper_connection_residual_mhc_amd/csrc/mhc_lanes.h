// mhc_lanes.h - device helpers shared by the library's kernel sources
// (internal; not part of the C ABI).
//
//  * Buffer resources: a base address and a byte length in scalar registers.
//    Loads past the length return 0 and stores past it are dropped by the
//    hardware, so a lane can never touch memory outside the range it was
//    given, and kernels need no bounds branches.
//  * from_lane_plus<OFF>: register-only lane movement for the halving trees
//    (offsets 32, 16, 8, 4, 2, 1) that every fixed-order sum here ends with.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcFormat = 0x00020000;  // gfx9 resource word 3: raw 32-bit data

__device__ __forceinline__ Rsrc make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kRsrcFormat);
}

// Cache-policy bits of a buffer access (the `aux` operand).
constexpr int kNontemporal = 2;   // bit 1, nt: streamed bytes, touched once
constexpr int kCached = 0;        // default policy: kept for other readers
constexpr int kWriteThrough = 16; // bit 4, sc1: device-scope store, written through the L2

// Lane j (< OFF) of a wave receives x from lane j + OFF; other lanes receive
// values that are never read. On gfx950: permlane32_swap brings the upper
// half-wave down, permlane16_swap the odd 16-lane rows onto the even ones,
// and DPP row_shl:n reads lane j + n within a 16-lane row. The whole wave
// must be active.
template <int OFF>
__device__ __forceinline__ float from_lane_plus(float x) {
  const uint32_t u = __float_as_uint(x);
  if constexpr (OFF == 32) {
    return __uint_as_float(__builtin_amdgcn_permlane32_swap(u, u, false, false)[1]);
  } else if constexpr (OFF == 16) {
    return __uint_as_float(__builtin_amdgcn_permlane16_swap(u, u, false, false)[1]);
  } else {
    static_assert(OFF == 8 || OFF == 4 || OFF == 2 || OFF == 1, "row shift within 16 lanes");
    return __int_as_float(__builtin_amdgcn_update_dpp(0, static_cast<int>(u), 0x100 + OFF, 0xF,
                                                      0xF, false));
  }
}

}  // namespace
