// mhc_launch.h - host-side kernel launch shared by the library sources
// (internal; not part of the C ABI).
//
// Every kernel is launched through hipExtLaunchKernel, whose return value is
// the status of that launch alone. The libraries report that status and
// never read or clear the thread's last-error state, so an error a caller
// had pending before calling in is still there for the caller afterwards.
// The launch can carry two caller-owned HIP events that take the dispatch's
// own start and end timestamps (no marker packets between kernels).

#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <tuple>

namespace {

// Launch `kernel` with `args` converted to its parameter types (so the
// argument array matches its signature exactly), no dynamic LDS, on
// `stream`; `start` / `stop` may be null.
template <typename... Params, typename... Args>
hipError_t launch_kernel(void (*kernel)(Params...), dim3 grid, dim3 block, hipStream_t stream,
                         hipEvent_t start, hipEvent_t stop, Args... args) {
  static_assert(sizeof...(Params) == sizeof...(Args), "kernel argument count");
  std::tuple<Params...> values{static_cast<Params>(args)...};
  void* ptrs[sizeof...(Params) > 0 ? sizeof...(Params) : 1] = {};
  std::apply(
      [&ptrs](auto&... v) {
        int i = 0;
        ((ptrs[i++] = static_cast<void*>(&v)), ...);
      },
      values);
  return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0, stream,
                            start, stop, 0);
}

}  // namespace
