// mhc_convert.h - the device's 16-bit conversions (internal; not part of
// the C ABI). Every bf16 result of the h_aggregate kernels is rounded by
// pack_bf16x2, and the rounding probe of the measurement library runs the
// same routine, so that tests can pin it over all 2^32 fp32 patterns; the
// coefficient epilogue's 16-bit forms use these routines for their inputs
// and grad_mix.
//
//  * widening is exact: a bf16 pattern is the top half of an fp32 pattern,
//    and every fp16 value is an fp32 value (v_cvt_f32_f16);
//  * narrowing rounds to nearest even: bf16 with gfx950's
//    v_cvt_pk_bf16_f32 (two values per instruction), fp16 with v_cvt_f16_f32
//    under the default round-to-nearest-even mode; denormals kept (the
//    kernels' default fp16/fp64 and fp32 denormal modes), overflow to
//    infinity.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values -> two bf16 patterns packed low|high in one dword, rounded
// to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  return static_cast<uint16_t>(pack_bf16x2(x, 0.0f));
}

// bf16 pattern(s) -> fp32, exact.
__device__ __forceinline__ float lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp16 bit pattern -> fp32, exact; fp32 -> fp16 bit pattern, nearest even.
__device__ __forceinline__ float f16_f32(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}
__device__ __forceinline__ uint16_t to_f16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

}  // namespace
