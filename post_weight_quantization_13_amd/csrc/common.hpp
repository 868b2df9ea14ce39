// Shared device-side definitions for the gfx950 GPTQ kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gptq {

// ---------------------------------------------------------------- vector types
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(double)))) double f64x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// Element type tags matching gptq_dtype.
enum : int { DT_BF16 = 0, DT_FP16 = 1, DT_FP32 = 2 };

// ---------------------------------------------------------------- scalar loads
__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
  _Float16 h;
  __builtin_memcpy(&h, &b, 2);
  return static_cast<float>(h);
}

template <int DT>
__device__ __forceinline__ float load_as_float(const void* p, int64_t idx) {
  if constexpr (DT == DT_BF16) {
    return bf16_bits_to_float(static_cast<const uint16_t*>(p)[idx]);
  } else if constexpr (DT == DT_FP16) {
    return half_bits_to_float(static_cast<const uint16_t*>(p)[idx]);
  } else {
    return static_cast<const float*>(p)[idx];
  }
}

// fp32 -> fp16 bit pattern, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t float_to_half_bits(float x) {
  _Float16 h = static_cast<_Float16>(x);
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace gptq
