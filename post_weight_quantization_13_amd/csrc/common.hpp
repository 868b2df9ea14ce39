// Shared device-side definitions for the gfx950 GPTQ kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

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

// Barrier for exchanges through LDS only: waits for this wave's LDS accesses,
// not for its global loads, which may stay in flight across it (operands
// prefetched into registers several steps ahead).  The memory clobber keeps
// the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Zero `words` 8-byte words at p.  A kernel rather than hipMemsetAsync, so the
// clearing also replays correctly when a caller captures the stream in a graph.
static __global__ void zero_words_kernel(uint64_t* __restrict__ p, size_t words) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < words;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = 0;
}

static inline hipError_t zero_words(void* p, size_t words, hipStream_t s) {
  if (words == 0) return hipSuccess;
  size_t blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_words_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<uint64_t*>(p), words);
  return hipGetLastError();
}

// Zero one int32 (a status flag that may sit in a caller's 4-byte buffer).
static __global__ void zero_i32_kernel(int32_t* __restrict__ p) { p[0] = 0; }

static inline hipError_t zero_i32(int32_t* p, hipStream_t s) {
  hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(1), 0, s, p);
  return hipGetLastError();
}

// Extra streams per device (which = 0, 1) for work that overlaps the
// caller's stream, created on first use and kept until the process ends.
// Calls may share them; each call orders its own work with its own events.
static inline hipError_t side_stream(hipStream_t* out, int which = 0) {
  static std::mutex mu;
  static hipStream_t streams[64][2] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64 || which < 0 || which > 1) return hipErrorInvalidValue;
  std::lock_guard<std::mutex> lock(mu);
  if (!streams[dev][which]) {
    e = hipStreamCreateWithFlags(&streams[dev][which], hipStreamNonBlocking);
    if (e != hipSuccess) {
      streams[dev][which] = nullptr;
      return e;
    }
  }
  *out = streams[dev][which];
  return hipSuccess;
}

// A pair of timing-free events, destroyed with the object.
struct EventPair {
  hipEvent_t fork = nullptr, join = nullptr;
  hipError_t create() {
    hipError_t e = hipEventCreateWithFlags(&fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&join, hipEventDisableTiming);
    return e;
  }
  ~EventPair() {
    if (fork) (void)hipEventDestroy(fork);
    if (join) (void)hipEventDestroy(join);
  }
};

}  // namespace gptq
