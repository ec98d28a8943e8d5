// Shared helpers of the HIP library: status handling, bf16 conversion, wave
// reductions and launch bookkeeping.  gfx950 (CDNA4, wave64) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spec_verify.h"

#define SPEC_HIP_TRY(expr)                          \
  do {                                              \
    hipError_t e_ = (expr);                         \
    if (e_ != hipSuccess) return SPEC_E_HIP;        \
  } while (0)

namespace specv {

constexpr int kWave = 64;

// bf16 <-> f32 (storage is raw 16-bit patterns; bf16 is the top half of f32).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ void report(int32_t* dev_error, int bits) {
  if (dev_error) atomicOr(dev_error, bits);
}

// Host: compute units of the current device (cached per device ordinal).
int device_cu_count();

}  // namespace specv
