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

// Rotary embedding: cosine and sine of pos * f.  The angle is formed and
// reduced to [-1/2, 1/2] revolutions in float64, so a position in the
// millions keeps float32 accuracy; the hardware sine and cosine
// (v_sin_f32 / v_cos_f32, which take revolutions) finish it.
__device__ __forceinline__ void rope_cs(int pos, float f, float* c, float* s) {
  constexpr double kInvTwoPi = 0.15915494309189533576888376337251;
  double r = (double)pos * (double)f * kInvTwoPi;
  r -= rint(r);
  const float rf = (float)r;
  *s = __builtin_amdgcn_sinf(rf);
  *c = __builtin_amdgcn_cosf(rf);
}

// Rotary pair layouts: 1 = dimension i with i + d/2, 2 = dimension 2i with 2i + 1.
constexpr int kRopeHalf = 1;
constexpr int kRopeInterleaved = 2;

__device__ __forceinline__ void report(int32_t* dev_error, int bits) {
  if (dev_error) atomicOr(dev_error, bits);
}

// Host: compute units of the current device (cached per device ordinal).
int device_cu_count();

}  // namespace specv
