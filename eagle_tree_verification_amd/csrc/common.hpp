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

// Where a sequence's logical cache row lives.  A contiguous cache (table ==
// nullptr) is [B][Hkv][L_cap][d]; a paged one is a pool of blocks
// [num_blocks][Hkv][block_size][d] with a [B][max_blocks] block table: row r
// of sequence b is row r % block_size of block table[b][r / block_size].
// block_size is a power of two; offsets are in units of `unit` (elements, or
// 16-byte chunks of a row).
struct KvRows {
  const int32_t* table;
  int max_blocks, bs_log2, num_blocks, Hkv, L_cap;

  __device__ __forceinline__ size_t offset(int b, int h, int r, int unit) const {
    if (!table) return (((size_t)b * Hkv + h) * L_cap + r) * unit;
    const int blk = table[(size_t)b * max_blocks + (r >> bs_log2)];
    return ((((size_t)blk * Hkv + h) << bs_log2) + (r & ((1 << bs_log2) - 1))) * unit;
  }

  // Every block holding rows [r0, r1) of sequence b exists (a contiguous
  // cache: always).  Called by every thread of the workgroup.
  __device__ bool blocks_ok(int b, int r0, int r1) const {
    int bad = 0;
    if (table && r1 > r0) {
      const int k0 = r0 >> bs_log2, k1 = (r1 - 1) >> bs_log2;
      for (int k = k0 + (int)threadIdx.x; k <= k1; k += (int)blockDim.x) {
        const int blk = table[(size_t)b * max_blocks + k];
        bad |= (blk < 0 || blk >= num_blocks);
      }
    }
    return !__syncthreads_or(bad);
  }
};

__host__ __device__ inline KvRows contiguous_rows(int Hkv, int L_cap) {
  return KvRows{nullptr, 0, 0, 0, Hkv, L_cap};
}

// Host checks of a paged cache's geometry: block_size a power of two in
// [16, 4096], max_blocks and num_blocks positive, the logical capacity and
// the pool's row count within 32-bit row indices.
inline spec_status_t make_paged_rows(const int32_t* table, int max_blocks, int block_size,
                                     int num_blocks, int Hkv, KvRows* kv) {
  if (block_size < 16 || block_size > 4096 || (block_size & (block_size - 1)) != 0 ||
      max_blocks <= 0 || num_blocks <= 0 || Hkv <= 0)
    return SPEC_E_SHAPE;
  if ((long)max_blocks * block_size >= (1L << 31) ||
      (long)num_blocks * Hkv * block_size >= (1L << 31))
    return SPEC_E_SHAPE;
  int lg = 0;
  while ((1 << lg) < block_size) ++lg;
  *kv = KvRows{table, max_blocks, lg, num_blocks, Hkv, max_blocks * block_size};
  return SPEC_OK;
}

// Host: compute units of the current device (cached per device ordinal).
int device_cu_count();

}  // namespace specv
