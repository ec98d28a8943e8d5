// The verify pass's write of the tree's K/V into the cache, with the rotary
// position embedding of the keys (gfx950).
//
// Tree node j's K/V go to cache row prefix_len + j (the layout
// spec_verify_tree_attn reads).  Its key is rotated at position prefix_len +
// depth(j): the draft candidates of one level share a position (page
// "EAGLE-1/2/3 拆解", the init_tree passage, where a level's position ids
// start as zeros), the root (depth 0) being the first position after the
// committed prefix.  The rotation is the published rotary embedding: plane i
// of the head dimension turns by pos * inv_freq[i]; planes pair dimension i
// with i + d/2, or 2i with 2i + 1.  Values are not rotated.
//
// The cache is contiguous, or paged (blocks of rows through a block table,
// KvRows); a sequence whose rows would land in a block outside the pool is
// not written and reports a capacity error.
//
// The work is a few MB per call (memory-bound, small).
#include <stdlib.h>

#include "common.hpp"

namespace specv {
namespace {

constexpr int NTW = 256;

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) {
  // round to nearest even (finite inputs; NaN stays NaN)
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// One plane pair (x, y) turned by the angle whose cosine and sine are (c, s).
// Both write kernels call this, so they round the same expressions.
__device__ __forceinline__ void rotate_pair(float x, float y, float c, float s, float* a,
                                            float* b) {
  *a = x * c - y * s;
  *b = y * c + x * s;
}

// One workgroup per (node, sequence).  Every workgroup of a sequence checks
// the whole tree (at most 64 parent walks) so that all of them agree on
// whether the sequence is written; the first one reports.
template <typename T>
__global__ __launch_bounds__(NTW) void tree_kv_write_kernel(
    const T* __restrict__ k_new, const T* __restrict__ v_new, T* __restrict__ kc,
    T* __restrict__ vc, const int32_t* __restrict__ prefix_len,
    const int32_t* __restrict__ n_nodes, const int32_t* __restrict__ parents, int n_max, int Hkv,
    int d, KvRows kv, const float* __restrict__ inv_freq, int style,
    int32_t* __restrict__ dev_error) {
  __shared__ int s_depth;
  __shared__ int s_bad;
  __shared__ int s_par[SPEC_MAX_NODES];
  const int j = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int n = n_nodes[b];
  const int L = prefix_len[b];
  const bool reporter = j == 0 && tid == 0;
  if (n < 1 || n > n_max) {
    if (reporter) report(dev_error, SPEC_DEVERR_TREE);
    return;
  }
  if (L < 0 || (int64_t)L + n > kv.L_cap) {
    if (reporter) report(dev_error, SPEC_DEVERR_CAPACITY);
    return;
  }
  if (tid == 0) s_bad = 0;
  if (tid < n) s_par[tid] = parents[(size_t)b * n_max + tid];
  __syncthreads();
  if (tid < n) {  // walk to the root in LDS: parents[x] < x, root -1
    int dep = 0, x = tid;
    bool bad = tid == 0 ? s_par[0] != -1 : false;
    while (!bad && x > 0) {
      const int p = s_par[x];
      if (p < 0 || p >= x) bad = true;
      else { x = p; ++dep; }
    }
    if (tid == j) s_depth = dep;
    if (bad) atomicOr(&s_bad, 1);
  }
  __syncthreads();
  if (s_bad) {
    if (reporter) report(dev_error, SPEC_DEVERR_TREE);
    return;
  }
  if (!kv.blocks_ok(b, L, L + n)) {
    if (reporter) report(dev_error, SPEC_DEVERR_CAPACITY);
    return;
  }
  if (j >= n) return;
  const int half = d / 2;
  const int pos = L + s_depth;
  // K: one thread per (head, plane)
  for (int e = tid; e < Hkv * half; e += NTW) {
    const int t = e % half;
    const int h = e / half;
    const T* src = k_new + (((size_t)b * n_max + j) * Hkv + h) * d;
    T* dst = kc + kv.offset(b, h, L + j, d);
    const int ia = style == kRopeInterleaved ? 2 * t : t;
    const int ib = style == kRopeInterleaved ? 2 * t + 1 : t + half;
    if (inv_freq) {
      float c, s, ra, rb;
      rope_cs(pos, inv_freq[t], &c, &s);
      rotate_pair(load_as_f32(src + ia), load_as_f32(src + ib), c, s, &ra, &rb);
      dst[ia] = from_f32<T>(ra);
      dst[ib] = from_f32<T>(rb);
    } else {
      dst[ia] = src[ia];
      dst[ib] = src[ib];
    }
  }
  // V: copied
  for (int e = tid; e < Hkv * d; e += NTW) {
    const int c = e % d;
    const int h = e / d;
    vc[kv.offset(b, h, L + j, d) + c] = v_new[(((size_t)b * n_max + j) * Hkv + h) * d + c];
  }
}

// bf16 caches with head_dim a multiple of 16 and 16-byte aligned buffers:
// the same write in 16-byte chunks (eight values per load and store).  The
// parent row is read together with the sequence's sizes, so a workgroup
// waits for one round trip before its tree check instead of two.
__device__ __forceinline__ void unpack8(const uint4& u, float* f) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ uint4 pack8(const float* f) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (uint32_t)from_f32<uint16_t>(f[2 * i]) | ((uint32_t)from_f32<uint16_t>(f[2 * i + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__global__ __launch_bounds__(NTW) void tree_kv_write_vec_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, const int32_t* __restrict__ prefix_len,
    const int32_t* __restrict__ n_nodes, const int32_t* __restrict__ parents, int n_max, int Hkv,
    int d, KvRows kv, const float* __restrict__ inv_freq, int style,
    int32_t* __restrict__ dev_error) {
  __shared__ int s_depth;
  __shared__ int s_bad;
  __shared__ int s_par[SPEC_MAX_NODES];
  const int j = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int n = n_nodes[b];
  const int L = prefix_len[b];
  const int par_t = tid < n_max ? parents[(size_t)b * n_max + tid] : -1;
  const bool reporter = j == 0 && tid == 0;
  if (n < 1 || n > n_max) {
    if (reporter) report(dev_error, SPEC_DEVERR_TREE);
    return;
  }
  if (L < 0 || (int64_t)L + n > kv.L_cap) {
    if (reporter) report(dev_error, SPEC_DEVERR_CAPACITY);
    return;
  }
  if (tid == 0) s_bad = 0;
  if (tid < n) s_par[tid] = par_t;
  __syncthreads();
  if (tid < n) {  // walk to the root in LDS: parents[x] < x, root -1
    int dep = 0, x = tid;
    bool bad = tid == 0 ? s_par[0] != -1 : false;
    while (!bad && x > 0) {
      const int p = s_par[x];
      if (p < 0 || p >= x) bad = true;
      else { x = p; ++dep; }
    }
    if (tid == j) s_depth = dep;
    if (bad) atomicOr(&s_bad, 1);
  }
  __syncthreads();
  if (s_bad) {
    if (reporter) report(dev_error, SPEC_DEVERR_TREE);
    return;
  }
  if (!kv.blocks_ok(b, L, L + n)) {
    if (reporter) report(dev_error, SPEC_DEVERR_CAPACITY);
    return;
  }
  if (j >= n) return;
  const int pos = L + s_depth;
  const int cpr = d / 8;  // 16-byte chunks per head row
  const size_t row = ((size_t)b * n_max + j) * Hkv;
  // V: copied chunk by chunk
  for (int e = tid; e < Hkv * cpr; e += NTW) {
    const int h = e / cpr, c = e % cpr;
    *reinterpret_cast<uint4*>(vc + kv.offset(b, h, L + j, d) + c * 8) =
        *reinterpret_cast<const uint4*>(v_new + (row + h) * d + c * 8);
  }
  if (!inv_freq) {
    for (int e = tid; e < Hkv * cpr; e += NTW) {
      const int h = e / cpr, c = e % cpr;
      *reinterpret_cast<uint4*>(kc + kv.offset(b, h, L + j, d) + c * 8) =
          *reinterpret_cast<const uint4*>(k_new + (row + h) * d + c * 8);
    }
  } else if (style == kRopeInterleaved) {
    // chunk c holds the planes 4c .. 4c + 3 as (2t, 2t + 1) pairs
    for (int e = tid; e < Hkv * cpr; e += NTW) {
      const int h = e / cpr, c = e % cpr;
      float f[8], r[8];
      unpack8(*reinterpret_cast<const uint4*>(k_new + (row + h) * d + c * 8), f);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        float cs, sn;
        rope_cs(pos, inv_freq[4 * c + p], &cs, &sn);
        rotate_pair(f[2 * p], f[2 * p + 1], cs, sn, &r[2 * p], &r[2 * p + 1]);
      }
      *reinterpret_cast<uint4*>(kc + kv.offset(b, h, L + j, d) + c * 8) = pack8(r);
    }
  } else {
    // chunk c of the first half (planes 8c .. 8c + 7) pairs with chunk
    // c + cpr / 2 of the second
    const int hc = cpr / 2;
    for (int e = tid; e < Hkv * hc; e += NTW) {
      const int h = e / hc, c = e % hc;
      const uint16_t* src = k_new + (row + h) * d + c * 8;
      uint16_t* dst = kc + kv.offset(b, h, L + j, d) + c * 8;
      float x[8], y[8], ra[8], rb[8];
      unpack8(*reinterpret_cast<const uint4*>(src), x);
      unpack8(*reinterpret_cast<const uint4*>(src + d / 2), y);
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        float cs, sn;
        rope_cs(pos, inv_freq[8 * c + p], &cs, &sn);
        rotate_pair(x[p], y[p], cs, sn, &ra[p], &rb[p]);
      }
      *reinterpret_cast<uint4*>(dst) = pack8(ra);
      *reinterpret_cast<uint4*>(dst + d / 2) = pack8(rb);
    }
  }
}

}  // namespace
}  // namespace specv

using namespace specv;

namespace specv {
namespace {

spec_status_t launch_kv_write(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              const int32_t* prefix_len, const int32_t* n_nodes,
                              const int32_t* parents, int32_t B, int32_t n_max, int32_t Hkv,
                              int32_t head_dim, int32_t dtype, const KvRows& kv,
                              const float* inv_freq, int32_t rope_style, int32_t* dev_error,
                              void* stream) {
  if (!k_new || !v_new || !k_cache || !v_cache || !prefix_len || !n_nodes || !parents)
    return SPEC_E_NULL;
  if (B <= 0 || B > 65535 || n_max <= 0 || n_max > SPEC_MAX_NODES || Hkv <= 0 ||
      kv.L_cap < n_max || (!kv.table && (long)B * Hkv * kv.L_cap >= (1L << 31)))
    return SPEC_E_SHAPE;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_E_DTYPE;
  if (head_dim < 2 || head_dim > 1024 || head_dim % 2) return SPEC_E_DTYPE;
  if (inv_freq && rope_style != kRopeHalf && rope_style != kRopeInterleaved) return SPEC_E_VALUE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // The chunked kernel needs bf16, head_dim a multiple of 16 (whole chunks,
  // and the half layout's planes paired chunk with chunk) and 16-byte
  // aligned buffers.  SPEC_KV_WRITE_SCALAR=1 selects the element-wise kernel
  // for comparisons; both write the same bits.
  const auto aligned = [](const void* p) { return ((uintptr_t)p & 15u) == 0; };
  bool vec_ok = dtype == SPEC_BF16 && head_dim % 16 == 0 && aligned(k_new) && aligned(v_new) &&
                aligned(k_cache) && aligned(v_cache);
  if (const char* env = getenv("SPEC_KV_WRITE_SCALAR")) vec_ok = vec_ok && env[0] != '1';
  if (dtype == SPEC_F32)
    hipLaunchKernelGGL(tree_kv_write_kernel<float>, dim3(n_max, B), dim3(NTW), 0, s,
                       static_cast<const float*>(k_new), static_cast<const float*>(v_new),
                       static_cast<float*>(k_cache), static_cast<float*>(v_cache), prefix_len,
                       n_nodes, parents, n_max, Hkv, head_dim, kv, inv_freq, rope_style,
                       dev_error);
  else if (vec_ok)
    hipLaunchKernelGGL(tree_kv_write_vec_kernel, dim3(n_max, B), dim3(NTW), 0, s,
                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                       static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
                       prefix_len, n_nodes, parents, n_max, Hkv, head_dim, kv, inv_freq,
                       rope_style, dev_error);
  else
    hipLaunchKernelGGL(tree_kv_write_kernel<uint16_t>, dim3(n_max, B), dim3(NTW), 0, s,
                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                       static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
                       prefix_len, n_nodes, parents, n_max, Hkv, head_dim, kv, inv_freq,
                       rope_style, dev_error);
  SPEC_HIP_TRY(hipGetLastError());
  return SPEC_OK;
}

}  // namespace
}  // namespace specv

extern "C" spec_status_t spec_tree_kv_write(const void* k_new, const void* v_new, void* k_cache,
                                            void* v_cache, const int32_t* prefix_len,
                                            const int32_t* n_nodes, const int32_t* parents,
                                            int32_t B, int32_t n_max, int32_t Hkv,
                                            int32_t head_dim, int32_t L_cap, int32_t dtype,
                                            const float* inv_freq, int32_t rope_style,
                                            int32_t* dev_error, void* stream) {
  if (L_cap <= 0) return SPEC_E_SHAPE;
  return launch_kv_write(k_new, v_new, k_cache, v_cache, prefix_len, n_nodes, parents, B, n_max,
                         Hkv, head_dim, dtype, contiguous_rows(Hkv, L_cap), inv_freq, rope_style,
                         dev_error, stream);
}

extern "C" spec_status_t spec_tree_kv_write_paged(
    const void* k_new, const void* v_new, void* k_pool, void* v_pool,
    const int32_t* block_table, int32_t max_blocks, int32_t block_size, int32_t num_blocks,
    const int32_t* prefix_len, const int32_t* n_nodes, const int32_t* parents, int32_t B,
    int32_t n_max, int32_t Hkv, int32_t head_dim, int32_t dtype, const float* inv_freq,
    int32_t rope_style, int32_t* dev_error, void* stream) {
  if (!block_table) return SPEC_E_NULL;
  KvRows kv;
  const spec_status_t st = make_paged_rows(block_table, max_blocks, block_size, num_blocks, Hkv,
                                           &kv);
  if (st != SPEC_OK) return st;
  return launch_kv_write(k_new, v_new, k_pool, v_pool, prefix_len, n_nodes, parents, B, n_max,
                         Hkv, head_dim, dtype, kv, inv_freq, rope_style, dev_error, stream);
}
