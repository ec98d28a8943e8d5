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
      float c, s;
      rope_cs(pos, inv_freq[t], &c, &s);
      const float x = load_as_f32(src + ia), y = load_as_f32(src + ib);
      dst[ia] = from_f32<T>(x * c - y * s);
      dst[ib] = from_f32<T>(y * c + x * s);
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
  if (dtype == SPEC_F32)
    hipLaunchKernelGGL(tree_kv_write_kernel<float>, dim3(n_max, B), dim3(NTW), 0, s,
                       static_cast<const float*>(k_new), static_cast<const float*>(v_new),
                       static_cast<float*>(k_cache), static_cast<float*>(v_cache), prefix_len,
                       n_nodes, parents, n_max, Hkv, head_dim, kv, inv_freq, rope_style,
                       dev_error);
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
