// KV commit of the accepted path (gfx950).
//
// Rollback keeps a physical cache and a logical length, or writes to scratch
// and commits on acceptance (page "推测解码与 EAGLE-3", section "KV cache
// 回滚"; build step 4 sets the logical length to prefix + accepted + 1).
//
// In place: the tree's K/V rows sit at prefix_len + node, so the accepted
// path (root plus a accepted drafts, node ids increasing along the path) is
// gathered to rows prefix_len + 0..a and the length advances by a + 1.  A
// chain-shaped path (path[i] == i) moves nothing.  Moves are in place and
// path[i] >= i, so a row can be both read and written (path [0, 2, 5]: row 2
// is read for slot 1 and written by slot 2): a workgroup loads every row it
// moves for its sequence and layer (all KV heads, K and V) into registers,
// waits at a barrier, then stores.  Moves that do not fit one round are done
// in rounds of increasing slot within each (head, K/V) plane; a later round
// reads only rows path[s] >= s beyond every row an earlier round wrote, so
// rounds never see each other's writes.
//
// From scratch: the verify pass wrote the tree's K/V to a separate buffer;
// cache rows prefix_len + 0..a receive scratch rows path[0..a] (no overlap, a
// plain gather).
//
// Paged caches (spec_kv_commit_layers_paged): the same moves on logical rows,
// each row found through the sequence's block table (KvRows).  A sequence
// whose rows would come from or go to a block outside the pool is left
// untouched and reports a capacity error.
//
// Lengths: spec_kv_commit has one workgroup per sequence, which also owns the
// sequence's length.  spec_kv_commit_layers has one workgroup per (sequence,
// layer), all of which read the length, so the lengths advance in a second,
// stream-ordered kernel.
#include "common.hpp"

namespace specv {
namespace {

constexpr int NT = 1024;       // spec_kv_commit: one workgroup per sequence
constexpr int NTL = 256;       // spec_kv_commit_layers: one per (sequence, layer)
constexpr int CPT = 16;        // 16-byte chunks per thread per round

// Loads sequence b's path into s_path and checks it: a <= max_depth, the
// committed rows fit (prefix + a + 1 <= L_cap), path[0] == 0, strictly
// increasing (so path[i] >= i), and every source row exists (prefix +
// path[i] < L_cap in place, n_rows == 0; path[i] < n_rows from scratch), and
// every block holding a row read or written exists.  Returns 0 or
// SPEC_DEVERR_* bits; *s_moves says whether the in-place form moves
// anything.  Called by every thread of the workgroup, a >= 0, blockDim.x > a.
__device__ int load_path(const int32_t* path, int b, int a, int L, const KvRows& kv,
                         int max_depth, int n_rows, int* s_path, int* s_moves) {
  const int L_cap = kv.L_cap;
  if (a > max_depth) return SPEC_DEVERR_TREE;
  if (L < 0 || (int64_t)L + a + 1 > L_cap) return SPEC_DEVERR_CAPACITY;
  const int tid = threadIdx.x;
  if (tid == 0) *s_moves = 0;
  __syncthreads();
  int bad = 0;
  if (tid <= a) {
    const int p = path[(size_t)b * (max_depth + 1) + tid];
    s_path[tid] = p;
    if (tid == 0) bad = (p != 0);
    if (p != tid) atomicOr(s_moves, 1);
    if (p < tid || (n_rows > 0 ? p >= n_rows : (int64_t)L + p >= L_cap)) bad = 1;
  }
  __syncthreads();
  if (tid > 0 && tid <= a && s_path[tid] <= s_path[tid - 1]) bad = 1;
  if (__syncthreads_or(bad)) return SPEC_DEVERR_TREE;
  // rows written: L .. L + a; rows read in place: up to L + path[a]
  const int hi = L + 1 + (n_rows > 0 ? a : s_path[a]);
  return kv.blocks_ok(b, L, hi) ? 0 : SPEC_DEVERR_CAPACITY;
}

// In-place gather of rows 1..a of every (head, K/V) plane of sequence b in
// one layer's cache kc, vc (rows located by kv, in 16-byte chunks).  Every
// thread of the workgroup calls it.
template <int NTH>
__device__ void move_in_place(uint4* kc, uint4* vc, const KvRows& kv, int b, int Hkv,
                              int row_chunks, int L, int a, const int* s_path) {
  // chunk c = ((g * 2 + kv) * a + slot - 1) * row_chunks + cc (row 0, the
  // root, is already in place)
  const int plane_chunks = a * row_chunks;
  const int total = Hkv * 2 * plane_chunks;
  auto offset = [&](int c, bool src, int* pl_out) -> size_t {
    const int pl = c / plane_chunks;
    const int rem = c - pl * plane_chunks;
    const int slot = 1 + rem / row_chunks;
    const int cc = rem - (slot - 1) * row_chunks;
    *pl_out = pl;
    const int row = src ? s_path[slot] : slot;
    return kv.offset(b, pl >> 1, L + row, row_chunks) + cc;
  };
  for (int r0 = 0; r0 < total; r0 += NTH * CPT) {
    uint4 regs[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = r0 + j * NTH + (int)threadIdx.x;
      int pl = 0;
      const size_t off = c < total ? offset(c, true, &pl) : 0;
      const uint4* src = (pl & 1) ? vc : kc;
      regs[j] = c < total ? src[off] : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = r0 + j * NTH + (int)threadIdx.x;
      if (c < total) {
        int pl = 0;
        const size_t off = offset(c, false, &pl);
        ((pl & 1) ? vc : kc)[off] = regs[j];
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(NT) void commit_kernel(uint4* kc, uint4* vc, int32_t* prefix_len,
                                                    const int32_t* path, const int32_t* accept_len,
                                                    int Hkv, int row_chunks, int L_cap,
                                                    int max_depth, int32_t* dev_error) {
  __shared__ int s_path[SPEC_MAX_NODES + 1];
  __shared__ int s_moves;
  const int b = blockIdx.x;
  const int a = accept_len[b];
  const int L = prefix_len[b];
  if (a < 0) return;
  const KvRows kv = contiguous_rows(Hkv, L_cap);
  const int err = load_path(path, b, a, L, kv, max_depth, 0, s_path, &s_moves);
  if (err) {
    if (threadIdx.x == 0) report(dev_error, err);
    return;
  }
  if (s_moves) move_in_place<NT>(kc, vc, kv, b, Hkv, row_chunks, L, a, s_path);
  if (threadIdx.x == 0) prefix_len[b] = L + a + 1;
}

// Whether any layer buffer of the call (cache, and scratch rows when given)
// is off the 16-byte alignment the chunked moves need.  The pointer arrays
// live on the device, so every workgroup checks all layers: then either every
// layer is committed or none is.  Called by every thread of the workgroup.
__device__ bool layers_misaligned(const uint4* const* kl, const uint4* const* vl,
                                  const uint4* const* kt, const uint4* const* vt,
                                  int num_layers) {
  uintptr_t bits = 0;
  for (int l = threadIdx.x; l < num_layers; l += blockDim.x) {
    bits |= reinterpret_cast<uintptr_t>(kl[l]) | reinterpret_cast<uintptr_t>(vl[l]);
    if (kt != nullptr)
      bits |= reinterpret_cast<uintptr_t>(kt[l]) | reinterpret_cast<uintptr_t>(vt[l]);
  }
  return __syncthreads_or((bits & 15) != 0);
}

// One workgroup per (sequence, layer): the in-place gather, or the gather
// from the layer's scratch rows (kt != nullptr).  Only the layer-0 workgroup
// reports a failed sequence; the length kernel skips it.
__global__ __launch_bounds__(NTL) void commit_layers_kernel(
    uint4* const* kl, uint4* const* vl, const uint4* const* kt, const uint4* const* vt,
    const int32_t* prefix_len, const int32_t* path, const int32_t* accept_len, int Hkv,
    int row_chunks, KvRows kv, int n_rows, int max_depth, int32_t* dev_error) {
  __shared__ int s_path[SPEC_MAX_NODES + 1];
  __shared__ int s_moves;
  const int b = blockIdx.x;
  const int layer = blockIdx.y;
  const int a = accept_len[b];
  const int L = prefix_len[b];
  if (a < 0) return;
  if (layers_misaligned(kl, vl, kt, vt, (int)gridDim.y)) {
    if (layer == 0 && threadIdx.x == 0) report(dev_error, SPEC_DEVERR_ALIGN);
    return;
  }
  const bool scratch = (kt != nullptr);
  const int err = load_path(path, b, a, L, kv, max_depth, scratch ? n_rows : 0, s_path, &s_moves);
  if (err) {
    if (layer == 0 && threadIdx.x == 0) report(dev_error, err);
    return;
  }
  uint4* kc = kl[layer];
  uint4* vc = vl[layer];
  if (!scratch) {
    if (s_moves) move_in_place<NTL>(kc, vc, kv, b, Hkv, row_chunks, L, a, s_path);
    return;
  }
  // from scratch: chunk c = ((g * 2 + kv) * (a + 1) + slot) * row_chunks + cc
  const size_t tree_stride = (size_t)n_rows * row_chunks;
  const uint4* ks = kt[layer] + (size_t)b * Hkv * tree_stride;
  const uint4* vs = vt[layer] + (size_t)b * Hkv * tree_stride;
  const int plane_chunks = (a + 1) * row_chunks;
  const int total = Hkv * 2 * plane_chunks;
  for (int c = threadIdx.x; c < total; c += NTL) {
    const int pl = c / plane_chunks;
    const int rem = c - pl * plane_chunks;
    const int slot = rem / row_chunks;
    const int cc = rem - slot * row_chunks;
    const size_t g = (size_t)(pl >> 1);
    const uint4 x = ((pl & 1) ? vs : ks)[g * tree_stride + (size_t)s_path[slot] * row_chunks + cc];
    ((pl & 1) ? vc : kc)[kv.offset(b, (int)g, L + slot, row_chunks) + cc] = x;
  }
}

// Advances the length of every sequence the copy kernel committed.
__global__ __launch_bounds__(64) void commit_length_kernel(
    int32_t* prefix_len, const int32_t* path, const int32_t* accept_len, KvRows kv, int n_rows,
    int max_depth, const uint4* const* kl, const uint4* const* vl, const uint4* const* kt,
    const uint4* const* vt, int num_layers) {
  __shared__ int s_path[SPEC_MAX_NODES + 1];
  __shared__ int s_moves;
  const int b = blockIdx.x;
  const int a = accept_len[b];
  const int L = prefix_len[b];
  if (a < 0) return;
  if (layers_misaligned(kl, vl, kt, vt, num_layers)) return;
  if (load_path(path, b, a, L, kv, max_depth, n_rows, s_path, &s_moves)) return;
  if (threadIdx.x == 0) prefix_len[b] = L + a + 1;
}

spec_status_t check_commit_shape(int B, int Hkv, int head_dim, int L_cap, int max_depth,
                                 int dtype) {
  if (B <= 0 || Hkv <= 0 || L_cap <= 0 || max_depth < 0 || max_depth >= SPEC_MAX_NODES)
    return SPEC_E_SHAPE;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_E_DTYPE;
  if (head_dim != 16 && head_dim != 32 && head_dim != 64 && head_dim != 128) return SPEC_E_DTYPE;
  // chunk counts per (sequence, layer) and grid sizes are 32-bit
  if ((long)Hkv * 2 * (max_depth + 1) * 32 >= (1L << 31)) return SPEC_E_SHAPE;
  return SPEC_OK;
}

}  // namespace
}  // namespace specv

using namespace specv;

extern "C" spec_status_t spec_kv_commit(void* k_cache, void* v_cache, int32_t* prefix_len,
                                        const int32_t* path, const int32_t* accept_len, int32_t B,
                                        int32_t Hkv, int32_t head_dim, int32_t L_cap,
                                        int32_t max_depth, int32_t dtype, int32_t* dev_error,
                                        void* stream) {
  if (!k_cache || !v_cache || !prefix_len || !path || !accept_len) return SPEC_E_NULL;
  const spec_status_t st = check_commit_shape(B, Hkv, head_dim, L_cap, max_depth, dtype);
  if (st != SPEC_OK) return st;
  // rows move in 16-byte chunks
  if (((reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) & 15) != 0)
    return SPEC_E_SHAPE;
  const int esz = dtype == SPEC_F32 ? 4 : 2;
  const int row_chunks = head_dim * esz / 16;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(commit_kernel, dim3(B), dim3(NT), 0, strm, static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache), prefix_len, path, accept_len, Hkv, row_chunks,
                     L_cap, max_depth, dev_error);
  SPEC_HIP_TRY(hipGetLastError());
  return SPEC_OK;
}

namespace specv {
namespace {

spec_status_t launch_commit_layers(void* const* k_layers, void* const* v_layers,
                                   const void* const* k_tree, const void* const* v_tree,
                                   int32_t num_layers, int32_t* prefix_len, const int32_t* path,
                                   const int32_t* accept_len, int32_t B, int32_t n_max,
                                   int32_t Hkv, int32_t head_dim, const KvRows& kv,
                                   int32_t max_depth, int32_t dtype, int32_t* dev_error,
                                   void* stream) {
  if (!k_layers || !v_layers || !prefix_len || !path || !accept_len) return SPEC_E_NULL;
  if ((k_tree == nullptr) != (v_tree == nullptr)) return SPEC_E_NULL;
  if (num_layers <= 0 || num_layers > 65535) return SPEC_E_SHAPE;
  const bool scratch = (k_tree != nullptr);
  if (scratch && (n_max <= 0 || n_max > SPEC_MAX_NODES)) return SPEC_E_SHAPE;
  const spec_status_t st = check_commit_shape(B, Hkv, head_dim, kv.L_cap, max_depth, dtype);
  if (st != SPEC_OK) return st;
  const int esz = dtype == SPEC_F32 ? 4 : 2;
  const int row_chunks = head_dim * esz / 16;
  const int n_rows = scratch ? n_max : 0;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(commit_layers_kernel, dim3(B, num_layers), dim3(NTL), 0, strm,
                     reinterpret_cast<uint4* const*>(k_layers),
                     reinterpret_cast<uint4* const*>(v_layers),
                     reinterpret_cast<const uint4* const*>(k_tree),
                     reinterpret_cast<const uint4* const*>(v_tree), prefix_len, path, accept_len,
                     Hkv, row_chunks, kv, n_rows, max_depth, dev_error);
  SPEC_HIP_TRY(hipGetLastError());
  hipLaunchKernelGGL(commit_length_kernel, dim3(B), dim3(64), 0, strm, prefix_len, path,
                     accept_len, kv, n_rows, max_depth,
                     reinterpret_cast<const uint4* const*>(k_layers),
                     reinterpret_cast<const uint4* const*>(v_layers),
                     reinterpret_cast<const uint4* const*>(k_tree),
                     reinterpret_cast<const uint4* const*>(v_tree), num_layers);
  SPEC_HIP_TRY(hipGetLastError());
  return SPEC_OK;
}

}  // namespace
}  // namespace specv

extern "C" spec_status_t spec_kv_commit_layers(
    void* const* k_layers, void* const* v_layers, const void* const* k_tree,
    const void* const* v_tree, int32_t num_layers, int32_t* prefix_len, const int32_t* path,
    const int32_t* accept_len, int32_t B, int32_t n_max, int32_t Hkv, int32_t head_dim,
    int32_t L_cap, int32_t max_depth, int32_t dtype, int32_t* dev_error, void* stream) {
  if (L_cap <= 0) return SPEC_E_SHAPE;
  return launch_commit_layers(k_layers, v_layers, k_tree, v_tree, num_layers, prefix_len, path,
                              accept_len, B, n_max, Hkv, head_dim, contiguous_rows(Hkv, L_cap),
                              max_depth, dtype, dev_error, stream);
}

extern "C" spec_status_t spec_kv_commit_layers_paged(
    void* const* k_layers, void* const* v_layers, const void* const* k_tree,
    const void* const* v_tree, int32_t num_layers, const int32_t* block_table,
    int32_t max_blocks, int32_t block_size, int32_t num_blocks, int32_t* prefix_len,
    const int32_t* path, const int32_t* accept_len, int32_t B, int32_t n_max, int32_t Hkv,
    int32_t head_dim, int32_t max_depth, int32_t dtype, int32_t* dev_error, void* stream) {
  if (!block_table) return SPEC_E_NULL;
  KvRows kv;
  const spec_status_t st = make_paged_rows(block_table, max_blocks, block_size, num_blocks, Hkv,
                                           &kv);
  if (st != SPEC_OK) return st;
  return launch_commit_layers(k_layers, v_layers, k_tree, v_tree, num_layers, prefix_len, path,
                              accept_len, B, n_max, Hkv, head_dim, kv, max_depth, dtype,
                              dev_error, stream);
}
