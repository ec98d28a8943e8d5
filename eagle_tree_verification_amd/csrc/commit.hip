// KV commit of the accepted path (gfx950).
//
// Rollback keeps a physical cache and a logical length, or writes to scratch
// and commits on acceptance (page "推测解码与 EAGLE-3", section "KV cache
// 回滚"; build step 4 sets the logical length to prefix + accepted + 1).  The
// tree's K/V rows sit at prefix_len + node, so the accepted path (root plus a
// accepted drafts, node ids increasing along the path) is gathered to rows
// prefix_len + 0..a and the length advances by a + 1.  A chain-shaped path
// (path[i] == i) moves nothing.  Moves are in place and path[i] >= i, so a
// row can be both read and written (path [0, 2, 5]: row 2 is read for slot 1
// and written by slot 2): one workgroup per sequence loads every row it moves
// (all KV heads, K and V) into registers, waits at a barrier, then stores.
// Moves that do not fit one round are done in rounds of increasing slot within
// each (head, K/V) plane; a later round reads only rows path[s] >= s beyond
// every row an earlier round wrote, so rounds never see each other's writes.
// The workgroup also owns the sequence's length, so no other workgroup can
// read it after it advances.
#include "common.hpp"

namespace specv {
namespace {

constexpr int NT = 1024;
constexpr int CPT = 16;  // 16-byte chunks per thread per round

__global__ __launch_bounds__(NT) void commit_kernel(uint4* kc, uint4* vc, int32_t* prefix_len,
                                                    const int32_t* path, const int32_t* accept_len,
                                                    int Hkv, int row_chunks, int L_cap,
                                                    int max_depth, int32_t* dev_error) {
  __shared__ int s_path[SPEC_MAX_NODES + 1];
  __shared__ int s_moves;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int a = accept_len[b];
  const int L = prefix_len[b];
  if (a < 0) return;
  if (a > max_depth || L < 0 || (int64_t)L + a + 1 > L_cap) {
    if (tid == 0) report(dev_error, a > max_depth ? SPEC_DEVERR_TREE : SPEC_DEVERR_CAPACITY);
    return;
  }
  if (tid == 0) s_moves = 0;
  __syncthreads();
  int bad = 0;
  if (tid <= a) {
    const int p = path[(size_t)b * (max_depth + 1) + tid];
    s_path[tid] = p;
    if (tid == 0) bad = (p != 0);
    if (p != tid) atomicOr(&s_moves, 1);
    if ((int64_t)L + p >= L_cap || p < tid) bad = 1;
  }
  __syncthreads();
  if (tid > 0 && tid <= a && s_path[tid] <= s_path[tid - 1]) bad = 1;
  if (__syncthreads_or(bad)) {
    if (tid == 0) report(dev_error, SPEC_DEVERR_TREE);
    return;
  }
  if (s_moves) {
    // chunk c = ((g * 2 + kv) * a + slot - 1) * row_chunks + cc: rows 1..a of
    // every plane (row 0 is the root, already in place)
    const int plane_chunks = a * row_chunks;
    const int total = Hkv * 2 * plane_chunks;
    const size_t plane_stride = (size_t)L_cap * row_chunks;
    // element offset of chunk c's row `row` (relative to the sequence's
    // prefix end) in its plane
    auto offset = [&](int c, int row_of_slot, int* pl_out) -> size_t {
      const int pl = c / plane_chunks;
      const int rem = c - pl * plane_chunks;
      const int slot = 1 + rem / row_chunks;
      const int cc = rem - (slot - 1) * row_chunks;
      *pl_out = pl;
      const int row = row_of_slot ? s_path[slot] : slot;
      return ((size_t)b * Hkv + (pl >> 1)) * plane_stride + (size_t)(L + row) * row_chunks + cc;
    };
    for (int r0 = 0; r0 < total; r0 += NT * CPT) {
      uint4 regs[CPT];
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int c = r0 + j * NT + tid;
        int pl = 0;
        const size_t off = c < total ? offset(c, 1, &pl) : 0;
        const uint4* src = (pl & 1) ? vc : kc;
        regs[j] = c < total ? src[off] : make_uint4(0, 0, 0, 0);
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int c = r0 + j * NT + tid;
        if (c < total) {
          int pl = 0;
          const size_t off = offset(c, 0, &pl);
          ((pl & 1) ? vc : kc)[off] = regs[j];
        }
      }
      __syncthreads();
    }
  }
  if (tid == 0) prefix_len[b] = L + a + 1;
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
  if (B <= 0 || Hkv <= 0 || L_cap <= 0 || max_depth < 0 || max_depth >= SPEC_MAX_NODES)
    return SPEC_E_SHAPE;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_E_DTYPE;
  if (head_dim != 16 && head_dim != 32 && head_dim != 64 && head_dim != 128) return SPEC_E_DTYPE;
  const int esz = dtype == SPEC_F32 ? 4 : 2;
  const int row_chunks = head_dim * esz / 16;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(commit_kernel, dim3(B), dim3(NT), 0, strm, static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache), prefix_len, path, accept_len, Hkv, row_chunks,
                     L_cap, max_depth, dev_error);
  SPEC_HIP_TRY(hipGetLastError());
  return SPEC_OK;
}
