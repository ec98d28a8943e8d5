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
// and written by slot 2): each workgroup loads every row it moves for one KV
// head into registers, waits at a barrier, then stores.
#include "common.hpp"

namespace specv {
namespace {

constexpr int NT = 256;
constexpr int MAXCH = (SPEC_MAX_NODES * 128 * 4 / 16 + NT - 1) / NT;  // 16-B chunks per thread

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
    // rows 1..a move (row 0 is the root, already in place)
    const int nchunks = a * row_chunks;
    for (int g = 0; g < Hkv; ++g) {
      for (int which = 0; which < 2; ++which) {
        uint4* base = (which == 0 ? kc : vc) + ((size_t)b * Hkv + g) * (size_t)L_cap * row_chunks +
                      (size_t)L * row_chunks;
        uint4 regs[MAXCH];
#pragma unroll
        for (int j = 0; j < MAXCH; ++j) {
          const int c = tid + j * NT;
          if (c < nchunks) {
            const int slot = 1 + c / row_chunks;
            regs[j] = base[(size_t)s_path[slot] * row_chunks + c % row_chunks];
          }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < MAXCH; ++j) {
          const int c = tid + j * NT;
          if (c < nchunks) {
            const int slot = 1 + c / row_chunks;
            base[(size_t)slot * row_chunks + c % row_chunks] = regs[j];
          }
        }
        __syncthreads();
      }
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
