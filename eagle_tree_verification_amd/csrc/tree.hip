// EAGLE-2 draft-tree construction (gfx950): expansion by path value, then a
// global rerank (page "EAGLE-1/2/3 拆解", sections "一个可核对的经验性质" and
// "两阶段"; page "EAGLE-3 完全拆解", section "EAGLE-3 和 EAGLE-2 动态树如何拼
// 在一起").
//
// A node's value is the sum of the draft's log-probabilities on its root path
// (the log of the product of confidences, same order).  Per level:
//   tree_partials_kernel -- one workgroup per (sequence, draft row, vocabulary
//     split) loads its chunk of the row into registers once, reduces the
//     maximum and the sum of exponentials, and keeps the chunk's top_k logits
//     (equal logits: lower id).  The k-th largest of a wave's 64 lane maxima
//     is a lower bound of the chunk's k-th largest logit (k lanes each hold an
//     element at least that large), so only elements at or above the best
//     such bound are ranked;
//   tree_select_kernel -- one workgroup per sequence combines the splits
//     (log-sum-exp, top_k per row), appends every row's top_k children to the
//     pool with value parent + logit - lse, and ranks the level's new nodes to
//     choose the top_k the draft runs on next (equal values: lower pool
//     index).
// tree_finalize_kernel -- one workgroup per sequence ranks the whole pool,
//   keeps the best total_tokens and emits them after the root in pool order,
//   with parents, depths, positions, values, draft rows and ancestor masks.
//
// A child's value never exceeds its parent's in float arithmetic (lse is at
// least the row maximum, so logit - lse <= 0, and rounding is monotone), and
// a parent's pool index is lower than its children's, so the chosen set
// always holds every ancestor of its members.
#include <limits.h>

#include "common.hpp"

namespace specv {
namespace {

constexpr int kMaxK = SPEC_TREE_MAX_TOP_K;       // children per expanded node
constexpr int kMaxDepth = SPEC_TREE_MAX_DEPTH;   // levels
constexpr int NTP = 256;                         // partials workgroup
constexpr int EPT = 64;                          // row elements per thread (registers)
constexpr int kChunk = NTP * EPT;                // largest chunk of one workgroup
constexpr int kCap = 256;                        // ranked candidates per chunk
constexpr int kRec = 2 + 2 * kMaxK;              // words per partial record
constexpr int NTS = 256;                         // select workgroup
constexpr int NTF = 1024;                        // finalize workgroup
constexpr float kL2E = 1.4426950408889634f;

// ---- state layout (per sequence, int32 words) -------------------------------
// [0] levels done, [1] failed, [2..3] spare,
// expanded[kDepth][k] pool ids, then pool token[P], parent[P], value[P] (f32).
__host__ __device__ inline int pool_size(int k, int depth) { return k + (depth - 1) * k * k; }
__host__ __device__ inline int level_base(int k, int level) {
  return level == 1 ? 0 : k + (level - 2) * k * k;
}
__host__ __device__ inline int level_of(int k, int p) { return p < k ? 1 : 2 + (p - k) / (k * k); }
__host__ __device__ inline size_t seq_words(int k, int depth) {
  const size_t w = 4 + (size_t)depth * k + 3 * (size_t)pool_size(k, depth);
  return (w + 63) & ~(size_t)63;
}
__host__ __device__ inline int max_splits(int k) { return (256 / k) < 64 ? 256 / k : 64; }
inline size_t partials_offset(int B, int k, int depth) {  // bytes
  return ((size_t)B * seq_words(k, depth) * 4 + 255) & ~(size_t)255;
}
inline size_t state_bytes_for(int B, int k, int depth) {
  return partials_offset(B, k, depth) + (size_t)B * k * max_splits(k) * kRec * 4;
}

struct SeqState {
  int32_t* hdr;
  int32_t* expanded;  // [depth][k]
  int32_t* token;     // [P]
  int32_t* parent;    // [P]
  float* value;       // [P]
};
__device__ inline SeqState seq_state(int32_t* base, int b, int k, int depth) {
  SeqState s;
  int32_t* w = base + (size_t)b * seq_words(k, depth);
  const int P = pool_size(k, depth);
  s.hdr = w;
  s.expanded = w + 4;
  s.token = s.expanded + depth * k;
  s.parent = s.token + P;
  s.value = reinterpret_cast<float*>(s.parent + P);
  return s;
}

// (x, id) order: larger logit first, then lower id.  id < 0 marks "none".
__device__ __forceinline__ bool beats(float xa, int ia, float xb, int ib) {
  return xa > xb || (xa == xb && ia < ib);
}

__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ float load1(const uint16_t* p) { return bf16_to_f32(*p); }

// 16-byte vector of W elements converted to f32.
__device__ __forceinline__ void load16(const float* p, float* o) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
__device__ __forceinline__ void load16(const uint16_t* p, float* o) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Descending bitonic sort of one float per lane across the wave.
__device__ __forceinline__ float wave_sort_desc(float v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const float o = __shfl_xor(v, stride);
      const bool up = (lane & size) == 0;        // this block sorts descending
      const bool low = (lane & stride) == 0;     // this lane keeps the larger
      v = (up == low) ? fmaxf(v, o) : fminf(v, o);
    }
  }
  return v;
}

template <typename T, bool VEC>
__global__ __launch_bounds__(NTP) void tree_partials_kernel(const T* __restrict__ logits, int Vd,
                                                            int R, int S, int chunk, int k,
                                                            float* __restrict__ part) {
  constexpr int W = 16 / sizeof(T);
  const int s = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const T* row = logits + ((size_t)b * R + r) * Vd;
  const int beg = s * chunk;
  const int end = min(Vd, beg + chunk);
  auto elem_id = [&](int i) -> int {
    return VEC ? beg + ((i / W) * NTP + tid) * W + (i % W) : beg + i * NTP + tid;
  };

  float x[EPT];
  if constexpr (VEC) {
#pragma unroll
    for (int v = 0; v < EPT / W; ++v) {
      const int e0 = beg + (v * NTP + tid) * W;
      if (e0 < end) {
        load16(row + e0, x + v * W);
      } else {
#pragma unroll
        for (int j = 0; j < W; ++j) x[v * W + j] = -INFINITY;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = beg + i * NTP + tid;
      x[i] = e < end ? load1(row + e) : -INFINITY;
    }
  }

  __shared__ float s_red[4];
  __shared__ float s_red2[4];
  __shared__ float s_cx[kCap];
  __shared__ int s_cid[kCap];
  __shared__ int s_cnt;
  __shared__ float s_wx[4];
  __shared__ int s_wid[4];

  // maximum and sum of exponentials (v_exp_f32 maps -inf to 0)
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPT; ++i) m = fmaxf(m, x[i]);
  const float mm = (m == -INFINITY) ? 0.f : m;
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < EPT; ++i) sum += __builtin_amdgcn_exp2f((x[i] - mm) * kL2E);

  const float sorted = wave_sort_desc(m);
  const float thr_w = __shfl(sorted, k - 1);
  const float mw = __shfl(sorted, 0);
  if (tid == 0) s_cnt = 0;
  if (lane == 0) { s_red[wid] = mw; s_red2[wid] = thr_w; }
  __syncthreads();
  const float M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  const float thr = fmaxf(fmaxf(s_red2[0], s_red2[1]), fmaxf(s_red2[2], s_red2[3]));
  // NaN entries make the sum NaN; a +inf entry makes it NaN too (inf - inf)
  // (a lane whose maximum is -inf has sum 0, or NaN if it read a NaN)
  float part_sum = (m == -INFINITY) ? sum : sum * __builtin_amdgcn_exp2f((m - M) * kL2E);
  part_sum = wave_sum(part_sum);

  // candidates: valid elements at or above the bound
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int id = elem_id(i);
    if (id < end && x[i] >= thr) {
      const int slot = atomicAdd(&s_cnt, 1);
      if (slot < kCap) { s_cx[slot] = x[i]; s_cid[slot] = id; }
    }
  }
  __syncthreads();
  if (lane == 0) s_red[wid] = part_sum;  // s_red's maxima were read before the barrier
  const int cnt = s_cnt;
  float* rec = part + (((size_t)b * R + r) * S + s) * kRec;
  float* rx = rec + 2;
  int* rid = reinterpret_cast<int*>(rec + 2 + kMaxK);

  if (cnt <= kCap) {
    if (tid < cnt) {
      const float cx = s_cx[tid];
      const int ci = s_cid[tid];
      int rank = 0;
      for (int j = 0; j < cnt; ++j) rank += beats(s_cx[j], s_cid[j], cx, ci);
      if (rank < k) { rx[rank] = cx; rid[rank] = ci; }
    }
    if (tid >= cnt && tid < k) { rx[tid] = -INFINITY; rid[tid] = -1; }
  } else {
    // many equal logits at the bound: k rounds of "best element after the
    // previous winner" over the registers
    float px = INFINITY;
    int pid = -1;
    for (int round = 0; round < k; ++round) {
      float bx = -INFINITY;
      int bi = INT_MAX;
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        const int id = elem_id(i);
        const bool after = x[i] < px || (x[i] == px && id > pid);
        if (id < end && after && beats(x[i], id, bx, bi)) { bx = x[i]; bi = id; }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ox = __shfl_xor(bx, o);
        const int oi = __shfl_xor(bi, o);
        if (beats(ox, oi, bx, bi)) { bx = ox; bi = oi; }
      }
      __syncthreads();
      if (lane == 0) { s_wx[wid] = bx; s_wid[wid] = bi; }
      __syncthreads();
      bx = s_wx[0];
      bi = s_wid[0];
#pragma unroll
      for (int w = 1; w < 4; ++w)
        if (beats(s_wx[w], s_wid[w], bx, bi)) { bx = s_wx[w]; bi = s_wid[w]; }
      if (tid == 0) {
        rx[round] = bi == INT_MAX ? -INFINITY : bx;
        rid[round] = bi == INT_MAX ? -1 : bi;
      }
      px = bx;
      pid = bi;
    }
  }
  __syncthreads();
  if (tid == 0) {
    rec[0] = M;
    rec[1] = s_red[0] + s_red[1] + s_red[2] + s_red[3];
  }
}

// One workgroup per sequence.
__global__ __launch_bounds__(NTS) void tree_select_kernel(
    const float* __restrict__ part, int R, int S, int k, int depth, int level,
    const int32_t* __restrict__ d2t, int32_t* __restrict__ state, int32_t* __restrict__ exp_tokens,
    int32_t* __restrict__ exp_ids, int32_t* __restrict__ dev_error) {
  const int b = blockIdx.x, tid = threadIdx.x;
  SeqState st = seq_state(state, b, k, depth);
  __shared__ int s_skip;
  __shared__ int s_bad;
  __shared__ float s_lse[kMaxK];
  __shared__ float s_pv[kMaxK];
  __shared__ int s_pid[kMaxK];
  __shared__ float s_x[kMaxK * 256];
  __shared__ int s_id[kMaxK * 256];
  __shared__ float s_val[kMaxK * kMaxK];
  __shared__ int s_tok[kMaxK * kMaxK];

  if (tid == 0) {
    int skip = 0;
    if (level == 1) {
      st.hdr[1] = 0;
    } else if (st.hdr[0] != level - 1) {  // levels out of order for this state
      report(dev_error, SPEC_DEVERR_TREE);
      st.hdr[1] = 1;
      skip = 1;
    } else {
      skip = st.hdr[1];
    }
    s_skip = skip;
    s_bad = 0;
  }
  __syncthreads();
  if (s_skip) {
    if (tid < k) {
      exp_tokens[(size_t)b * k + tid] = -1;
      if (exp_ids) exp_ids[(size_t)b * k + tid] = -1;
      st.expanded[(level - 1) * k + tid] = -1;
    }
    if (tid == 0) st.hdr[0] = level;
    return;
  }

  const int nc = S * k;  // candidates per row
  if (tid < R) {
    const float* rec0 = part + ((size_t)b * R + tid) * S * kRec;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, rec0[(size_t)s * kRec]);
    float sum = 0.f;
    for (int s = 0; s < S; ++s) {
      const float ms = rec0[(size_t)s * kRec];
      const float ss = rec0[(size_t)s * kRec + 1];
      sum += (ms == -INFINITY) ? ss : ss * expf(ms - M);  // ss is 0 or NaN there
    }
    const bool bad = !(M < INFINITY) || M == -INFINITY || !(sum == sum) || !(sum < INFINITY);
    if (bad) atomicOr(&s_bad, 1);
    s_lse[tid] = M + fmaxf(logf(sum), 0.f);
    const int pid = level == 1 ? -1 : st.expanded[(level - 2) * k + tid];
    const bool pid_ok = level == 1 || (pid >= level_base(k, level - 1) && pid < level_base(k, level));
    if (!pid_ok) atomicOr(&s_bad, 2);
    s_pid[tid] = pid;
    s_pv[tid] = pid_ok && level > 1 ? st.value[pid] : 0.f;
  }
  for (int c = tid; c < R * nc; c += NTS) {
    const int r = c / nc, rem = c - r * nc;
    const int s = rem / k, j = rem - s * k;
    const float* rec = part + (((size_t)b * R + r) * S + s) * kRec;
    s_x[c] = rec[2 + j];
    s_id[c] = reinterpret_cast<const int*>(rec + 2 + kMaxK)[j];
  }
  __syncthreads();
  if (s_bad) {
    if (tid == 0) {
      report(dev_error, (s_bad & 1 ? SPEC_DEVERR_NONFINITE : 0) | (s_bad & 2 ? SPEC_DEVERR_TREE : 0));
      st.hdr[1] = 1;
      st.hdr[0] = level;
    }
    if (tid < k) {
      exp_tokens[(size_t)b * k + tid] = -1;
      if (exp_ids) exp_ids[(size_t)b * k + tid] = -1;
      st.expanded[(level - 1) * k + tid] = -1;
    }
    return;
  }

  // top_k children of every row: rank each split candidate within its row
  const int base = level_base(k, level);
  for (int c = tid; c < R * nc; c += NTS) {
    const int id = s_id[c];
    if (id < 0) continue;
    const int r = c / nc;
    const float x = s_x[c];
    const float* rx = s_x + r * nc;
    const int* ri = s_id + r * nc;
    int rank = 0;
    for (int j = 0; j < nc && rank < k; ++j) rank += (ri[j] >= 0) && beats(rx[j], ri[j], x, id);
    if (rank < k) {
      const int q = r * k + rank;
      const float v = s_pv[r] + (x - s_lse[r]);
      const int tok = id + (d2t ? d2t[id] : 0);
      st.token[base + q] = tok;
      st.parent[base + q] = s_pid[r];
      st.value[base + q] = v;
      s_val[q] = v;
      s_tok[q] = tok;
    }
  }
  __syncthreads();

  // expansion: the top_k of the level's R * k new nodes
  const int nn = R * k;
  if (tid < nn) {
    const float v = s_val[tid];
    int rank = 0;
    for (int j = 0; j < nn; ++j) rank += s_val[j] > v || (s_val[j] == v && j < tid);
    if (rank < k) {
      st.expanded[(level - 1) * k + rank] = base + tid;
      exp_tokens[(size_t)b * k + rank] = s_tok[tid];
      if (exp_ids) exp_ids[(size_t)b * k + rank] = base + tid;
    }
  }
  if (tid == 0) st.hdr[0] = level;
}

__global__ __launch_bounds__(NTF) void tree_finalize_kernel(
    const int32_t* __restrict__ state, int k, int depth, int N, const int32_t* __restrict__ root_token,
    const int32_t* __restrict__ prefix_len, int n_max, int32_t* __restrict__ tokens,
    int32_t* __restrict__ parents, int32_t* __restrict__ n_nodes, int32_t* __restrict__ node_depth,
    int32_t* __restrict__ positions, uint64_t* __restrict__ anc_mask,
    int32_t* __restrict__ draft_row, float* __restrict__ value, int32_t* __restrict__ dev_error) {
  constexpr int kMaxPool = kMaxK + (kMaxDepth - 1) * kMaxK * kMaxK;
  const int b = blockIdx.x, tid = threadIdx.x;
  SeqState st = seq_state(const_cast<int32_t*>(state), b, k, depth);
  __shared__ float s_v[kMaxPool];
  __shared__ short s_node[kMaxPool];  // node id of a chosen pool entry, else 0
  __shared__ short s_row[kMaxPool];   // draft row of an expanded pool entry, else -1
  __shared__ int s_par[SPEC_MAX_NODES];
  __shared__ int s_scan[NTF / 64];
  const int levels = st.hdr[0];
  const int failed = st.hdr[1];
  if (failed || levels < 1 || levels > depth) {
    if (tid == 0) {
      n_nodes[b] = 0;
      if (!failed) report(dev_error, SPEC_DEVERR_TREE);
    }
    return;
  }
  const int P = pool_size(k, levels);
  for (int p = tid; p < P; p += NTF) { s_v[p] = st.value[p]; s_row[p] = -1; }
  __syncthreads();
  for (int i = tid; i < (levels - 1) * k; i += NTF) {
    const int e = st.expanded[i];
    if (e >= 0 && e < P) s_row[e] = (short)(1 + i);
  }
  // rank among live entries: value desc, pool index asc; keep the best N
  constexpr int PPT = (kMaxPool + NTF - 1) / NTF;
  int flags = 0;
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int p = tid * PPT + j;
    if (p < P) {
      const float v = s_v[p];
      if (v > -INFINITY) {
        int rank = 0;
        for (int q = 0; q < P && rank < N; ++q) rank += s_v[q] > v || (s_v[q] == v && q < p);
        if (rank < N) { flags |= 1 << j; ++cnt; }
      }
    }
  }
  // exclusive scan of the counts in thread order = pool order
  const int lane = tid & 63, wid = tid >> 6;
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) s_scan[wid] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < NTF / 64; ++w) {
    const int c = s_scan[w];
    before += w < wid ? c : 0;
    total += c;
  }
  int node = before + incl - cnt + 1;
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int p = tid * PPT + j;
    if (p < P) s_node[p] = (flags >> j & 1) ? (short)node++ : (short)0;
  }
  __syncthreads();
  const size_t o = (size_t)b * n_max;
  const int L = prefix_len ? prefix_len[b] : 0;
  int bad = 0;
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int p = tid * PPT + j;
    if (p < P && (flags >> j & 1)) {
      const int nd = s_node[p];
      const int pp = st.parent[p];
      const int pn = pp < 0 ? 0 : s_node[pp];
      if (pp >= 0 && pn == 0) bad = 1;  // cannot happen: values never rise along a path
      const int d = level_of(k, p);
      tokens[o + nd] = st.token[p];
      parents[o + nd] = pn;
      s_par[nd] = pn;
      if (node_depth) node_depth[o + nd] = d;
      if (positions) positions[o + nd] = L + d;
      if (value) value[o + nd] = s_v[p];
      if (draft_row) draft_row[o + nd] = s_row[p];
    }
  }
  if (tid == 0) {
    tokens[o] = root_token ? root_token[b] : -1;
    parents[o] = -1;
    s_par[0] = -1;
    if (node_depth) node_depth[o] = 0;
    if (positions) positions[o] = L;
    if (value) value[o] = 0.f;
    if (draft_row) draft_row[o] = 0;
  }
  if (__syncthreads_or(bad)) {
    if (tid == 0) {
      report(dev_error, SPEC_DEVERR_TREE);
      n_nodes[b] = 0;
    }
    return;
  }
  if (anc_mask && tid <= total) {
    uint64_t mask = 0;
    for (int x = tid; x >= 0; x = s_par[x]) mask |= 1ull << x;
    anc_mask[o + tid] = mask;
  }
  if (tid == 0) n_nodes[b] = total + 1;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace
}  // namespace specv

using namespace specv;

extern "C" size_t spec_tree_state_size(int32_t B, int32_t top_k, int32_t depth) {
  if (B <= 0 || top_k < 1 || top_k > kMaxK || depth < 1 || depth > kMaxDepth) return 0;
  return state_bytes_for(B, top_k, depth);
}

extern "C" spec_status_t spec_tree_expand(const void* draft_logits, int32_t dtype,
                                          const int32_t* d2t, int32_t B, int32_t Vd, int32_t top_k,
                                          int32_t depth, int32_t level, void* state,
                                          size_t state_bytes, int32_t* expanded_tokens,
                                          int32_t* expanded_ids, int32_t* dev_error,
                                          void* stream) {
  if (!draft_logits || !state || !expanded_tokens) return SPEC_E_NULL;
  if (B <= 0 || top_k < 1 || top_k > kMaxK || depth < 1 || depth > kMaxDepth || level < 1 ||
      level > depth || Vd < top_k || B > 65535)
    return SPEC_E_SHAPE;
  const int smax = max_splits(top_k);
  if ((long)Vd > (long)kChunk * smax) return SPEC_E_SHAPE;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_E_DTYPE;
  if (state_bytes < state_bytes_for(B, top_k, depth)) return SPEC_E_WORKSPACE;
  const int R = level == 1 ? 1 : top_k;
  // splits: enough for the chunk to fit the registers, more when the grid is
  // small (at most one split per 2048 elements)
  const int s_min = (Vd + kChunk - 1) / kChunk;
  const int s_par = (4 * device_cu_count() + B * R - 1) / (B * R);
  int S = s_par < Vd / 2048 ? s_par : Vd / 2048;
  if (S < s_min) S = s_min;
  if (S > smax) S = smax;
  int chunk = (Vd + S - 1) / S;
  chunk = (chunk + 7) & ~7;
  S = (Vd + chunk - 1) / chunk;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* st = static_cast<int32_t*>(state);
  float* part = reinterpret_cast<float*>(static_cast<char*>(state) +
                                         partials_offset(B, top_k, depth));
  const dim3 grid(S, R, B);
  const int W = dtype == SPEC_F32 ? 4 : 8;
  const bool vec = Vd % W == 0 && aligned16(draft_logits);
  if (dtype == SPEC_F32) {
    const float* lg = static_cast<const float*>(draft_logits);
    if (vec)
      hipLaunchKernelGGL((tree_partials_kernel<float, true>), grid, dim3(NTP), 0, s, lg, Vd, R, S,
                         chunk, top_k, part);
    else
      hipLaunchKernelGGL((tree_partials_kernel<float, false>), grid, dim3(NTP), 0, s, lg, Vd, R,
                         S, chunk, top_k, part);
  } else {
    const uint16_t* lg = static_cast<const uint16_t*>(draft_logits);
    if (vec)
      hipLaunchKernelGGL((tree_partials_kernel<uint16_t, true>), grid, dim3(NTP), 0, s, lg, Vd,
                         R, S, chunk, top_k, part);
    else
      hipLaunchKernelGGL((tree_partials_kernel<uint16_t, false>), grid, dim3(NTP), 0, s, lg, Vd,
                         R, S, chunk, top_k, part);
  }
  SPEC_HIP_TRY(hipGetLastError());
  hipLaunchKernelGGL(tree_select_kernel, dim3(B), dim3(NTS), 0, s, part, R, S, top_k, depth,
                     level, d2t, st, expanded_tokens, expanded_ids, dev_error);
  SPEC_HIP_TRY(hipGetLastError());
  return SPEC_OK;
}

extern "C" spec_status_t spec_tree_finalize(
    const void* state, size_t state_bytes, int32_t B, int32_t top_k, int32_t depth,
    int32_t total_tokens, const int32_t* root_token, const int32_t* prefix_len, int32_t n_max,
    int32_t* tokens, int32_t* parents, int32_t* n_nodes, int32_t* node_depth, int32_t* positions,
    uint64_t* anc_mask, int32_t* draft_row, float* value, int32_t* dev_error, void* stream) {
  if (!state || !tokens || !parents || !n_nodes) return SPEC_E_NULL;
  if (B <= 0 || top_k < 1 || top_k > kMaxK || depth < 1 || depth > kMaxDepth ||
      total_tokens < 1 || total_tokens >= SPEC_MAX_NODES || n_max < total_tokens + 1 ||
      n_max > SPEC_MAX_NODES || B > 65535)
    return SPEC_E_SHAPE;
  if (state_bytes < state_bytes_for(B, top_k, depth)) return SPEC_E_WORKSPACE;
  hipLaunchKernelGGL(tree_finalize_kernel, dim3(B), dim3(NTF), 0,
                     static_cast<hipStream_t>(stream), static_cast<const int32_t*>(state), top_k,
                     depth, total_tokens, root_token, prefix_len, n_max, tokens, parents, n_nodes,
                     node_depth, positions, anc_mask, draft_row, value, dev_error);
  SPEC_HIP_TRY(hipGetLastError());
  return SPEC_OK;
}
