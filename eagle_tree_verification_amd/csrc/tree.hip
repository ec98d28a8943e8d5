// EAGLE-2 draft-tree construction (gfx950): expansion by path value, then a
// global rerank (page "EAGLE-1/2/3 拆解", sections "一个可核对的经验性质" and
// "两阶段"; page "EAGLE-3 完全拆解", section "EAGLE-3 和 EAGLE-2 动态树如何拼
// 在一起").
//
// A node's value is the sum of the draft's log-probabilities on its root path
// (the log of the product of confidences, same order).  Per level:
//   tree_partials_kernel -- one workgroup per (sequence, draft row, vocabulary
//     split) streams its chunk once with two tiles in flight per wave,
//     keeping a running maximum and sum of exponentials per lane and a sorted
//     top_k (logit, id) list per wave (equal logits: lower id).  An element
//     is looked at again only if it reaches the list's k-th logit; before the
//     list fills, the k-th largest of the wave's 64 lane maxima over its
//     first tile serves as the bound (k lanes each hold an element at least
//     that large);
//   tree_select_kernel -- one workgroup per sequence combines the splits
//     (log-sum-exp, top_k per row), appends every row's top_k children to the
//     pool with value parent + logit - lse, ranks the level's new nodes to
//     choose the top_k the draft runs on next (equal values: lower pool
//     index), and merges them into the sequence's running list of the 63 most
//     valuable nodes.
// tree_finalize_kernel -- one wave per sequence keeps the first total_tokens
//   of that list and emits them after the root in pool order, with parents,
//   depths, positions, values, draft rows and ancestor masks.
//
// A child's value never exceeds its parent's in float arithmetic (lse is at
// least the row maximum, so logit - lse <= 0, and rounding is monotone), and
// a parent's pool index is lower than its children's, so any top-N set holds
// every ancestor of its members; the top 63 of all levels is the top 63 of
// (the top 63 of the levels before) and (this level's nodes).
#include <limits.h>

#include <atomic>

#include "common.hpp"

namespace specv {
namespace {

constexpr int kMaxK = SPEC_TREE_MAX_TOP_K;       // children per expanded node
constexpr int kMaxDepth = SPEC_TREE_MAX_DEPTH;   // levels
constexpr int kBest = SPEC_MAX_NODES - 1;        // most valuable nodes kept across levels
constexpr int NTP = 256;                         // partials workgroup (4 waves)
constexpr int kMaxVocab = 1 << 24;               // draft vocabulary limit
constexpr int kRec = 2 + 3 * kMaxK;              // words per split record
constexpr int NTS = 1024;                        // selection workgroup
constexpr float kL2E = 1.4426950408889634f;

// ---- state layout (per sequence, int32 words) -------------------------------
// hdr[8]: [0] levels grown, [1] failed, [2] entries in the best list;
// expanded[depth][k] pool ids, exp_val[depth][k] (f32) their values;
// best_id[64], best_val[64] (f32): the most valuable pool nodes, best first;
// pool token[P], parent[P], value[P] (f32).
constexpr int kHdr = 8;
__host__ __device__ inline int pool_size(int k, int depth) { return k + (depth - 1) * k * k; }
__host__ __device__ inline int level_base(int k, int level) {
  return level == 1 ? 0 : k + (level - 2) * k * k;
}
__host__ __device__ inline int level_of(int k, int p) { return p < k ? 1 : 2 + (p - k) / (k * k); }
__host__ __device__ inline size_t seq_words(int k, int depth) {
  const size_t w = kHdr + 2 * (size_t)depth * k + 2 * 64 + 3 * (size_t)pool_size(k, depth);
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
  int32_t* expanded;  // [depth][k] pool ids chosen for expansion, best first
  float* exp_val;     // [depth][k] their values
  int32_t* best_id;   // [64]
  float* best_val;    // [64]
  int32_t* token;     // [P]
  int32_t* parent;    // [P]
  float* value;       // [P]
};
__device__ inline SeqState seq_state(int32_t* base, int b, int k, int depth) {
  SeqState s;
  int32_t* w = base + (size_t)b * seq_words(k, depth);
  const int P = pool_size(k, depth);
  s.hdr = w;
  s.expanded = w + kHdr;
  s.exp_val = reinterpret_cast<float*>(s.expanded + depth * k);
  s.best_id = s.expanded + 2 * depth * k;
  s.best_val = reinterpret_cast<float*>(s.best_id + 64);
  s.token = s.best_id + 128;
  s.parent = s.token + P;
  s.value = reinterpret_cast<float*>(s.parent + P);
  return s;
}

// (x, id) order: larger logit first, then lower id.  id < 0 marks "none".
__device__ __forceinline__ bool beats(float xa, int ia, float xb, int ib) {
  return xa > xb || (xa == xb && ia < ib);
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

__device__ __forceinline__ float rl_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ int rl_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

// One wave's share of a chunk is read in tiles of 64 lanes x EL elements.
// Vector layout: load j of a lane covers W consecutive elements at
// j * 64 * W + lane * W (each load instruction reads one contiguous run);
// scalar layout: element i of a lane is i * 64 + lane.
template <typename T>
constexpr int tile_elems() { return 16; }
template <typename T>
constexpr int block_tile() { return (NTP / 64) * 64 * tile_elems<T>(); }

template <typename T, bool VEC>
struct TileIO {
  static constexpr int EL = tile_elems<T>();
  static constexpr int W = VEC ? 16 / (int)sizeof(T) : 1;  // elements per load
  static constexpr int NL = EL / W;                        // loads per lane
  uint32_t w[VEC ? EL * sizeof(T) / 4 : EL];

  __device__ static int off(int lane, int i) {
    return VEC ? (i / W) * 64 * W + lane * W + (i % W) : i * 64 + lane;
  }
  // Loads the tile at `base`; loads whose first element is at or beyond
  // `end` read `safe` instead (always in range), so every load is issued
  // unconditionally.
  __device__ void load(const T* row, int base, int end, int safe, int lane) {
    if constexpr (VEC) {
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int e = base + j * 64 * W + lane * W;
        const uint4 v = *reinterpret_cast<const uint4*>(row + (e < end ? e : safe));
        w[4 * j] = v.x; w[4 * j + 1] = v.y; w[4 * j + 2] = v.z; w[4 * j + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < EL; ++i) {
        const int e = base + i * 64 + lane;
        if constexpr (sizeof(T) == 4)
          w[i] = __float_as_uint(row[e < end ? e : safe]);
        else
          w[i] = static_cast<uint32_t>(row[e < end ? e : safe]) << 16;
      }
    }
  }
  __device__ float get(int i) const {
    if constexpr (!VEC || sizeof(T) == 4) return __uint_as_float(w[i]);
    else return __uint_as_float((i & 1) ? (w[i >> 1] & 0xffff0000u) : (w[i >> 1] << 16));
  }
};

// One workgroup per sequence, after the level's splits: wave w reduces draft
// rows w, w+16, ... (log-sum-exp over the splits), every thread ranks split
// candidates within their row to give each row's top_k children, the
// level's R * k new nodes are ranked to choose the top_k to expand, and the
// best list is updated.
__global__ __launch_bounds__(NTS) void tree_select_kernel(
    const float* __restrict__ part, int R, int S, int k, int depth, int level,
    int32_t* __restrict__ state, int32_t* __restrict__ exp_tokens, int32_t* __restrict__ exp_ids,
    int32_t* __restrict__ dev_error) {
  constexpr int NT = NTS;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  SeqState st = seq_state(state, b, k, depth);
  __shared__ float s_x[kMaxK * 256];  // split candidates, row-major
  __shared__ int s_id[kMaxK * 256];
  __shared__ int s_tk[kMaxK * 256];
  __shared__ int s_skip;
  __shared__ int s_bad;
  __shared__ int s_live;
  __shared__ float s_lse[kMaxK];
  __shared__ float s_pv[kMaxK];
  __shared__ int s_pid[kMaxK];
  __shared__ float s_cv[kBest + kMaxK * kMaxK];  // best-list candidates: old list, then new nodes
  __shared__ int s_cp[kBest + kMaxK * kMaxK];
  __shared__ int s_tok[kMaxK * kMaxK];

  // every load of the prologue is independent of the others
  const int h0 = st.hdr[0], h1 = st.hdr[1];
  const int nb = level == 1 ? 0 : min(max(st.hdr[2], 0), kBest);
  if (tid == 0) {
    s_bad = 0;
    s_live = 0;
    s_skip = level == 1 ? 0 : (h0 != level - 1 ? 2 : h1);
  }
  if (tid < nb) {
    s_cp[tid] = st.best_id[tid];
    s_cv[tid] = st.best_val[tid];
  }
  const int nc = S * k;  // candidates per row
  const float* seq_part = part + (size_t)b * R * S * kRec;
  __syncthreads();  // s_bad cleared
  for (int r = wid; r < R; r += NT / 64) {  // S <= 64: one lane per split
    const float* rec = seq_part + ((size_t)r * S + lane) * kRec;
    const float ms = lane < S ? rec[0] : -INFINITY;
    const float ss = lane < S ? rec[1] : 0.f;
    const int pid = level == 1 ? -1 : st.expanded[(level - 2) * k + r];
    const float pv = level == 1 ? 0.f : st.exp_val[(level - 2) * k + r];
    const float M = wave_max(ms);
    const float sum = wave_sum(ms == -INFINITY ? ss : ss * expf(ms - M));  // ss is 0 or NaN there
    if (lane == 0) {
      const bool bad = !(M < INFINITY) || M == -INFINITY || !(sum == sum) || !(sum < INFINITY);
      const bool pid_ok =
          level == 1 || (pid >= level_base(k, level - 1) && pid < level_base(k, level));
      if (bad || !pid_ok) atomicOr(&s_bad, (bad ? 1 : 0) | (pid_ok ? 0 : 2));
      s_lse[r] = M + fmaxf(logf(sum), 0.f);
      s_pid[r] = pid;
      s_pv[r] = pv;
    }
  }
  for (int c = tid; c < R * nc; c += NT) {
    const int r = c / nc, rem = c - r * nc;
    const int sp = rem / k, j = rem - sp * k;
    const float* rec = seq_part + ((size_t)r * S + sp) * kRec;
    s_x[c] = rec[2 + j];
    s_id[c] = reinterpret_cast<const int*>(rec + 2 + kMaxK)[j];
    s_tk[c] = reinterpret_cast<const int*>(rec + 2 + 2 * kMaxK)[j];
  }
  __syncthreads();
  if (s_skip || s_bad) {  // failed before, levels out of order, or a bad row
    if (tid < k) {
      exp_tokens[(size_t)b * k + tid] = -1;
      if (exp_ids) exp_ids[(size_t)b * k + tid] = -1;
      st.expanded[(level - 1) * k + tid] = -1;
    }
    if (tid == 0) {
      const int bits = s_skip == 2 ? SPEC_DEVERR_TREE
                       : s_skip  ? 0
                                 : (s_bad & 1 ? SPEC_DEVERR_NONFINITE : 0) |
                                       (s_bad & 2 ? SPEC_DEVERR_TREE : 0);
      if (bits) report(dev_error, bits);
      st.hdr[1] = 1;
      st.hdr[0] = level;
    }
    return;
  }

  // top_k children of every row: rank each split candidate within its row
  const int base = level_base(k, level);
  for (int c = tid; c < R * nc; c += NT) {
    const int id = s_id[c];
    const int r = c / nc;
    const float x = s_x[c];
    const float* rx = s_x + r * nc;
    const int* ri = s_id + r * nc;
    int rank = 0;
#pragma unroll 4
    for (int j = 0; j < nc; ++j) rank += (ri[j] >= 0) & beats(rx[j], ri[j], x, id);
    if (id >= 0 && rank < k) {
      const int q = r * k + rank;
      const float v = s_pv[r] + (x - s_lse[r]);
      const int tok = s_tk[c];
      st.token[base + q] = tok;
      st.parent[base + q] = s_pid[r];
      st.value[base + q] = v;
      s_cv[nb + q] = v;
      s_cp[nb + q] = base + q;
      s_tok[q] = tok;
    }
  }
  __syncthreads();

  // expansion: the top_k of the level's R * k new nodes; best list: the
  // kBest most valuable of the old list and the new nodes (value -inf never
  // enters it)
  const int nn = R * k;
  const int ncand = nb + nn;
  for (int c = tid; c < ncand; c += NT) {
    const float v = s_cv[c];
    const int pc = s_cp[c];
    if (c >= nb) {
      int rank = 0;
#pragma unroll 4
      for (int j = nb; j < ncand; ++j) rank += (s_cv[j] > v) | ((s_cv[j] == v) & (s_cp[j] < pc));
      if (rank < k) {
        st.expanded[(level - 1) * k + rank] = pc;
        st.exp_val[(level - 1) * k + rank] = v;
        exp_tokens[(size_t)b * k + rank] = s_tok[c - nb];
        if (exp_ids) exp_ids[(size_t)b * k + rank] = pc;
      }
    }
    if (v > -INFINITY) {
      int rank = 0;
#pragma unroll 4
      for (int j = 0; j < ncand; ++j) rank += (s_cv[j] > v) | ((s_cv[j] == v) & (s_cp[j] < pc));
      if (rank < kBest) {
        st.best_id[rank] = pc;
        st.best_val[rank] = v;
      }
    }
  }
  for (int c = tid; c < ncand; c += NT)
    if (s_cv[c] > -INFINITY) atomicAdd(&s_live, 1);
  __syncthreads();
  if (tid == 0) {
    st.hdr[0] = level;
    st.hdr[1] = 0;
    st.hdr[2] = min(s_live, kBest);
  }
}

// Per (sequence, draft row, split): streams its chunk once, two tiles in
// flight per wave.  Each lane keeps a running maximum and sum of
// exponentials; each wave keeps its top_k (logit, id) list in lanes 0..k-1,
// sorted.  An element is looked at again only if it reaches the list's k-th
// logit (a wave-uniform test per element); the first tile's bound is the
// k-th largest lane maximum, so the list fills from at most a few dozen
// candidates.  At the end the four waves' lists and sums are merged.
template <typename T, bool VEC>
__global__ __launch_bounds__(NTP) void tree_partials_kernel(
    const T* __restrict__ logits, int Vd, int R, int S, int chunk, int k,
    const int32_t* __restrict__ d2t, float* __restrict__ part) {
  using IO = TileIO<T, VEC>;
  const int s = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const T* row = logits + ((size_t)b * R + r) * Vd;
  const int beg = s * chunk;
  const int end = min(Vd, beg + chunk);
  constexpr int EL = IO::EL, WTILE = 64 * EL, BTILE = block_tile<T>();
  const int nt = (end - beg + BTILE - 1) / BTILE;
  auto tile_base = [&](int i) { return beg + i * BTILE + wid * WTILE; };

  float m = -INFINITY, sum = 0.f;
  float lx = -INFINITY;      // lanes 0..k-1: the wave's list, best first
  int li = INT_MAX;          // (-inf, INT_MAX) = empty slot
  float kx = -INFINITY;      // the list's k-th entry (wave-uniform)
  int ki = INT_MAX;
  float tb = -INFINITY;      // ballot bound (wave-uniform)

  auto process = [&](const IO& t, int i) {
    const int base = tile_base(i);
    if (base >= end) return;  // this wave's part of the last tile is empty
    float x[EL];
#pragma unroll
    for (int e = 0; e < EL; ++e) x[e] = t.get(e);
    if (base + WTILE > end) {
#pragma unroll
      for (int e = 0; e < EL; ++e) x[e] = base + IO::off(lane, e) < end ? x[e] : -INFINITY;
    }
    float tm = x[0];
#pragma unroll
    for (int e = 1; e < EL; ++e) tm = fmaxf(tm, x[e]);
    if (tm > m) {  // rescale the running sum (m = -inf means it is 0 or NaN)
      sum = m == -INFINITY ? sum : sum * __builtin_amdgcn_exp2f((m - tm) * kL2E);
      m = tm;
    }
    const float mml = (m == -INFINITY ? 0.f : m) * kL2E;
#pragma unroll
    for (int e = 0; e < EL; ++e) sum += __builtin_amdgcn_exp2f(fmaf(x[e], kL2E, -mml));
    if (i == 0) {  // bound for the first tile: k lanes hold an element >= it
      const float srt = wave_sort_desc(tm);
      tb = fmaxf(tb, rl_f(srt, k - 1));
    }
    if (!__ballot(tm >= tb)) return;  // no lane holds a candidate in this tile
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      uint64_t bal = __ballot(x[e] >= tb);
      while (bal) {
        const int L = __ffsll((unsigned long long)bal) - 1;
        bal &= bal - 1;
        const float xv = rl_f(x[e], L);
        const int iv = base + IO::off(L, e);
        if (iv < end && beats(xv, iv, kx, ki)) {
          const bool ahead = lane < k && beats(lx, li, xv, iv);
          const int pos = __popcll(__ballot(ahead));
          const float ux = __shfl_up(lx, 1);
          const int ui = __shfl_up(li, 1);
          if (lane > pos) { lx = ux; li = ui; }
          if (lane == pos) { lx = xv; li = iv; }
          kx = rl_f(lx, k - 1);
          ki = rl_i(li, k - 1);
          tb = fmaxf(tb, kx);
        }
      }
    }
  };

  IO A, B;
  A.load(row, tile_base(0), end, beg, lane);
  for (int i = 0;; i += 2) {
    // prefetch the next tile (re-reading this one past the last: a cache hit)
    B.load(row, tile_base(i + 1 < nt ? i + 1 : i), end, beg, lane);
    process(A, i);
    if (i + 1 >= nt) break;
    A.load(row, tile_base(i + 2 < nt ? i + 2 : i + 1), end, beg, lane);
    process(B, i + 1);
    if (i + 2 >= nt) break;
  }

  __shared__ float s_m[NTP / 64];
  __shared__ float s_s[NTP / 64];
  __shared__ float s_lx[NTP / 64 * kMaxK];
  __shared__ int s_li[NTP / 64 * kMaxK];
  __shared__ float s_rx[kMaxK];
  __shared__ int s_rid[kMaxK];
  const float wm = wave_max(m);
  if (lane < k) { s_lx[wid * k + lane] = lx; s_li[wid * k + lane] = li; }
  if (lane == 0) s_m[wid] = wm;
  if (tid < k) { s_rx[tid] = -INFINITY; s_rid[tid] = -1; }
  __syncthreads();
  const float M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
  // NaN entries make a lane's sum NaN; a +inf entry does too (inf - inf)
  const float contrib = m == -INFINITY ? sum : sum * __builtin_amdgcn_exp2f((m - M) * kL2E);
  const float ws = wave_sum(contrib);
  if (lane == 0) s_s[wid] = ws;
  const int nc = (NTP / 64) * k;
  if (tid < nc) {
    const float cx = s_lx[tid];
    const int ci = s_li[tid];
    if (ci != INT_MAX) {
      int rank = 0;
      for (int j = 0; j < nc; ++j) rank += beats(s_lx[j], s_li[j], cx, ci);
      if (rank < k) { s_rx[rank] = cx; s_rid[rank] = ci; }
    }
  }
  __syncthreads();
  float* rec = part + (((size_t)b * R + r) * S + s) * kRec;
  if (tid < k) {  // logit, draft id, target token (id + d2t[id])
    const int id = s_rid[tid];
    rec[2 + tid] = s_rx[tid];
    reinterpret_cast<int*>(rec + 2 + kMaxK)[tid] = id;
    reinterpret_cast<int*>(rec + 2 + 2 * kMaxK)[tid] = id >= 0 && d2t ? id + d2t[id] : id;
  }
  if (tid == 0) {
    rec[0] = M;
    rec[1] = s_s[0] + s_s[1] + s_s[2] + s_s[3];
  }
}

// One wave per sequence: the first total_tokens entries of the best list
// (fewer if fewer nodes have a finite value) follow the root in pool order.
// A chosen entry's node id is 1 + the number of chosen entries with a lower
// pool index; its parent is chosen too and gets its id the same way.
__global__ __launch_bounds__(64) void tree_finalize_kernel(
    const int32_t* __restrict__ state, int k, int depth, int N, const int32_t* __restrict__ root_token,
    const int32_t* __restrict__ prefix_len, int n_max, int32_t* __restrict__ tokens,
    int32_t* __restrict__ parents, int32_t* __restrict__ n_nodes, int32_t* __restrict__ node_depth,
    int32_t* __restrict__ positions, uint64_t* __restrict__ anc_mask,
    int32_t* __restrict__ draft_row, float* __restrict__ value, int32_t* __restrict__ dev_error) {
  const int b = blockIdx.x, lane = threadIdx.x;
  SeqState st = seq_state(const_cast<int32_t*>(state), b, k, depth);
  __shared__ int s_p[64];
  __shared__ int s_exp[kMaxK * (kMaxDepth - 1)];
  __shared__ int s_par[SPEC_MAX_NODES];
  const int levels = st.hdr[0];
  const int failed = st.hdr[1];
  const int cnt = st.hdr[2];
  if (failed || levels < 1 || levels > depth || cnt < 0 || cnt > kBest) {
    if (lane == 0) {
      n_nodes[b] = 0;
      if (!failed) report(dev_error, SPEC_DEVERR_TREE);
    }
    return;
  }
  const int n = min(N, cnt);
  const int P = pool_size(k, levels);
  const int ne = (levels - 1) * k;
  const int p = lane < n ? st.best_id[lane] : INT_MAX;
  const float v = lane < n ? st.best_val[lane] : 0.f;
  s_p[lane] = p;
  for (int i = lane; i < ne; i += 64) s_exp[i] = st.expanded[i];
  __syncthreads();
  const size_t o = (size_t)b * n_max;
  const int L = prefix_len ? prefix_len[b] : 0;
  int bad = 0;
  int nd = 0, pn = 0;
  if (lane < n) {
    const int pp = (p >= 0 && p < P) ? st.parent[p] : INT_MAX;
    int before = 0, pbefore = 0, found = 0;
    for (int i = 0; i < n; ++i) {
      const int q = s_p[i];
      before += q < p;
      pbefore += q < pp;
      found |= q == pp;
    }
    // the parent precedes its child and is chosen with it (values never
    // rise along a path); anything else is a corrupted state
    if (p < 0 || p >= P || (pp >= 0 && (pp >= p || !found))) bad = 1;
    nd = 1 + before;
    pn = pp < 0 ? 0 : 1 + pbefore;
    int row = -1;
    for (int i = 0; i < ne; ++i) row = s_exp[i] == p ? 1 + i : row;
    const int d = level_of(k, p);
    if (!bad) {
      tokens[o + nd] = st.token[p];
      parents[o + nd] = pn;
      if (node_depth) node_depth[o + nd] = d;
      if (positions) positions[o + nd] = L + d;
      if (value) value[o + nd] = v;
      if (draft_row) draft_row[o + nd] = row;
      s_par[nd] = pn;
    }
  }
  if (lane == 0) {
    tokens[o] = root_token ? root_token[b] : -1;
    parents[o] = -1;
    s_par[0] = -1;
    if (node_depth) node_depth[o] = 0;
    if (positions) positions[o] = L;
    if (value) value[o] = 0.f;
    if (draft_row) draft_row[o] = 0;
  }
  if (__syncthreads_or(bad)) {
    if (lane == 0) {
      report(dev_error, SPEC_DEVERR_TREE);
      n_nodes[b] = 0;
    }
    return;
  }
  if (anc_mask && lane <= n) {
    uint64_t mask = 0;
    for (int x = lane; x >= 0; x = s_par[x]) mask |= 1ull << x;
    anc_mask[o + lane] = mask;
  }
  if (lane == 0) n_nodes[b] = n + 1;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Partials workgroups resident per compute unit (cached per kernel variant
// and device).
int resident_blocks(const void* kern) {
  static std::atomic<int> cache[4][64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  const int v = kern == reinterpret_cast<const void*>(tree_partials_kernel<float, true>)       ? 0
                : kern == reinterpret_cast<const void*>(tree_partials_kernel<float, false>)    ? 1
                : kern == reinterpret_cast<const void*>(tree_partials_kernel<uint16_t, true>) ? 2
                                                                                                : 3;
  int n = cache[v][dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, NTP, 0) != hipSuccess || n <= 0)
    n = 4;
  cache[v][dev].store(n, std::memory_order_relaxed);
  return n;
}

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
  if (Vd > kMaxVocab) return SPEC_E_SHAPE;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_E_DTYPE;
  if (state_bytes < state_bytes_for(B, top_k, depth) || !aligned16(state)) return SPEC_E_WORKSPACE;
  const int R = level == 1 ? 1 : top_k;
  const int W = dtype == SPEC_F32 ? 4 : 8;
  const bool vec = Vd % W == 0 && aligned16(draft_logits);
  const void* kern = dtype == SPEC_F32
                         ? (vec ? reinterpret_cast<const void*>(tree_partials_kernel<float, true>)
                                : reinterpret_cast<const void*>(tree_partials_kernel<float, false>))
                         : (vec ? reinterpret_cast<const void*>(tree_partials_kernel<uint16_t, true>)
                                : reinterpret_cast<const void*>(tree_partials_kernel<uint16_t, false>));
  // splits: as many workgroups as are resident at once (all start together
  // and stream equal shares), each streaming at least two block tiles where
  // the row allows
  const int resident = resident_blocks(kern) * device_cu_count();
  const int s_par = resident / (B * R) > 1 ? resident / (B * R) : 1;
  const int btile = block_tile<float>();
  const int s_len = Vd / (2 * btile) > 1 ? Vd / (2 * btile) : 1;
  int S = s_par < s_len ? s_par : s_len;
  if (S > max_splits(top_k)) S = max_splits(top_k);
  int chunk = (Vd + S - 1) / S;
  chunk = (chunk + 7) & ~7;
  S = (Vd + chunk - 1) / chunk;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* st = static_cast<int32_t*>(state);
  float* part = reinterpret_cast<float*>(static_cast<char*>(state) +
                                         partials_offset(B, top_k, depth));
  const dim3 grid(S, R, B);
  auto launch = [&](auto kern, const auto* lg) {
    hipLaunchKernelGGL(kern, grid, dim3(NTP), 0, s, lg, Vd, R, S, chunk, top_k, d2t, part);
  };
  if (dtype == SPEC_F32) {
    const float* lg = static_cast<const float*>(draft_logits);
    if (vec)
      launch(tree_partials_kernel<float, true>, lg);
    else
      launch(tree_partials_kernel<float, false>, lg);
  } else {
    const uint16_t* lg = static_cast<const uint16_t*>(draft_logits);
    if (vec)
      launch(tree_partials_kernel<uint16_t, true>, lg);
    else
      launch(tree_partials_kernel<uint16_t, false>, lg);
  }
  SPEC_HIP_TRY(hipGetLastError());
  hipLaunchKernelGGL(tree_select_kernel, dim3(B), dim3(NTS), 0, s, part, R, S, top_k, depth,
                     level, st, expanded_tokens, expanded_ids, dev_error);
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
  if (state_bytes < state_bytes_for(B, top_k, depth) || !aligned16(state)) return SPEC_E_WORKSPACE;
  hipLaunchKernelGGL(tree_finalize_kernel, dim3(B), dim3(64), 0,
                     static_cast<hipStream_t>(stream), static_cast<const int32_t*>(state), top_k,
                     depth, total_tokens, root_token, prefix_len, n_max, tokens, parents, n_nodes,
                     node_depth, positions, anc_mask, draft_row, value, dev_error);
  SPEC_HIP_TRY(hipGetLastError());
  return SPEC_OK;
}
