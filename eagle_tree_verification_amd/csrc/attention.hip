// Tree-masked attention for draft-tree verification (gfx950).
//
// Every draft-tree node attends to the whole committed prefix and to the
// nodes on its own root path, itself included: the verifier's attention uses
// a non-causal mask that follows the tree (page "推测解码与 EAGLE-3", section
// "KV cache 回滚"; page "EAGLE-1/2/3 拆解", section on EAGLE-2's two stages,
// identity initial tree mask; page "EAGLE-3 完全拆解", section on the
// training-time mask, ancestors only).  The tree rows sit right behind the
// prefix in the cache, so one sweep over keys [0, L + n) serves every node:
// prefix keys are visible to all nodes and key L + j is visible to node i iff
// bit j of i's ancestor mask is set.  Only the dot products the mask needs
// for the prefix part are dense; the tree part is one 64-key tile.
//
// Two implementations:
//   * attn_mfma_kernel (bf16, head_dim 128): one workgroup per (sequence,
//     KV head, row block, prefix split).  All n * (Hq/Hkv) query rows of a KV
//     head share each K/V tile, so the tile is streamed once from HBM into
//     LDS and every wave contracts it with its own 32- or 64-row Q block on
//     the matrix cores (v_mfma_f32_32x32x16_bf16).  Scores are produced
//     transposed (keys x query rows) so each lane owns one query row and the
//     online-softmax row statistics need a single cross-lane exchange.
//   * attn_valu_kernel (f32 or bf16, any head_dim): one wave per (sequence,
//     node, head) on the vector ALU; used for small or f32 problems.
// Splits of the prefix are merged by attn_merge_kernel (log-sum-exp).
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "common.hpp"

namespace specv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.f;  // log2 of the largest weight the online softmax lets through

// ---------------------------------------------------------------------------
// Tree validation and ancestor masks.  anc[j] has bit i set iff node i is on
// the root path of node j (j included).  Returns false for an invalid tree.
// par_t is this thread's entry of the parent row (thread t < n holds node
// t's parent), loaded by the caller together with the sequence's sizes: the
// row is staged in LDS (par_s, 64 ints) and every root path is walked there,
// so a deep tree costs LDS reads, not a chain of dependent global loads.
// Called by every thread of the block; blockDim.x >= 64.
// ---------------------------------------------------------------------------
__device__ bool build_ancestors(int par_t, int n, uint64_t* anc, int* par_s, int* flag) {
  const int t = threadIdx.x;
  if (t == 0) *flag = 0;
  if (t < n) par_s[t] = par_t;
  __syncthreads();
  if (t < n) {
    uint64_t m = 1ull << t;
    bool bad = (t == 0) ? (par_s[0] != -1) : false;
    int j = t;
    while (!bad && j > 0) {
      const int p = par_s[j];
      if (p < 0 || p >= j) {
        bad = true;
      } else {
        m |= 1ull << p;
        j = p;
      }
    }
    anc[t] = m;
    if (bad) atomicOr(flag, 1);
  }
  __syncthreads();
  return *flag == 0;
}

// ---------------------------------------------------------------------------
// Vector-ALU path: one wave per (b, node, query head).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void attn_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
    const int32_t* __restrict__ prefix_len, const int32_t* __restrict__ n_nodes,
    const int32_t* __restrict__ parents, int n_max, int Hq, int Hkv, int d, KvRows kv,
    float c, const float* __restrict__ inv_freq, int rope, float* __restrict__ out,
    int32_t* dev_error) {
  __shared__ uint64_t anc[64];
  __shared__ int flag;
  __shared__ int par_s[64];
  __shared__ int rows[64];
  __shared__ float qs[128];
  const int b = blockIdx.y;
  const int i = blockIdx.x / Hq;
  const int h = blockIdx.x % Hq;
  const int lane = threadIdx.x;
  const bool reporter = (blockIdx.x == 0 && lane == 0);
  const int n = n_nodes[b];
  const int L = prefix_len[b];
  const int par_t = lane < n_max ? parents[(size_t)b * n_max + lane] : -1;
  if (n < 1 || n > n_max) {
    if (reporter) report(dev_error, SPEC_DEVERR_TREE);
    return;
  }
  if (L < 0 || (int64_t)L + n > kv.L_cap) {
    if (reporter) report(dev_error, SPEC_DEVERR_CAPACITY);
    return;
  }
  if (!build_ancestors(par_t, n, anc, par_s, &flag)) {
    if (reporter) report(dev_error, SPEC_DEVERR_TREE);
    return;
  }
  if (!kv.blocks_ok(b, 0, L + n)) {
    if (reporter) report(dev_error, SPEC_DEVERR_CAPACITY);
    return;
  }
  if (i >= n) return;

  const uint64_t a = anc[i];
  const bool mine = lane < n && ((a >> lane) & 1ull);
  const uint64_t bal = __ballot(mine);
  if (mine) rows[__popcll(bal & ((1ull << lane) - 1ull))] = L + lane;
  const int npath = __popcll(bal);
  const int g = h / (Hq / Hkv);
  const T* qrow = q + (((size_t)b * n_max + i) * Hq + h) * d;
  for (int k = lane; k < d; k += 64) qs[k] = load_as_f32(qrow + k);
  __syncthreads();
  if (rope) {  // rotate the query at prefix_len + depth(i), in float32
    const int pos = L + __popcll(a) - 1;
    const int half = d / 2;
    for (int t = lane; t < half; t += 64) {
      const int ia = rope == kRopeInterleaved ? 2 * t : t;
      const int ib = rope == kRopeInterleaved ? 2 * t + 1 : t + half;
      float cs, sn;
      rope_cs(pos, inv_freq[t], &cs, &sn);
      const float x = qs[ia], y = qs[ib];
      qs[ia] = x * cs - y * sn;
      qs[ib] = y * cs + x * sn;
    }
    __syncthreads();
  }

  const int total = L + npath;
  float m = -INFINITY, l = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int c0 = 0; c0 < total; c0 += 64) {
    const int t = c0 + lane;
    const bool valid = t < total;
    const int row = valid ? (t < L ? t : rows[t - L]) : 0;
    float s = -INFINITY;
    if (valid) {
      const T* kr = kc + kv.offset(b, g, row, d);
      float dot = 0.f;
      for (int k = 0; k < d; ++k) dot = fmaf(qs[k], load_as_f32(kr + k), dot);
      s = dot * c;
    }
    const float mn = fmaxf(m, wave_max(s));
    const float alpha = exp2f(m - mn);
    const float p = valid ? exp2f(s - mn) : 0.f;
    l = l * alpha + wave_sum(p);
    acc0 *= alpha;
    acc1 *= alpha;
    const int cnt = min(64, total - c0);
    for (int kk = 0; kk < cnt; ++kk) {
      const float w = __shfl(p, kk);
      const int r = __shfl(row, kk);
      const T* vr = vc + kv.offset(b, g, r, d);
      if (lane < d) acc0 = fmaf(w, load_as_f32(vr + lane), acc0);
      if (lane + 64 < d) acc1 = fmaf(w, load_as_f32(vr + lane + 64), acc1);
    }
    m = mn;
  }
  float* orow = out + (((size_t)b * n_max + i) * Hq + h) * d;
  const float inv = 1.f / l;
  if (lane < d) orow[lane] = acc0 * inv;
  if (lane + 64 < d) orow[lane + 64] = acc1 * inv;
}

// ---------------------------------------------------------------------------
// Matrix-core path (bf16, head_dim 128).
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int KT = 64;              // keys per tile
constexpr int HD = 128;             // head dim
constexpr int KS_STRIDE = HD + 8;   // K tile row stride in LDS (bf16 elements): 272 B
// V tile row stride: 320 B, so the four key rows one transpose read touches
// per 32 lanes start 64 B apart modulo the 256 B of LDS banks.
constexpr int VS_STRIDE = HD + 32;
typedef short v4i16_t __attribute__((ext_vector_type(4)));

struct MfmaArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* prefix_len;
  const int32_t* n_nodes;
  const int32_t* parents;
  int B, n_max, Hq, Hkv, G, L_cap;
  KvRows kv;   // where cache rows live (contiguous, or paged through a block table)
  int RB;      // row blocks per (b, g)
  int S_max;   // prefix splits
  int chunk;   // prefix keys per split (multiple of KT)
  int units;   // B * Hkv * S_max
  int sort;    // map units to sequences longest prefix first
  float c;     // scale * log2(e)
  const float* inv_freq;  // rotary frequencies [HD/2], or null
  int rope;               // 0: none; kRopeHalf or kRopeInterleaved
  float* out;
  float* part_o;     // [B*Hkv][RB*RPW][S_max][HD]
  float2* part_ml;   // [B*Hkv][RB*RPW][S_max]  (running max, running sum)
  int32_t* dev_error;
};

// 2^x on the hardware's transcendental unit (v_exp_f32): results below the
// normal range flush to zero, which is harmless for softmax weights.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// PAGED: cache rows are found through the block table (a.kv); otherwise the
// cache is contiguous and the kernel never looks at a.kv.table.
template <int NB, int NW, int SUB, bool PAGED, bool PIPE = false>
__global__ __launch_bounds__(NW * 64) void attn_mfma_kernel(MfmaArgs a) {
  constexpr int NT = NW * 64;
  constexpr int RPW = NW * NB * 32;                    // query rows per workgroup
  constexpr int ST = SUB * KT;                         // keys per load stage
  constexpr int CH = ST * HD / 8 / NT;                 // 16-byte chunks per thread per stage (K or V)
  static_assert(CH * NT * 8 == ST * HD, "stage split");

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][ST * KS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][ST * VS_STRIDE];
  __shared__ uint64_t anc[64];
  __shared__ int flag;
  __shared__ int par_s[64];
  __shared__ int sorted_b;
  __shared__ int lens[256];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 31;
  const int lh = lane >> 5;

  // Block index -> (unit, row block).  The row blocks of one unit land on the
  // same XCD (same blockIdx mod 8) and are dispatched close together, so the
  // second one reads the unit's K/V from that XCD's L2.
  const int w = blockIdx.x;
  const int rb = (w >> 3) % a.RB;
  const int u = (w / (8 * a.RB)) * 8 + (w & 7);
  if (u >= a.units) return;
  const int s = u % a.S_max;
  const int g = (u / a.S_max) % a.Hkv;
  const int rank = u / (a.S_max * a.Hkv);
  int b = rank;
  if (a.sort) {
    // rank-th longest prefix (ties: lower sequence id first)
    for (int t = tid; t < a.B; t += NT) lens[t] = a.prefix_len[t];
    __syncthreads();
    for (int t = tid; t < a.B; t += NT) {
      const int Lt = lens[t];
      int r = 0;
      for (int j = 0; j < a.B; ++j) {
        const int Lj = lens[j];
        r += (Lj > Lt) || (Lj == Lt && j < t);
      }
      if (r == rank) sorted_b = t;
    }
    __syncthreads();
    b = sorted_b;
  }

  const int n = a.n_nodes[b];
  const int L = a.prefix_len[b];
  const int par_t = tid < a.n_max ? a.parents[(size_t)b * a.n_max + tid] : -1;
  const bool reporter = (g == 0 && rb == 0 && s == 0 && tid == 0);
  if (n < 1 || n > a.n_max) {
    if (reporter) report(a.dev_error, SPEC_DEVERR_TREE);
    return;
  }
  if (L < 0 || (int64_t)L + n > a.L_cap) {
    if (reporter) report(a.dev_error, SPEC_DEVERR_CAPACITY);
    return;
  }
  const int nsplit = L > 0 ? (L + a.chunk - 1) / a.chunk : 1;
  if (s >= nsplit) return;
  const int Mb = n * a.G;
  if (rb * RPW >= Mb) return;
  if (!build_ancestors(par_t, n, anc, par_s, &flag)) {
    if (reporter) report(a.dev_error, SPEC_DEVERR_TREE);
    return;
  }
  if (PAGED && !a.kv.blocks_ok(b, 0, L + n)) {
    if (reporter) report(a.dev_error, SPEC_DEVERR_CAPACITY);
    return;
  }
  const bool last = (s == nsplit - 1);

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds query row lr of
  // its 32-row block, head dims 16*ks + 8*lh .. +7.
  bf16x8_t qf[NB][8];
  uint64_t anc_r[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int r = rb * RPW + (wave * NB + nb) * 32 + lr;
    const bool valid = r < Mb;
    const int i = valid ? r / a.G : 0;
    const int hh = valid ? r % a.G : 0;
    anc_r[nb] = valid ? anc[i] : 0ull;
    const uint16_t* qp = a.q + (((size_t)b * a.n_max + i) * a.Hq + (size_t)g * a.G + hh) * HD + lh * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      qf[nb][ks] = valid ? *reinterpret_cast<const bf16x8_t*>(qp + ks * 16) : bf16x8_t{};
    if (a.rope && valid) {
      // Rotary embedding of the query at prefix_len + depth(i), rounded back
      // to bf16.  The lane holds dims 16*ks + 8*lh + e: the pair (t, t + 64)
      // of the half layout is (qf[ks][e], qf[ks + 4][e]); the pair (2t, 2t+1)
      // of the interleaved layout is (qf[ks][e], qf[ks][e + 1]).
      const int pos = L + __popcll(anc_r[nb]) - 1;
      if (a.rope == kRopeHalf) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float cs, sn;
            rope_cs(pos, a.inv_freq[16 * ks + 8 * lh + e], &cs, &sn);
            const float x = (float)qf[nb][ks][e], y = (float)qf[nb][ks + 4][e];
            qf[nb][ks][e] = (__bf16)(x * cs - y * sn);
            qf[nb][ks + 4][e] = (__bf16)(y * cs + x * sn);
          }
      } else {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            float cs, sn;
            rope_cs(pos, a.inv_freq[(16 * ks + 8 * lh + e) >> 1], &cs, &sn);
            const float x = (float)qf[nb][ks][e], y = (float)qf[nb][ks][e + 1];
            qf[nb][ks][e] = (__bf16)(x * cs - y * sn);
            qf[nb][ks][e + 1] = (__bf16)(y * cs + x * sn);
          }
      }
    }
  }

  f32x16_t o[NB][4];
  float mrow[NB], lrow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    mrow[nb] = -INFINITY;
    lrow[nb] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) o[nb][db] = f32x16_t{};
  }

  const size_t bg = (size_t)b * a.Hkv + g;
  const uint16_t* kbg = a.k + bg * (size_t)a.L_cap * HD;
  const uint16_t* vbg = a.v + bg * (size_t)a.L_cap * HD;
  const int kb0 = s * a.chunk;
  const int ke0 = min(L, kb0 + a.chunk);
  const int ntp = ke0 > kb0 ? (ke0 - kb0 + ST - 1) / ST : 0;  // prefix stages
  const int nt = ntp + (last ? 1 : 0);                        // + the tree stage

  // Stage t: rows [row0, row0 + nrows) of the cache.
  auto stage_rows = [&](int t, int& row0, int& nrows) {
    row0 = t < ntp ? kb0 + t * ST : L;
    nrows = t < ntp ? min(ST, ke0 - row0) : n;
  };

  // Paged: the physical block of each of this thread's rows of a stage,
  // read from the block table one stage before the rows themselves, so the
  // table's latency never delays the K/V loads.  The read is unconditional
  // (index clamped into the sequence's table row): a conditional one would
  // leave a register copy that waits for every outstanding load.  Entries
  // for rows past the stage are never used.
  int tblk[CH];
  auto table_entries = [&](int t) {
    if constexpr (PAGED) {
      int row0, nrows;
      stage_rows(t, row0, nrows);
      const int32_t* trow = a.kv.table + (size_t)b * a.kv.max_blocks;
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int r = (tid + j * NT) >> 4;
        tblk[j] = trow[min((row0 + r) >> a.kv.bs_log2, a.kv.max_blocks - 1)];
      }
    }
  };

  uint4 kreg[CH], vreg[CH];
  auto load_stage = [&](int t) {
    int row0, nrows;
    stage_rows(t, row0, nrows);
    if constexpr (PAGED) {
      const int mask = (1 << a.kv.bs_log2) - 1;
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int cidx = tid + j * NT;
        const int r = cidx >> 4;
        const size_t off = ((((size_t)tblk[j] * a.Hkv + g) << a.kv.bs_log2) + ((row0 + r) & mask)) *
                               HD + (cidx & 15) * 8;
        kreg[j] = r < nrows ? *reinterpret_cast<const uint4*>(a.k + off) : make_uint4(0, 0, 0, 0);
        vreg[j] = r < nrows ? *reinterpret_cast<const uint4*>(a.v + off) : make_uint4(0, 0, 0, 0);
      }
    } else {
      const uint16_t* kbase = kbg + (size_t)row0 * HD;
      const uint16_t* vbase = vbg + (size_t)row0 * HD;
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int cidx = tid + j * NT;
        const int r = cidx >> 4;
        const size_t off = (size_t)r * HD + (cidx & 15) * 8;
        kreg[j] = r < nrows ? *reinterpret_cast<const uint4*>(kbase + off) : make_uint4(0, 0, 0, 0);
        vreg[j] = r < nrows ? *reinterpret_cast<const uint4*>(vbase + off) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int cidx = tid + j * NT;
      *reinterpret_cast<uint4*>(Ks[buf] + (cidx >> 4) * KS_STRIDE + (cidx & 15) * 8) = kreg[j];
      *reinterpret_cast<uint4*>(Vs[buf] + (cidx >> 4) * VS_STRIDE + (cidx & 15) * 8) = vreg[j];
    }
  };

  // Transpose-read source of this lane for the V^T operand of one 32x32x16
  // contraction step: within each 16-lane group the read hands lane d the
  // (d % 4)-th entry of the 8-byte chunks of lanes 4j + d / 4, j = 0..3, so
  // lane L points at key row 4 (L / 32) + (L % 16) / 4 of the step's key
  // block and head dims 16 ((L / 16) % 2) + 4 (L % 4) .. +3 of the dim block;
  // it receives head dim L % 32 of keys 4 (L / 32) + 0..3 (and, from the
  // second read 8 keys further on, keys 8 + 4 (L / 32) + 0..3), matching the
  // key order of the P^T operand taken straight from the score accumulators.
  const int tr_key = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int tr_dim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  const float cs = a.c;
  // One 64-key sub-tile: keys [64 * sub, 64 * sub + nrows) of the stage.
  auto compute_sub = [&](int buf, int sub, int nrows, bool tree) {
    // S^T (keys x rows) for the two 32-key halves of the sub-tile.
    f32x16_t sacc[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      sacc[nb][0] = f32x16_t{};
      sacc[nb][1] = f32x16_t{};
    }
    const uint16_t* ks_ = Ks[buf] + sub * KT * KS_STRIDE;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(ks_ + (kb * 32 + lr) * KS_STRIDE + ks * 16 + lh * 8);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          sacc[nb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[nb][ks], sacc[nb][kb], 0, 0, 0);
      }
    }

    // Mask only the ragged last prefix sub-tile and the tree tile (uniform).
    // Lane (lr, lh) holds keys 8*gq + 4*lh + e4 of each 32-key half.
    if (tree || nrows < KT) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kb * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
            const bool vis = key < nrows && (!tree || ((anc_r[nb] >> key) & 1ull));
            if (!vis) sacc[nb][kb][e] = -INFINITY;
          }
    }

    // Online softmax with the rescale of O skipped unless a row max moved.
    bf16x8_t pf[NB][2][2];
    float alpha[NB];
    int moved = 0;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mt = fmaxf(mt, sacc[nb][kb][e]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      // The reference max moves only when the row max exceeds it by more
      // than 2^kLazy in weight (always at the first finite score), so O and l
      // are rarely rescaled; weights stay <= 2^kLazy, harmless in fp32 and
      // bf16, and O and l always share one reference.
      const bool up = (mt - mrow[nb]) * cs > kLazy;
      const float mn = up ? mt : mrow[nb];
      const float mu = (mn == -INFINITY) ? 0.f : mn;
      const float muc = mu * cs;
      alpha[nb] = up ? fast_exp2(mrow[nb] * cs - muc) : 1.f;
      moved |= up;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = fast_exp2(fmaf(sacc[nb][kb][e], cs, -muc));
          ls += p;
          pf[nb][kb][e >> 3][e & 7] = static_cast<__bf16>(p);
        }
      lrow[nb] = lrow[nb] * alpha[nb] + ls;
      mrow[nb] = mn;
    }
    if (__any(moved)) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int db = 0; db < 4; ++db) o[nb][db] *= alpha[nb];
    }

    // O^T (dims x rows) += V^T P^T, V^T gathered by LDS transpose reads.
    const uint16_t* vs_ = Vs[buf] + (sub * KT + tr_key) * VS_STRIDE + tr_dim;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const uint16_t* src = vs_ + (kb * 32 + hb * 16) * VS_STRIDE + db * 32;
          const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (v4i16_t __attribute__((address_space(3)))*)(src));
          const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (v4i16_t __attribute__((address_space(3)))*)(src + 8 * VS_STRIDE));
          const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            o[nb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[nb][kb][hb], o[nb][db], 0, 0, 0);
        }
      }
    }
  };

  // Pipelined order (PIPE, two sub-tiles per stage): the PV product of the
  // previous sub-tile is issued step by step between the exponentials of
  // the current one, so each wave's matrix and vector work overlap.  The
  // operations on O keep their order (the previous sub-tile's PV, then the
  // current rescale, then the current PV one sub-tile later), so the result
  // equals the plain order's bit for bit.  The pending sub-tile's weights
  // sit in pfA at the end of every stage, its keys in (pbuf, psub); the
  // first pending product is of zero weights.
  // (pipelined order) S^T (keys x rows) of the sub-tile of keys
  // [64 * sub, 64 * sub + nrows) of the stage in buffer buf, for its two
  // 32-key halves, masked.  The plain order keeps its own inline copy of
  // these lines: routing both through one helper changed the code generated
  // for the other variants and made them slower.
  auto qk = [&](int buf, int sub, int nrows, bool tree, f32x16_t (*sacc)[2]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      sacc[nb][0] = f32x16_t{};
      sacc[nb][1] = f32x16_t{};
    }
    const uint16_t* ks_ = Ks[buf] + sub * KT * KS_STRIDE;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(ks_ + (kb * 32 + lr) * KS_STRIDE + ks * 16 + lh * 8);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          sacc[nb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[nb][ks], sacc[nb][kb], 0, 0, 0);
      }
    }

    // Mask only the ragged last prefix sub-tile and the tree tile (uniform).
    // Lane (lr, lh) holds keys 8*gq + 4*lh + e4 of each 32-key half.
    if (tree || nrows < KT) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kb * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
            const bool vis = key < nrows && (!tree || ((anc_r[nb] >> key) & 1ull));
            if (!vis) sacc[nb][kb][e] = -INFINITY;
          }
    }
  };

  // V^T operand of contraction step `step` (key block step / 8, half
  // (step / 4) % 2, dim block step % 4) of the sub-tile whose transpose-read
  // base is vs_.
  auto vread = [&](const uint16_t* vs_, int step) {
    const int kb = step >> 3, hb = (step >> 2) & 1, db = step & 3;
    const uint16_t* src = vs_ + (kb * 32 + hb * 16) * VS_STRIDE + db * 32;
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (v4i16_t __attribute__((address_space(3)))*)(src));
    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (v4i16_t __attribute__((address_space(3)))*)(src + 8 * VS_STRIDE));
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  bf16x8_t pfA[NB][2][2], pfB[NB][2][2];
  int pbuf = 0, psub = 0;
  if constexpr (PIPE) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) pfA[nb][kb][hb] = bf16x8_t{};
  }
  // One sub-tile in the pipelined order: its scores, the softmax reductions,
  // then 16 steps of (one PV instruction of the pending sub-tile, two of
  // this sub-tile's exponentials), then the rescale.  pold holds the pending
  // weights, pnew receives this sub-tile's.
  auto piped_sub = [&](int buf, int sub, int nrows, bool tree, bf16x8_t (*pnew)[2][2],
                       bf16x8_t (*pold)[2][2]) {
    f32x16_t sacc[NB][2];
    qk(buf, sub, nrows, tree, sacc);
    float alpha[NB], muc[NB], ls[NB];
    int moved = 0;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mt = fmaxf(mt, sacc[nb][kb][e]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      // the lazy reference max of the plain order
      const bool up = (mt - mrow[nb]) * cs > kLazy;
      const float mn = up ? mt : mrow[nb];
      const float mu = (mn == -INFINITY) ? 0.f : mn;
      muc[nb] = mu * cs;
      alpha[nb] = up ? fast_exp2(mrow[nb] * cs - muc[nb]) : 1.f;
      moved |= up;
      mrow[nb] = mn;
      ls[nb] = 0.f;
    }
    // the transposed V reads run two steps ahead of their product
    const uint16_t* vs_ = Vs[pbuf] + (psub * KT + tr_key) * VS_STRIDE + tr_dim;
    bf16x8_t vf_q[3];
    vf_q[0] = vread(vs_, 0);
    vf_q[1] = vread(vs_, 1);
    // raised issue priority while this wave interleaves matrix and vector
    // work, so the SIMD's other wave (in its score phase) fills the gaps
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int step = 0; step < 16; ++step) {
      const int kb = step >> 3, hb = (step >> 2) & 1, db = step & 3;
      const bf16x8_t vf = vf_q[step % 3];
      if (step + 2 < 16) vf_q[(step + 2) % 3] = vread(vs_, step + 2);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        o[nb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pold[nb][kb][hb], o[nb][db], 0, 0, 0);
      // scores 2 step and 2 step + 1 of the 32 this lane holds, in the plain
      // order's summation order
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int idx = 2 * step + q, skb = idx >> 4, e = idx & 15;
          float pw = fast_exp2(fmaf(sacc[nb][skb][e], cs, -muc[nb]));
          // An empty asm ties each exponential to its step: without it the
          // exponentials, whose results are not needed until the next
          // sub-tile, all sink below the 16 matrix instructions.
          asm volatile("" : "+v"(pw));
          ls[nb] += pw;
          pnew[nb][skb][e >> 3][e & 7] = static_cast<__bf16>(pw);
        }
      // nothing crosses a step boundary
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) lrow[nb] = lrow[nb] * alpha[nb] + ls[nb];
    if (__any(moved)) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int db = 0; db < 4; ++db) o[nb][db] *= alpha[nb];
    }
    pbuf = buf;
    psub = sub;
  };

  if (nt > 0) {
    table_entries(0);
    load_stage(0);
    store_stage(0);
    if (nt > 1) table_entries(1);
    __syncthreads();
  }
  if constexpr (PAGED) {
    // Every load issued so far (the Q fragments included) has completed on
    // all paths into the loop.  Without this the compiler cannot prove the
    // Q registers ready at the loop's first matrix instruction (the block
    // check and table reads add paths) and waits there for every load in
    // flight, the next stage's K/V too, every iteration.
    __builtin_amdgcn_s_waitcnt(0);
  }
  for (int t = 0; t < nt; ++t) {
    const int buf = t & 1;
    if (t + 1 < nt) {
      load_stage(t + 1);
      if (t + 2 < nt) table_entries(t + 2);
    }
    int row0, nrows;
    stage_rows(t, row0, nrows);
    const bool tree = (t >= ntp);
    if constexpr (PIPE) {
      static_assert(SUB == 2, "the pipelined order alternates two weight buffers");
      piped_sub(buf, 0, min(KT, nrows), tree, pfB, pfA);
      if (nrows > KT) {
        piped_sub(buf, 1, min(KT, nrows - KT), tree, pfA, pfB);
      } else {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) pfA[nb][kb][hb] = pfB[nb][kb][hb];
      }
      // The store below overwrites the other buffer, whose last sub-tile
      // the first product above read: every wave must be past it.
      __syncthreads();
    } else {
#pragma unroll
      for (int sub = 0; sub < SUB; ++sub) {
        const int rows_sub = nrows - sub * KT;
        if (rows_sub <= 0) break;
        compute_sub(buf, sub, min(KT, rows_sub), tree);
      }
    }
    if (t + 1 < nt) store_stage(buf ^ 1);
    __syncthreads();
  }
  if constexpr (PIPE) {
    // the last sub-tile's product
    if (nt > 0) {
      const uint16_t* vs_ = Vs[pbuf] + (psub * KT + tr_key) * VS_STRIDE + tr_dim;
#pragma unroll
      for (int step = 0; step < 16; ++step) {
        const int kb = step >> 3, hb = (step >> 2) & 1, db = step & 3;
        const bf16x8_t vf = vread(vs_, step);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          o[nb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pfA[nb][kb][hb], o[nb][db], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: lane holds dims db*32 + 8*gq + 4*lh + e4 of its query row.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float lt = lrow[nb] + __shfl_xor(lrow[nb], 32);
    const int r = rb * RPW + (wave * NB + nb) * 32 + lr;
    if (r >= Mb) continue;
    const int i = r / a.G;
    const int hh = r % a.G;
    if (a.S_max == 1) {
      const float inv = 1.f / lt;
      float* op = a.out + (((size_t)b * a.n_max + i) * a.Hq + (size_t)g * a.G + hh) * HD;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
          *reinterpret_cast<float4*>(op + db * 32 + gq * 8 + lh * 4) =
              make_float4(o[nb][db][gq * 4 + 0] * inv, o[nb][db][gq * 4 + 1] * inv,
                          o[nb][db][gq * 4 + 2] * inv, o[nb][db][gq * 4 + 3] * inv);
    } else {
      const size_t prow = (bg * (size_t)(a.RB * RPW) + r) * a.S_max + s;
      float* pp = a.part_o + prow * HD;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
          *reinterpret_cast<float4*>(pp + db * 32 + gq * 8 + lh * 4) =
              make_float4(o[nb][db][gq * 4 + 0], o[nb][db][gq * 4 + 1], o[nb][db][gq * 4 + 2],
                          o[nb][db][gq * 4 + 3]);
      if (lh == 0) a.part_ml[prow] = make_float2(mrow[nb], lt);
    }
  }
}

// Log-sum-exp merge of prefix splits.  32 lanes per query row, four head
// dims each (16-byte loads and stores); a 256-thread block merges
// kMergeRows rows of one (sequence, KV head).  The parent row is read with
// the sequence's sizes, so a block waits for one round trip before its tree
// check.  Per element the splits are combined in split order, as ever.
constexpr int kMergeRows = 8;
__global__ __launch_bounds__(32 * kMergeRows) void attn_merge_kernel(MfmaArgs a,
                                                                     int rows_per_bg) {
  static_assert(HD == 32 * 4, "32 lanes of four dims cover a row");
  const int tid = threadIdx.x;
  const int r = blockIdx.x * kMergeRows + (tid >> 5);
  const int lane = tid & 31;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int n = a.n_nodes[b];
  const int L = a.prefix_len[b];
  const int par_t = tid < a.n_max ? a.parents[(size_t)b * a.n_max + tid] : -1;
  if (n < 1 || n > a.n_max || L < 0 || (int64_t)L + n > a.L_cap) return;
  if (blockIdx.x * kMergeRows >= n * a.G) return;
  // an invalid tree was skipped by the main kernel; skip it here as well
  __shared__ int bad;
  if (tid == 0) bad = 0;
  __syncthreads();
  if (tid < n && (tid == 0 ? par_t != -1 : (par_t < 0 || par_t >= tid))) atomicOr(&bad, 1);
  __syncthreads();
  if (bad) return;
  // so was a sequence whose rows sit in a block outside the pool
  if (a.kv.table && !a.kv.blocks_ok(b, 0, L + n)) return;
  if (r >= n * a.G) return;
  const int nsplit = L > 0 ? (L + a.chunk - 1) / a.chunk : 1;
  const size_t base = (((size_t)b * a.Hkv + g) * rows_per_bg + r) * a.S_max;
  float mstar = -INFINITY;
  for (int s = 0; s < nsplit; ++s) mstar = fmaxf(mstar, a.part_ml[base + s].x);
  float lsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < nsplit; ++s) {
    const float2 ml = a.part_ml[base + s];
    const float wgt = fast_exp2((ml.x - mstar) * a.c);
    lsum += ml.y * wgt;
    const float4 po = *reinterpret_cast<const float4*>(a.part_o + (base + s) * HD + lane * 4);
    acc.x += po.x * wgt;
    acc.y += po.y * wgt;
    acc.z += po.z * wgt;
    acc.w += po.w * wgt;
  }
  const int i = r / a.G;
  const int hh = r % a.G;
  *reinterpret_cast<float4*>(a.out + (((size_t)b * a.n_max + i) * a.Hq + (size_t)g * a.G + hh) * HD +
                             lane * 4) =
      make_float4(acc.x / lsum, acc.y / lsum, acc.z / lsum, acc.w / lsum);
}

// ---------------------------------------------------------------------------
// Host planning.
// ---------------------------------------------------------------------------
struct Plan {
  bool mfma = false;
  int nb = 0, nw = 0, sub = 1, rpw = 0, rb = 0, S_max = 1, chunk = 0, units = 0, sort = 0;
  bool pipe = false;
  size_t ws = 0;
};

Plan make_plan(int B, int n_max, int Hq, int Hkv, int d, int L_cap, int dtype) {
  Plan p;
  p.mfma = (dtype == SPEC_BF16 && d == HD);
  if (!p.mfma) return p;
  const int G = Hq / Hkv;
  const int M = n_max * G;
  const long cus = device_cu_count();
  const long smax_by_len = (L_cap + 127) / 128;  // splits keep >= 128 keys
  if (M <= 64) {
    p.nb = 1; p.nw = 2;
  } else if (M <= 128) {
    p.nb = 1; p.nw = 4;
  } else {
    p.nb = 1; p.nw = 8; p.sub = 2;
    // Few (sequence, head) units and short prefixes leave the 8-wave kernel
    // fewer workgroups than CUs even at the most splits; 2-wave workgroups
    // of 64 rows then fill the GPU (their row blocks re-read K/V from the
    // XCD's L2).  Measured on one sequence of the 8B layout: 32 -> 25 us.
    const long units8 = (long)B * Hkv * ((M + 255) / 256);
    if (units8 * smax_by_len < cus) {
      p.nw = 2; p.sub = 1;
    }
  }
  if (const char* env = getenv("SPEC_ATTN_VARIANT")) {  // "NBxNW[xSUB]", tuning sweeps
    int nb = 0, nw = 0;
    int sub = 1;
    if (sscanf(env, "%dx%dx%d", &nb, &nw, &sub) >= 2 &&
        ((nb == 1 && (nw == 2 || nw == 4 || nw == 8)) || (nb == 2 && nw == 4))) {
      p.nb = nb; p.nw = nw;
      p.sub = (nb == 1 && nw == 8 && sub == 2) ? 2 : 1;
    }
  }
  // The two-sub-tile variant runs in the pipelined order (SPEC_ATTN_PIPE=0:
  // the plain order, for comparisons).
  p.pipe = p.sub == 2;
  if (const char* env = getenv("SPEC_ATTN_PIPE")) p.pipe = p.pipe && env[0] != '0';
  p.rpw = p.nw * p.nb * 32;
  p.rb = (M + p.rpw - 1) / p.rpw;
  const long base = (long)B * Hkv * p.rb;
  // Split the prefix until about one workgroup per CU: the 8-wave kernel's
  // stages fill a CU's LDS, and every further split only adds partial
  // outputs to write and merge (measured: a 16-sequence 70B-layout batch
  // runs 22% faster unsplit than in two splits, an 8-way KV-head shard 25%
  // faster in 4 splits than in 8).
  const long target = cus;
  long S = base >= target ? 1 : (target + base - 1) / base;
  if (const char* env = getenv("SPEC_ATTN_SPLITS")) {  // prefix splits, tuning sweeps
    const long v = atol(env);
    if (v >= 1) S = v;
  }
  if (S > smax_by_len) S = smax_by_len;
  if (S < 1) S = 1;
  long chunk = (L_cap + S - 1) / S;
  chunk = (chunk + KT - 1) / KT * KT;
  p.chunk = (int)chunk;
  p.S_max = (int)((L_cap + chunk - 1) / chunk);
  p.units = B * Hkv * p.S_max;
  p.sort = (p.S_max == 1 && B >= 8 && B <= 256) ? 1 : 0;
  if (p.S_max > 1) {
    const size_t rows = (size_t)B * Hkv * p.rb * p.rpw * p.S_max;
    p.ws = rows * HD * sizeof(float) + rows * sizeof(float2) + 256;
  }
  return p;
}

spec_status_t check_args(const void* q, const void* k, const void* v, const int32_t* pl,
                         const int32_t* nn, const int32_t* par, int B, int n_max, int Hq,
                         int Hkv, int d, int L_cap, float scale, int dtype, const float* out,
                         bool paged) {
  if (!q || !k || !v || !pl || !nn || !par || !out) return SPEC_E_NULL;
  if (B <= 0 || n_max <= 0 || n_max > SPEC_MAX_NODES || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 ||
      L_cap < n_max)
    return SPEC_E_SHAPE;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_E_DTYPE;
  if (d != 16 && d != 32 && d != 64 && d != 128) return SPEC_E_DTYPE;
  if (!(scale > 0.f) || !isfinite(scale)) return SPEC_E_VALUE;
  // query rows and cache rows are counted in 32-bit ints (grid sizes, row
  // indices); byte offsets are 64-bit
  if ((long)B * n_max * Hq > (1L << 30) || (!paged && (long)B * Hkv * L_cap >= (1L << 31)))
    return SPEC_E_SHAPE;
  return SPEC_OK;
}

}  // namespace
}  // namespace specv

using namespace specv;

extern "C" size_t spec_verify_tree_attn_workspace_size(int32_t B, int32_t n_max, int32_t Hq,
                                                      int32_t Hkv, int32_t head_dim, int32_t L_cap,
                                                      int32_t dtype) {
  if (B <= 0 || n_max <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || L_cap <= 0) return 0;
  return make_plan(B, n_max, Hq, Hkv, head_dim, L_cap, dtype).ws;
}

namespace {
template <bool PAGED>
void launch_variant(const Plan& p, unsigned grid, hipStream_t strm, const MfmaArgs& a) {
  if (p.nb == 1 && p.nw == 2)
    hipLaunchKernelGGL((attn_mfma_kernel<1, 2, 1, PAGED>), dim3(grid), dim3(128), 0, strm, a);
  else if (p.nb == 1 && p.nw == 4)
    hipLaunchKernelGGL((attn_mfma_kernel<1, 4, 1, PAGED>), dim3(grid), dim3(256), 0, strm, a);
  else if (p.nb == 1 && p.nw == 8 && p.sub == 2 && p.pipe)
    hipLaunchKernelGGL((attn_mfma_kernel<1, 8, 2, PAGED, true>), dim3(grid), dim3(512), 0, strm,
                       a);
  else if (p.nb == 1 && p.nw == 8 && p.sub == 2)
    hipLaunchKernelGGL((attn_mfma_kernel<1, 8, 2, PAGED>), dim3(grid), dim3(512), 0, strm, a);
  else if (p.nb == 1 && p.nw == 8)
    hipLaunchKernelGGL((attn_mfma_kernel<1, 8, 1, PAGED>), dim3(grid), dim3(512), 0, strm, a);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<2, 4, 1, PAGED>), dim3(grid), dim3(256), 0, strm, a);
}

spec_status_t launch_attn(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* prefix_len, const int32_t* n_nodes,
                          const int32_t* parents, int32_t B, int32_t n_max, int32_t Hq,
                          int32_t Hkv, int32_t head_dim, const KvRows& kv, float scale,
                          int32_t dtype, const float* inv_freq, int rope, float* out,
                          void* workspace, size_t workspace_bytes, int32_t* dev_error,
                          void* stream) {
  spec_status_t st = check_args(q, k_cache, v_cache, prefix_len, n_nodes, parents, B, n_max, Hq,
                                Hkv, head_dim, kv.L_cap, scale, dtype, out, kv.table != nullptr);
  if (st != SPEC_OK) return st;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  const float c = scale * kLog2e;
  const int L_cap = kv.L_cap;
  const Plan p = make_plan(B, n_max, Hq, Hkv, head_dim, L_cap, dtype);
  if (!p.mfma) {
    dim3 grid(n_max * Hq, B);
    if (dtype == SPEC_F32) {
      hipLaunchKernelGGL(attn_valu_kernel<float>, grid, dim3(64), 0, strm,
                         static_cast<const float*>(q), static_cast<const float*>(k_cache),
                         static_cast<const float*>(v_cache), prefix_len, n_nodes, parents, n_max,
                         Hq, Hkv, head_dim, kv, c, inv_freq, rope, out, dev_error);
    } else {
      hipLaunchKernelGGL(attn_valu_kernel<uint16_t>, grid, dim3(64), 0, strm,
                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                         static_cast<const uint16_t*>(v_cache), prefix_len, n_nodes, parents, n_max,
                         Hq, Hkv, head_dim, kv, c, inv_freq, rope, out, dev_error);
    }
    SPEC_HIP_TRY(hipGetLastError());
    return SPEC_OK;
  }
  // 16-byte vector loads and stores (Q and K/V fragments, output rows,
  // split partials)
  const auto aligned = [](const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; };
  if (!aligned(q) || !aligned(k_cache) || !aligned(v_cache) || !aligned(out)) return SPEC_E_SHAPE;
  if (p.ws > 0 && (workspace == nullptr || workspace_bytes < p.ws || !aligned(workspace)))
    return SPEC_E_WORKSPACE;

  MfmaArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_cache);
  a.v = static_cast<const uint16_t*>(v_cache);
  a.prefix_len = prefix_len;
  a.n_nodes = n_nodes;
  a.parents = parents;
  a.B = B; a.n_max = n_max; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.L_cap = L_cap;
  a.kv = kv;
  a.RB = p.rb; a.S_max = p.S_max; a.chunk = p.chunk; a.units = p.units; a.sort = p.sort;
  a.c = c;
  a.inv_freq = inv_freq;
  a.rope = rope;
  a.out = out;
  a.dev_error = dev_error;
  a.part_o = nullptr;
  a.part_ml = nullptr;
  if (p.S_max > 1) {
    const size_t rows = (size_t)B * Hkv * p.rb * p.rpw * p.S_max;
    char* ws = static_cast<char*>(workspace);
    a.part_o = reinterpret_cast<float*>(ws);
    a.part_ml = reinterpret_cast<float2*>(ws + rows * HD * sizeof(float));
  }
  const unsigned grid = (unsigned)(((p.units + 7) / 8) * 8 * p.rb);
  if (kv.table)
    launch_variant<true>(p, grid, strm, a);
  else
    launch_variant<false>(p, grid, strm, a);
  SPEC_HIP_TRY(hipGetLastError());
  if (p.S_max > 1) {
    hipLaunchKernelGGL(attn_merge_kernel,
                       dim3((p.rb * p.rpw + kMergeRows - 1) / kMergeRows, Hkv, B),
                       dim3(32 * kMergeRows), 0, strm, a, p.rb * p.rpw);
    SPEC_HIP_TRY(hipGetLastError());
  }
  return SPEC_OK;
}
}  // namespace

extern "C" spec_status_t spec_verify_tree_attn(
    const void* q, const void* k_cache, const void* v_cache, const int32_t* prefix_len,
    const int32_t* n_nodes, const int32_t* parents, int32_t B, int32_t n_max, int32_t Hq,
    int32_t Hkv, int32_t head_dim, int32_t L_cap, float scale, int32_t dtype, float* out,
    void* workspace, size_t workspace_bytes, int32_t* dev_error, void* stream) {
  if (L_cap <= 0) return SPEC_E_SHAPE;
  return launch_attn(q, k_cache, v_cache, prefix_len, n_nodes, parents, B, n_max, Hq, Hkv,
                     head_dim, contiguous_rows(Hkv, L_cap), scale, dtype, nullptr, 0, out,
                     workspace, workspace_bytes, dev_error, stream);
}

extern "C" spec_status_t spec_verify_tree_attn_rope(
    const void* q, const void* k_cache, const void* v_cache, const int32_t* prefix_len,
    const int32_t* n_nodes, const int32_t* parents, int32_t B, int32_t n_max, int32_t Hq,
    int32_t Hkv, int32_t head_dim, int32_t L_cap, float scale, int32_t dtype,
    const float* inv_freq, int32_t rope_style, float* out, void* workspace,
    size_t workspace_bytes, int32_t* dev_error, void* stream) {
  if (!inv_freq) return SPEC_E_NULL;
  if (rope_style != kRopeHalf && rope_style != kRopeInterleaved) return SPEC_E_VALUE;
  if (L_cap <= 0) return SPEC_E_SHAPE;
  return launch_attn(q, k_cache, v_cache, prefix_len, n_nodes, parents, B, n_max, Hq, Hkv,
                     head_dim, contiguous_rows(Hkv, L_cap), scale, dtype, inv_freq, rope_style,
                     out, workspace, workspace_bytes, dev_error, stream);
}

extern "C" spec_status_t spec_verify_tree_attn_paged(
    const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
    int32_t max_blocks, int32_t block_size, int32_t num_blocks, const int32_t* prefix_len,
    const int32_t* n_nodes, const int32_t* parents, int32_t B, int32_t n_max, int32_t Hq,
    int32_t Hkv, int32_t head_dim, float scale, int32_t dtype, const float* inv_freq,
    int32_t rope_style, float* out, void* workspace, size_t workspace_bytes, int32_t* dev_error,
    void* stream) {
  if (!block_table) return SPEC_E_NULL;
  if (inv_freq && rope_style != kRopeHalf && rope_style != kRopeInterleaved) return SPEC_E_VALUE;
  KvRows kv;
  const spec_status_t st = make_paged_rows(block_table, max_blocks, block_size, num_blocks,
                                           Hkv > 0 ? Hkv : 1, &kv);
  if (st != SPEC_OK) return st;
  return launch_attn(q, k_pool, v_pool, prefix_len, n_nodes, parents, B, n_max, Hq, Hkv,
                     head_dim, kv, scale, dtype, inv_freq, inv_freq ? rope_style : 0, out,
                     workspace, workspace_bytes, dev_error, stream);
}
