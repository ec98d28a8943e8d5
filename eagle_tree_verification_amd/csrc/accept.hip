// Leviathan acceptance walked down a draft tree (gfx950).
//
// Rule (page "推测解码与 EAGLE-3", section "不变量：Leviathan 拒绝采样" and
// build steps 1-3): a draft token x drawn from the draft distribution p is
// accepted with probability min(1, q(x)/p(x)); on rejection one token is
// drawn from the residual norm(max(0, q - p)) and the step stops; when every
// draft is accepted a bonus token is drawn from the verifier's distribution
// after the last one.  p(x) <= 0 accepts; a zero-mass residual falls back to
// the distribution being corrected.  A node counts only if its whole root
// path is accepted (page "EAGLE-1/2/3 拆解", section "一个可核对的经验性质"),
// so the walk starts at the root and descends.  Several children of one node
// (all drawn from p_v) are tested in ascending id against the running
// residual: after k rejections the distribution being tested is
// max(0, q - C_k p) / Z_k with C_0 = 0, Z_0 = 1, C_{k+1} = C_k + Z_k and
// Z_{k+1} = sum(max(0, q - C_{k+1} p)), so no row is materialised.
// Temperature 0 is greedy decoding (accept iff the token is the verifier's
// argmax; emit the argmax).
//
// Sampling filters (page "EAGLE-1/2/3 拆解", section "一次 eagenerate 调用的完整
// 流转": top_k and top_p are sampling arguments beside the temperature).
// Both restrict q to the tokens whose logit is at least a threshold t that
// is itself one of the row's logits: top-k's t is the k-th largest logit,
// top-p's is the largest logit whose tokens at or above it hold at least
// the mass p of the tempered q; with both, the larger.  The threshold is
// found by a radix select over an order-preserving 32-bit key of the float
// logit, 8 bits per round, on per-bucket counts and 2^-47 fixed-point masses
// of q (integers, so the sums are exact and order-free), each round's
// histograms combined over the KP workgroups; then one more pass sums
// exp(z - M) over the kept tokens, and the walk proceeds with every q masked
// to logit >= t.
//
// Shape on the GPU.  The walk is serial along the tree but every step is a
// reduction over the 32k-128k vocabulary, so a sequence gets KP workgroups,
// each owning a slice of NT * W * NG entries (thread t reads W consecutive
// entries of each of its NG groups, groups NT * W entries apart, so loads are
// coalesced 16-byte vectors).  The workgroups run the same control flow and
// meet at a per-sequence barrier (one atomic counter) after every pass,
// exchanging two float64 partials; partials are combined in slice order, so
// every workgroup takes the same decisions.  A visited node costs one pass
// (max and sum of exp, online per batch); a rejected child one pass of
// max(0, exp(z - M) - C S p); the terminal token needs no extra pass: the
// slice masses of the current residual are already known, and only the
// workgroup whose slice holds the threshold scans it in order.  All vocab
// arithmetic is float64 (z = logit / T); exp runs on the vector ALU (a
// 256-entry table method in the per-entry passes, a Cody-Waite reduction with
// a Taylor polynomial elsewhere; arguments are never positive here).  The
// launch plan keeps all KP workgroups of every sequence of a launch resident
// at once; a batch too large for that is walked in consecutive groups.  Every
// inter-workgroup wait is bounded and reports SPEC_DEVERR_SYNC when it gives
// up, so a walk that cannot complete ends instead of hanging.
#include <math.h>
#include <stdlib.h>
#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <chrono>

#include "common.hpp"

namespace specv {
namespace {

constexpr int NT = 256;   // threads per workgroup
constexpr double kTieBand = 1e-6;
constexpr double kSampleBand = 1e-9;
// top-p boundaries: the masses are fixed point of 2^-47 per entry, so their
// truncation error stays below V * 2^-47, under 1e-9 for a 128k vocabulary
constexpr double kFilterBand = 1e-8;
constexpr double kDegenerate = 1e-12;

// exp(y) for y <= 0 in float64: y = n ln2 + r with |r| <= ln2 / 2 (ln2 split
// in two parts so n * ln2_hi is exact), exp(r) by its Taylor series to degree
// 13 (truncation below 5e-18 relative), then scaled by 2^n.  Underflows to 0.
__device__ __forceinline__ double exp_nonpos(double y) {
  constexpr double kLog2e = 1.4426950408889634;
  constexpr double kLn2Hi = 6.93147180369123816490e-01;
  constexpr double kLn2Lo = 1.90821492927058770002e-10;
  const double n = rint(y * kLog2e);
  double r = fma(-n, kLn2Hi, y);
  r = fma(-n, kLn2Lo, r);
  double p = 1.0 / 6227020800.0;             // 1/13!
  p = fma(p, r, 1.0 / 479001600.0);          // 1/12!
  p = fma(p, r, 1.0 / 39916800.0);
  p = fma(p, r, 1.0 / 3628800.0);
  p = fma(p, r, 1.0 / 362880.0);
  p = fma(p, r, 1.0 / 40320.0);
  p = fma(p, r, 1.0 / 5040.0);
  p = fma(p, r, 1.0 / 720.0);
  p = fma(p, r, 1.0 / 120.0);
  p = fma(p, r, 1.0 / 24.0);
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  const double v = ldexp(p, (int)n);
  return y < -745.5 ? 0.0 : v;
}

// exp(y) for y <= 0 (or -inf) in float64, for the per-entry passes: with
// n = round(256 y / ln2) = 256 k + j, exp(y) = 2^k * tab[j] * exp(r), where
// tab[j] = 2^(j/256), r = y - n ln2 / 256 (ln2 / 256 in two parts, so
// |r| <= ln2 / 512 up to rounding) and exp(r) is its Taylor series to degree
// 4 (truncation below 4e-17 relative).  n comes from the low word of
// y * 256 / ln2 + 1.5 * 2^52, whose addition rounds to an integer.  Within two
// ulp; -inf and anything below -746 give 0 (ldexp underflows); no branch.
constexpr int kTabBits = 8;
constexpr int kTab = 1 << kTabBits;

__device__ __forceinline__ double exp_tab(double y, const double* tab) {
  constexpr double kInvLn2xT = 369.3299304675746;  // 256 / ln2
  constexpr double kShift = 6755399441055744.0;     // 1.5 * 2^52
  constexpr double kLn2HiT = 6.93147180369123816490e-01 / kTab;
  constexpr double kLn2LoT = 1.90821492927058770002e-10 / kTab;
  const double yc = fmax(y, -746.0);
  const double t = fma(yc, kInvLn2xT, kShift);
  const double n = t - kShift;
  const int ni = __double2loint(t);
  double r = fma(-n, kLn2HiT, yc);
  r = fma(-n, kLn2LoT, r);
  double p = 1.0 / 24.0;
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  return ldexp(tab[ni & (kTab - 1)] * p, ni >> kTabBits);
}

// exp(y) for -700 <= y <= 0 (up to rounding; the caller checks the bound):
// exp_tab without the clamp, and 2^k applied by an integer add to the
// exponent field instead of ldexp.  tab2[j] is tab[j] with j << 12 taken off
// its high word, so adding ni << 12 = (k << 20) + (j << 12) adds k to the
// exponent; the scaled entry stays normal (k >= -1011), so the product
// rounds exactly as exp_tab's does: the same bits.
__device__ __forceinline__ double exp_fast(double y, const double* tab2) {
  constexpr double kInvLn2xT = 369.3299304675746;  // 256 / ln2
  constexpr double kShift = 6755399441055744.0;     // 1.5 * 2^52
  constexpr double kLn2HiT = 6.93147180369123816490e-01 / kTab;
  constexpr double kLn2LoT = 1.90821492927058770002e-10 / kTab;
  const double t = fma(y, kInvLn2xT, kShift);
  const double n = t - kShift;
  const int ni = __double2loint(t);
  double r = fma(-n, kLn2HiT, y);
  r = fma(-n, kLn2LoT, r);
  double p = 1.0 / 24.0;
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  const double tv = tab2[ni & (kTab - 1)];
  const int hi = (int)((uint32_t)__double2hiint(tv) + ((uint32_t)ni << 12));
  return p * __hiloint2double(hi, __double2loint(tv));
}

// Lower bound on z - m (the running max) under which a batch uses exp_fast.
constexpr double kFastFloor = -700.0;

struct AcceptArgs {
  const int32_t* tokens;
  const int32_t* parents;
  const int32_t* n_nodes;
  const float* draft_p;
  const float* logits;
  int B, n_max, V, max_depth, greedy;
  double inv_T;
  const float* temps;       // per-sequence temperatures, or null (inv_T / greedy apply)
  const int32_t* t2d;       // target -> draft id (-1: none), when p is over a draft vocabulary
  const int32_t* t2d_bad;   // nonzero when the draft map is not one-to-one into [0, V)
  int pstride;              // entries per draft_p row (V, or the draft vocabulary size)
  const float* u_accept;
  const float* u_sample;
  int32_t* accept_len;
  int32_t* path;
  int32_t* out_tokens;
  int32_t* n_out;
  float* final_dist;
  spec_tie_t* tie_log;
  int tie_cap;
  int32_t* tie_count;
  int b0;       // first sequence of this launch
  int KP;       // workgroups per sequence
  int chunk;    // vocabulary entries per workgroup (NT * W * NG)
  uint64_t* slots;  // [group size][2][KP][16] tagged exchange words
  uint64_t epoch;   // launch id (32 bits), part of every exchange tag
  const int32_t* top_k;   // per-sequence top-k (<= 0 or >= V: off), or null
  const float* top_p;     // per-sequence top-p (<= 0 or >= 1: off), or null
  uint64_t* hist;         // [B][2][KP][512] tagged histogram words
  int32_t* dev_error;
  int spin_limit;
  uint32_t* seq_epoch;    // [B] per-sequence launch counters (workspace), see walk_epoch
};

// ---- wave-uniform values ------------------------------------------------------
// The walk's combined statistics are identical in every lane and wave (they
// come from fixed-order butterfly reductions whose every lane holds the same
// bits).  Taking them from the first lane tells the compiler so, which keeps
// them in scalar registers.
__device__ __forceinline__ double uni(double x) {
  const long long bits = __double_as_longlong(x);
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(bits & 0xffffffffll));
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(bits >> 32));
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// ---- block reductions (fixed order, so results are deterministic) ---------
__device__ float block_max(float v, double* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int wv = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wv] = (double)v;
  __syncthreads();
  float t = -INFINITY;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) t = fmaxf(t, (float)red[k]);
  return t;
}

// Reductions over one wave on DPP lane moves (no LDS round trip per step):
// swaps within quads (lane ^ 1, lane ^ 2), mirrors within eight and sixteen
// lanes, then the row broadcasts that add row 0 into row 1, row 2 into row 3,
// and rows 0-1 into rows 2-3, leaving the total in lane 63, which is read
// back as a wave-uniform value.  A fixed sequence of operations: every wave
// reducing the same 64 inputs gets the same bits, so all workgroups of a
// sequence reach identical decisions.  Lanes a row broadcast leaves out take
// the operation's identity.
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_move(double x, double ident) {
  const unsigned long long xb = (unsigned long long)__double_as_longlong(x);
  const unsigned long long ib = (unsigned long long)__double_as_longlong(ident);
  const unsigned lo = (unsigned)__builtin_amdgcn_update_dpp((int)(ib & 0xffffffffu),
                                                            (int)(xb & 0xffffffffu), CTRL, ROWS,
                                                            0xf, false);
  const unsigned hi = (unsigned)__builtin_amdgcn_update_dpp((int)(ib >> 32), (int)(xb >> 32),
                                                            CTRL, ROWS, 0xf, false);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

__device__ __forceinline__ double lane63(double x) {
  const unsigned long long xb = (unsigned long long)__double_as_longlong(x);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(xb & 0xffffffffu), 63);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(xb >> 32), 63);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

constexpr int kDppXor1 = 0xB1;        // quad_perm(1, 0, 3, 2)
constexpr int kDppXor2 = 0x4E;        // quad_perm(2, 3, 0, 1)
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppBcast15 = 0x142;
constexpr int kDppBcast31 = 0x143;

__device__ __forceinline__ double wave_max_d(double v) {
  v = fmax(v, dpp_move<kDppXor1, 0xf>(v, -INFINITY));
  v = fmax(v, dpp_move<kDppXor2, 0xf>(v, -INFINITY));
  v = fmax(v, dpp_move<kDppHalfMirror, 0xf>(v, -INFINITY));
  v = fmax(v, dpp_move<kDppMirror, 0xf>(v, -INFINITY));
  v = fmax(v, dpp_move<kDppBcast15, 0xa>(v, -INFINITY));
  v = fmax(v, dpp_move<kDppBcast31, 0xc>(v, -INFINITY));
  return lane63(v);
}

__device__ __forceinline__ double wave_sum_d(double v) {
  v += dpp_move<kDppXor1, 0xf>(v, 0.0);
  v += dpp_move<kDppXor2, 0xf>(v, 0.0);
  v += dpp_move<kDppHalfMirror, 0xf>(v, 0.0);
  v += dpp_move<kDppMirror, 0xf>(v, 0.0);
  v += dpp_move<kDppBcast15, 0xa>(v, 0.0);
  v += dpp_move<kDppBcast31, 0xc>(v, 0.0);
  return lane63(v);
}

__device__ double block_sum(double v, double* red) {
  v = wave_sum_d(v);
  const int wv = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wv] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) t += red[k];
  return t;
}

// Combines per-thread (max, sum of exp relative to max) over the workgroup:
// one wave max, one rescale per lane, one wave sum, then the NT / 64 wave
// results.
__device__ void block_lse(double& m, double& s, double* red, const double* tab) {
  const double wm = wave_max_d(m);
  const double ts = wave_sum_d(m == -INFINITY ? 0.0 : s * exp_tab(m - wm, tab));
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) {
    red[2 * wv] = wm;
    red[2 * wv + 1] = ts;
  }
  __syncthreads();
  // the waves' partials combined across lanes (lane k takes wave k's), so the
  // rescaling exponentials run side by side rather than one after another
  const bool has = lane < NT / 64;
  const double km = has ? red[2 * lane] : -INFINITY;
  const double mm = wave_max_d(km);
  const double ss = wave_sum_d(has && km != -INFINITY ? red[2 * lane + 1] * exp_tab(km - mm, tab) : 0.0);
  m = mm;
  s = ss;
}

// argmax with lowest index on ties; NaN never wins (flagged separately)
__device__ __forceinline__ void amax_combine(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

__device__ void block_argmax(float& v, int& i, double* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(v, o);
    const int i2 = __shfl_xor(i, o);
    amax_combine(v, i, v2, i2);
  }
  const int wv = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    red[2 * wv] = (double)v;
    red[2 * wv + 1] = (double)i;
  }
  __syncthreads();
  float bv = -INFINITY;
  int bi = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) amax_combine(bv, bi, (float)red[2 * k], (int)red[2 * k + 1]);
  v = bv;
  i = bi;
}

__device__ __forceinline__ int block_or(int f, int*) { return __syncthreads_or(f); }

// ---- inter-workgroup exchange ---------------------------------------------
// Tag of exchange number gen: 32 bits of launch id, 16 of exchange number (a
// walk makes well under 2^16 exchanges), 48 bits in all.
constexpr int kSlotWords = 16;  // exchange words per workgroup and buffer

__device__ __forceinline__ uint64_t exchange_tag(uint32_t ep, int gen) {
  return ((uint64_t)ep << 16) | (uint64_t)(gen & 0xffff);
}

// Publishes this workgroup's two partials and gathers all KP workgroups'
// partials into xs.  Each partial travels as four 64-bit words of 16 payload
// bits under a 48-bit tag (launch id, exchange number), written and read with
// device-coherent 64-bit atomic accesses.  A word is valid once its tag is
// current, whatever order the words arrive in, so the readers poll the data
// itself: one memory round trip per exchange, with no counter, no fence and
// nothing to clear between calls.  Slots alternate between two buffers (16
// words per workgroup each, room for exchange4's four partials); a
// workgroup reuses a buffer only after every workgroup has published the next
// exchange, which each does only after reading this one.
__device__ bool exchange(const AcceptArgs& a, uint32_t ep, int bl, int part, int& gen, double v0,
                         double v1, double (*xs)[2], int* s_or) {
  const int t = threadIdx.x;
  __syncthreads();  // xs of the previous exchange is no longer read
  if (a.KP == 1) {
    if (t == 0) {
      xs[0][0] = v0;
      xs[0][1] = v1;
    }
    __syncthreads();
    return true;
  }
  const uint64_t tag = exchange_tag(ep, gen);
  uint64_t* slot = a.slots + ((size_t)bl * 2 + (gen & 1)) * (size_t)a.KP * kSlotWords;
  ++gen;
  if (t < 8) {
    const uint64_t bits = (uint64_t)__double_as_longlong(t < 4 ? v0 : v1);
    const uint64_t w = (tag << 16) | ((bits >> (16 * (t & 3))) & 0xffffull);
    __hip_atomic_store(slot + part * kSlotWords + t, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const int nw = a.KP * 8;
  int bad = 0;
  // every word this thread reads is requested at once, then re-polled until
  // its tag is current: one memory round trip when the words are there
  constexpr int kRounds = (SPEC_MAX_NODES * 8 + NT - 1) / NT;
  uint64_t w[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int i = t + r * NT;  // word i: part i / 8, value (i / 4) % 2, bits 16 (i % 4)
    w[r] = i < nw ? __hip_atomic_load(slot + (i >> 3) * kSlotWords + (i & 7), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT)
                  : 0;
  }
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int i = t + r * NT;
    if (i < nw) {
      int spins = 0;
      while (a.spin_limit < 0 || (w[r] >> 16) != tag) {
        if (a.spin_limit < 0 || ++spins > a.spin_limit) {  // a negative bound: test hook
          bad = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        w[r] = __hip_atomic_load(slot + (i >> 3) * kSlotWords + (i & 7), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    // the four words of one value sit in four consecutive lanes
    const uint64_t p0 = w[r] & 0xffffull;
    const uint64_t p1 = __shfl_down(p0, 1);
    const uint64_t p2 = __shfl_down(p0, 2);
    const uint64_t p3 = __shfl_down(p0, 3);
    if (i < nw && (i & 3) == 0)
      xs[i >> 3][(i >> 2) & 1] = __longlong_as_double((long long)(p0 | (p1 << 16) | (p2 << 32) | (p3 << 48)));
  }
  const bool ok = !block_or(bad, s_or);
  // Every workgroup of the sequence has published its first word, so has
  // read the sequence's launch counter: the next launch may advance it.
  if (ok && gen == 1 && part == 0 && t == 0)
    __hip_atomic_store(a.seq_epoch + a.b0 + bl, ep - (uint32_t)a.epoch + 1u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  return ok;
}

// exchange() for four partials (a statistics pass that also covers a node's
// first child): the same tagged words, 16 per workgroup.
__device__ bool exchange4(const AcceptArgs& a, uint32_t ep, int bl, int part, int& gen,
                          double v0, double v1, double v2, double v3, double (*xs)[4],
                          int* s_or) {
  constexpr int NV = 4;
  constexpr int kWords = 4 * NV;  // words per workgroup
  const int t = threadIdx.x;
  __syncthreads();  // xs of the previous exchange is no longer read
  if (a.KP == 1) {
    if (t == 0) {
#pragma unroll
      for (int k = 0; k < NV; ++k) xs[0][k] = k == 0 ? v0 : k == 1 ? v1 : k == 2 ? v2 : v3;
    }
    __syncthreads();
    return true;
  }
  const uint64_t tag = exchange_tag(ep, gen);
  uint64_t* slot = a.slots + ((size_t)bl * 2 + (gen & 1)) * (size_t)a.KP * kSlotWords;
  ++gen;
  if (t < kWords) {
    const int k = t >> 2;
    const double x = k == 0 ? v0 : k == 1 ? v1 : k == 2 ? v2 : v3;
    const uint64_t bits = (uint64_t)__double_as_longlong(x);
    const uint64_t w = (tag << 16) | ((bits >> (16 * (t & 3))) & 0xffffull);
    __hip_atomic_store(slot + part * kSlotWords + t, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const int nw = a.KP * kWords;
  int bad = 0;
  // every word this thread reads is requested at once, then re-polled until
  // its tag is current: one memory round trip when the words are there
  constexpr int kRounds = (SPEC_MAX_NODES * kWords + NT - 1) / NT;
  uint64_t w[kRounds];
  // word i: part i / kWords, value (i / 4) % NV, bits 16 (i % 4)
  auto addr = [&](int i) { return slot + (i / kWords) * kSlotWords + i % kWords; };
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int i = t + r * NT;
    w[r] = i < nw ? __hip_atomic_load(addr(i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
  }
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int i = t + r * NT;
    if (i < nw) {
      int spins = 0;
      while (a.spin_limit < 0 || (w[r] >> 16) != tag) {
        if (a.spin_limit < 0 || ++spins > a.spin_limit) {  // a negative bound: test hook
          bad = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        w[r] = __hip_atomic_load(addr(i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    // the four words of one value sit in four consecutive lanes
    const uint64_t p0 = w[r] & 0xffffull;
    const uint64_t p1 = __shfl_down(p0, 1);
    const uint64_t p2 = __shfl_down(p0, 2);
    const uint64_t p3 = __shfl_down(p0, 3);
    if (i < nw && (i & 3) == 0)
      xs[i / kWords][(i >> 2) % NV] =
          __longlong_as_double((long long)(p0 | (p1 << 16) | (p2 << 32) | (p3 << 48)));
  }
  const bool ok = !block_or(bad, s_or);
  // Every workgroup of the sequence has published its first word, so has
  // read the sequence's launch counter: the next launch may advance it.
  if (ok && gen == 1 && part == 0 && t == 0)
    __hip_atomic_store(a.seq_epoch + a.b0 + bl, ep - (uint32_t)a.epoch + 1u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  return ok;
}

__device__ void log_tie(const AcceptArgs& a, int b, int node, int kind, float u, double margin) {
  if (!a.tie_count) return;
  const int k = atomicAdd(a.tie_count, 1);
  if (a.tie_log && k < a.tie_cap) {
    spec_tie_t r;
    r.b = b;
    r.node = node;
    r.kind = kind;
    r.u = u;
    r.margin = margin;
    a.tie_log[k] = r;
  }
}

__device__ void write_failure(const AcceptArgs& a, int b, int bits) {
  if (threadIdx.x == 0) {
    a.accept_len[b] = -1;
    a.n_out[b] = 0;
    report(a.dev_error, bits);
  }
  for (int k = threadIdx.x; k <= a.max_depth; k += NT) {
    a.path[(size_t)b * (a.max_depth + 1) + k] = -1;
    a.out_tokens[(size_t)b * (a.max_depth + 1) + k] = -1;
  }
}

// A wait that hit its bound: every workgroup that sees it reports it; the
// sequence's first workgroup also marks the sequence failed.  Workgroups of
// the sequence that got past the same exchange may still write outputs, so
// after SPEC_DEVERR_SYNC the batch's outputs are unspecified.
__device__ void fail_sync(const AcceptArgs& a, int b, bool writer0) {
  if (writer0) {
    write_failure(a, b, SPEC_DEVERR_SYNC);
  } else if (threadIdx.x == 0) {
    report(a.dev_error, SPEC_DEVERR_SYNC);
  }
}

__device__ void write_outputs(const AcceptArgs& a, int b, int depth, const int* s_path, const int* s_out) {
  if (threadIdx.x == 0) {
    a.accept_len[b] = depth;
    a.n_out[b] = depth + 1;
  }
  for (int k = threadIdx.x; k <= a.max_depth; k += NT) {
    a.path[(size_t)b * (a.max_depth + 1) + k] = k <= depth ? s_path[k] : -1;
    a.out_tokens[(size_t)b * (a.max_depth + 1) + k] = k <= depth ? s_out[k] : -1;
  }
}

// Element k of a thread's slice share: group k / W (NT * W entries apart),
// entry k % W within the thread's W consecutive entries of that group.
template <int W>
__device__ __forceinline__ int elem_index(int lo, int k) {
  return lo + ((k / W) * NT + (int)threadIdx.x) * W + (k % W);
}

// Loads group g (W consecutive entries) of this thread's share of a row
// slice; entries past `hi` read as `fill`.  The load itself is unconditional,
// at an index clamped into the slice (a slice holds at least W entries, and
// with W = 4 its bounds are multiples of 4), and the fill is a select: a load
// under a branch makes the compiler wait for it at once, which would undo the
// prefetching of stream_slice.
template <int W>
__device__ __forceinline__ void load_group(const float* row, int lo, int hi, int g, float fill, float* x) {
  const int i = elem_index<W>(lo, g * W);
  const bool ok = i < hi;
  const int ic = ok ? i : hi - W;
  if (W == 4) {
    const float4 f = *reinterpret_cast<const float4*>(row + ic);
    x[0] = ok ? f.x : fill;
    x[1] = ok ? f.y : fill;
    x[2] = ok ? f.z : fill;
    x[3] = ok ? f.w : fill;
  } else {
    const float f = row[ic];
    x[0] = ok ? f : fill;
  }
}

// Group g of a draft row held over a draft vocabulary: target entry i reads
// p_draft[t2d[i]], or 0 when no draft id maps to i.  Loads and gathers are
// unconditional (clamped index, id -1 read as id 0) for the same reason.
template <int W>
__device__ __forceinline__ void load_group_mapped(const float* row, const int32_t* t2d, int lo,
                                                  int hi, int g, float fill, float* x) {
  const int i = elem_index<W>(lo, g * W);
  const bool ok = i < hi;
  const int ic = ok ? i : hi - W;
  if (W == 4) {
    const int4 t = *reinterpret_cast<const int4*>(t2d + ic);
    const float p0 = row[max(t.x, 0)], p1 = row[max(t.y, 0)];
    const float p2 = row[max(t.z, 0)], p3 = row[max(t.w, 0)];
    x[0] = ok ? (t.x >= 0 ? p0 : 0.f) : fill;
    x[1] = ok ? (t.y >= 0 ? p1 : 0.f) : fill;
    x[2] = ok ? (t.z >= 0 ? p2 : 0.f) : fill;
    x[3] = ok ? (t.w >= 0 ? p3 : 0.f) : fill;
  } else {
    const int t = t2d[ic];
    const float p = row[max(t, 0)];
    x[0] = ok ? (t >= 0 ? p : 0.f) : fill;
  }
}

template <int W, bool MAPPED>
__device__ __forceinline__ void load_group_p(const float* row, const int32_t* t2d, int lo, int hi,
                                             int g, float fill, float* x) {
  if constexpr (MAPPED) load_group_mapped<W>(row, t2d, lo, hi, g, fill, x);
  else load_group<W>(row, lo, hi, g, fill, x);
}

// Group g as load_group_p loads it, without the fill: entries past `hi` hold
// what the clamped load returned until fill_batch replaces them.
template <int W, bool MAPPED>
__device__ __forceinline__ void load_group_raw(const float* row, const int32_t* t2d, int lo,
                                               int hi, int g, float* x) {
  const int i = elem_index<W>(lo, g * W);
  const int ic = i < hi ? i : hi - W;
  if (W == 4) {
    if constexpr (MAPPED) {
      const int4 t = *reinterpret_cast<const int4*>(t2d + ic);
      const float p0 = row[max(t.x, 0)], p1 = row[max(t.y, 0)];
      const float p2 = row[max(t.z, 0)], p3 = row[max(t.w, 0)];
      x[0] = t.x >= 0 ? p0 : 0.f;
      x[1] = t.y >= 0 ? p1 : 0.f;
      x[2] = t.z >= 0 ? p2 : 0.f;
      x[3] = t.w >= 0 ? p3 : 0.f;
    } else {
      const float4 f = *reinterpret_cast<const float4*>(row + ic);
      x[0] = f.x;
      x[1] = f.y;
      x[2] = f.z;
      x[3] = f.w;
    }
  } else {
    if constexpr (MAPPED) {
      const int t = t2d[ic];
      const float p = row[max(t, 0)];
      x[0] = t >= 0 ? p : 0.f;
    } else {
      x[0] = row[ic];
    }
  }
}

// Sets the entries of groups g0 .. g0+BG-1 that lie past `hi` to `fill`.  The
// last entry any thread holds in the batch is lo + (g0 + BG) * NT * W - 1, so
// a batch wholly inside the slice (the same answer for every thread: one
// scalar branch) keeps its loaded values without a select per entry.
template <int W, int BG>
__device__ __forceinline__ void fill_batch(int lo, int hi, int g0, float fill, float (*xv)[W]) {
  if (lo + (g0 + BG) * NT * W <= hi) return;
#pragma unroll
  for (int gb = 0; gb < BG; ++gb) {
    const bool ok = elem_index<W>(lo, (g0 + gb) * W) < hi;
#pragma unroll
    for (int j = 0; j < W; ++j) xv[gb][j] = ok ? xv[gb][j] : fill;
  }
}

// Streams this thread's NG groups of a row slice (two rows when R2) through
// `body(g0, x, y)`, BG groups at a time, with the next batch's loads issued
// before the current batch is processed.  Groups past the slice read as fill
// and touch no memory.
template <int NG, int W, int BG, bool R2, bool MAPPED = false, typename F>
__device__ __forceinline__ void stream_slice(const float* r1, float f1, const float* r2, float f2,
                                             int lo, int hi, F body,
                                             const int32_t* t2d = nullptr) {
  float xa[BG][W], xb[BG][W], ya[BG][W], yb[BG][W];
  auto load = [&](int g0, float (*x)[W], float (*y)[W]) {
#pragma unroll
    for (int gb = 0; gb < BG; ++gb) load_group_raw<W, false>(r1, nullptr, lo, hi, g0 + gb, x[gb]);
    if (R2) {
#pragma unroll
      for (int gb = 0; gb < BG; ++gb) load_group_raw<W, MAPPED>(r2, t2d, lo, hi, g0 + gb, y[gb]);
    }
  };
  auto run = [&](int g0, float (*x)[W], float (*y)[W]) {
    fill_batch<W, BG>(lo, hi, g0, f1, x);
    if (R2) fill_batch<W, BG>(lo, hi, g0, f2, y);
    body(g0, x, y);
  };
  load(0, xa, ya);
#pragma unroll 1
  for (int g0 = 0; g0 < NG; g0 += 2 * BG) {
    load(g0 + BG, xb, yb);
    run(g0, xa, ya);
    if (g0 + BG >= NG) break;
    load(g0 + 2 * BG, xa, ya);
    run(g0 + BG, xb, yb);
  }
}

// One batch of a statistics pass over a row: the running max m of z = x / T
// and the sum es of exp(z - m) over the slice's entries (those past the slice
// hold -inf); nf flags a non-finite entry of the slice.
template <int W, int BG>
__device__ __forceinline__ void batch_stats(int lo, int hi, int g0, const float (*xv)[W],
                                            double invT, double& m, double& es, int& nf,
                                            const double* tab, const double* tab2) {
  float bmax = -INFINITY, bmin = INFINITY;
#pragma unroll
  for (int gb = 0; gb < BG; ++gb)
#pragma unroll
    for (int j = 0; j < W; ++j) {
      const bool valid = elem_index<W>(lo, (g0 + gb) * W + j) < hi;
      nf |= valid && !isfinite(xv[gb][j]);
      bmax = fmaxf(bmax, xv[gb][j]);
      bmin = fminf(bmin, xv[gb][j]);
    }
  if (bmax == -INFINITY) return;  // nothing valid in this batch
  const double zb = (double)bmax * invT;
  if (zb > m) {
    es *= exp_tab(m - zb, tab);  // m = -inf: es is still 0
    m = zb;
  }
  if (__all(fma((double)bmin, invT, -m) >= kFastFloor)) {
#pragma unroll
    for (int gb = 0; gb < BG; ++gb) {
      double sg = exp_fast(fma((double)xv[gb][0], invT, -m), tab2);
#pragma unroll
      for (int j = 1; j < W; ++j) sg += exp_fast(fma((double)xv[gb][j], invT, -m), tab2);
      es += sg;
    }
  } else {
#pragma unroll
    for (int gb = 0; gb < BG; ++gb) {
      double sg = exp_tab(fma((double)xv[gb][0], invT, -m), tab);
#pragma unroll
      for (int j = 1; j < W; ++j) sg += exp_tab(fma((double)xv[gb][j], invT, -m), tab);
      es += sg;
    }
  }
}

// ---- sampling filters -------------------------------------------------------
static_assert(NT == 256, "one radix bucket per thread");
// 2^47: fixed-point unit of q.  A slice's bucket then stays below 2^48 (q <= 1
// up to rounding), the width of its mass field in an exchange word.
constexpr double kMassOne = 140737488355328.0;

// Order-preserving 32-bit key of a finite float: a larger float has a larger
// key, and -0 shares the key of +0 (they compare equal).  Finite floats map
// into [0x00800000, 0xFF7FFFFF].
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = x == 0.f ? 0u : __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// A float f with (x >= f) == (order_key(x) >= k) for every finite x, for a
// key k at or below some finite float's key.
__device__ __forceinline__ float key_floor_float(uint32_t k) {
  if (k <= 0x00800000u) return -INFINITY;
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

struct FilterShared {
  uint64_t wc[NT / 64], wm[NT / 64];  // wave totals of the bucket scan
  uint64_t sel_C, sel_F, sel_cnt, sel_mass;
};

// Publishes this workgroup's 256-bucket histogram (h_cnt, h_mass: bucket j at
// index j * kCopies) and returns
// the sums over the KP workgroups of bucket jb.  Like exchange(), with no
// fence: every 64-bit word carries a 32-bit tag (a set top bit, 19 bits of
// launch id, 12 of exchange number) above 32 payload bits, is written and read
// with device-coherent atomic accesses, and is valid once its tag is current.
// A tag this short could recur after 2^19 launches, so every call clears the
// buffers first (hist_clear_kernel); the set bit keeps a tag from ever
// matching a cleared word, and the launch id keeps the launches of one call
// (consecutive groups of sequences) apart.  A
// bucket is two words: count (16 bits; a slice holds at most 16384 entries)
// with mass bits 47..32, then mass bits 31..0.  Each thread issues the loads
// of kHistBatch workgroups at once before checking tags.  Buffers alternate with
// the exchange number as in exchange(), whose numbering this shares.
constexpr int kHistBatch = 4;  // workgroups whose words one thread loads at once
// Lanes spread their histogram atomics over kCopies copies of every bucket
// (lane % kCopies; the copies of one bucket are adjacent words, so in
// different banks), which cuts same-address serialisation when many lanes
// share a digit; the copies are folded into copy 0 before the exchange.
constexpr int kCopies = 4;
// A wave gathers a filtered row's kept entries for a residual pass when none
// of its threads holds more than this many; otherwise it streams its slices.
constexpr int kMaskMax = 2;

__device__ bool exchange_hist(const AcceptArgs& a, uint32_t ep, int bl, int part, int& gen,
                              const uint32_t* h_cnt, const uint64_t* h_mass, int jb,
                              uint64_t& cnt, uint64_t& mass, int* s_or) {
  const int t = threadIdx.x;
  if (a.KP == 1) {
    cnt = h_cnt[jb * kCopies];
    mass = h_mass[jb * kCopies];
    return true;
  }
  const uint64_t tag = (((0x80000ull | (ep & 0x7FFFFull)) << 12) | (uint64_t)(gen & 0xfff))
                       << 32;
  uint64_t* data = a.hist + ((size_t)bl * 2 + (gen & 1)) * (size_t)a.KP * 512;
  ++gen;
  const uint64_t m = h_mass[t * kCopies];
  __hip_atomic_store(data + part * 512 + 2 * t,
                     tag | ((uint64_t)h_cnt[t * kCopies] << 16) | ((m >> 32) & 0xffffull),
                     __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(data + part * 512 + 2 * t + 1, tag | (m & 0xffffffffull), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  int bad = 0;
  uint64_t c = 0, ms = 0;
  for (int k0 = 0; k0 < a.KP; k0 += kHistBatch) {
    const int nk = a.KP - k0 < kHistBatch ? a.KP - k0 : kHistBatch;
    uint64_t w[2 * kHistBatch];
#pragma unroll
    for (int i = 0; i < 2 * kHistBatch; ++i)
      w[i] = i / 2 < nk ? __hip_atomic_load(data + (size_t)(k0 + i / 2) * 512 + 2 * jb + (i & 1),
                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                        : tag;
#pragma unroll
    for (int i = 0; i < 2 * kHistBatch; ++i) {
      int spins = 0;
      while ((w[i] >> 32) != (tag >> 32)) {
        if (a.spin_limit < 0 || ++spins > a.spin_limit) {  // a negative bound: test hook
          bad = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        w[i] = __hip_atomic_load(data + (size_t)(k0 + i / 2) * 512 + 2 * jb + (i & 1),
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
#pragma unroll
    for (int i = 0; i < 2 * kHistBatch; i += 2)
      if (i / 2 < nk) {
        c += (w[i] >> 16) & 0xffffull;
        ms += ((w[i] & 0xffffull) << 32) | (w[i + 1] & 0xffffffffull);
      }
  }
  cnt = c;
  mass = ms;
  return !block_or(bad, s_or);
}

// The filters' threshold t for the row at lrow (identical in every workgroup
// of the sequence): thr is a float with (x >= thr) exactly for the kept
// logits x.  fk: top-k (0 = off); P: top-p in units of 2^-47 (0 = off).
// Radix select, most significant digit first.  In each round the entries
// whose key matches the digits chosen so far are counted (and their masses
// exp(z - M) / S summed in fixed point) per next digit; with C(j) and F(j) the
// count and mass of all keys at or above bucket j, top-k's threshold lies in
// the highest bucket with C(j) >= k and top-p's in the highest with
// F(j) >= P, and the higher of the two is refined next.  It stops when the
// chosen bucket is one key (four rounds), holds a single entry, or (top-k
// deciding) holds exactly the entries still needed.  margin: distance of P
// to the masses above and at the threshold (in units of q), or a large
// value when top-p cannot flip a kept token.
template <int NG, int W, int BG>
__device__ bool filter_threshold(const AcceptArgs& a, uint32_t ep, int bl, int part, int& gen,
                                 const float* lrow, int lo, int hi, double invT, double M,
                                 double S, int fk, uint64_t P, const double* tab,
                                 uint32_t* h_cnt, uint64_t* h_mass, FilterShared& fs, int* s_or,
                                 float& thr, double& margin) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int jb = NT - 1 - tid;  // this thread's bucket in the descending scan
  const int cp = lane % kCopies;
  const bool use_k = fk > 0, use_p = P > 0;
  const double fscale = kMassOne / S;
  const uint64_t band = (uint64_t)(kFilterBand * kMassOne);
  uint32_t prefix = 0;
  uint64_t above_c = 0, above_m = 0;
  margin = 1.0;
  for (int r = 0;; ++r) {
    const int sh = 24 - 8 * r;
#pragma unroll
    for (int c = 0; c < kCopies; ++c) {
      h_cnt[tid * kCopies + c] = 0;
      h_mass[tid * kCopies + c] = 0;
    }
    __syncthreads();
    // one entry of the current range into the histogram
    auto add = [&](float x) {
      const int dg = (order_key(x) >> sh) & 255;
      atomicAdd(&h_cnt[dg * kCopies + cp], 1u);
      if (use_p) {
        const double e = exp_tab(fma((double)x, invT, -M), tab);
        atomicAdd((unsigned long long*)&h_mass[dg * kCopies + cp],
                  (unsigned long long)(e * fscale));
      }
    };
    stream_slice<NG, W, BG, false>(lrow, -INFINITY, lrow, 0.f, lo, hi,
        [&](int g0, float (*xv)[W], float (*)[W]) {
#pragma unroll
          for (int gb = 0; gb < BG; ++gb)
#pragma unroll
            for (int j = 0; j < W; ++j)
              if (elem_index<W>(lo, (g0 + gb) * W + j) < hi &&
                  (uint32_t)((uint64_t)order_key(xv[gb][j]) >> (sh + 8)) == prefix)
                add(xv[gb][j]);
        });
    __syncthreads();
    {
      uint32_t fc = 0;
      uint64_t fm = 0;
#pragma unroll
      for (int c = 0; c < kCopies; ++c) {
        fc += h_cnt[tid * kCopies + c];
        fm += h_mass[tid * kCopies + c];
      }
      h_cnt[tid * kCopies] = fc;
      h_mass[tid * kCopies] = fm;
    }
    __syncthreads();
    uint64_t cnt, mass;
    if (!exchange_hist(a, ep, bl, part, gen, h_cnt, h_mass, jb, cnt, mass, s_or)) return false;
    // suffix sums over buckets (prefix sums over threads)
    uint64_t c = cnt, m = mass;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint64_t c2 = __shfl_up(c, o), m2 = __shfl_up(m, o);
      if (lane >= o) {
        c += c2;
        m += m2;
      }
    }
    if (lane == 63) {
      fs.wc[wv] = c;
      fs.wm[wv] = m;
    }
    __syncthreads();
    for (int k = 0; k < wv; ++k) {
      c += fs.wc[k];
      m += fs.wm[k];
    }
    const uint64_t Cj = above_c + c, Fj = above_m + m;
    const int jk = use_k ? __syncthreads_count(Cj >= (uint64_t)fk) - 1 : -1;
    const int jp = use_p ? __syncthreads_count(Fj >= P) - 1 : -1;
    int js = jk > jp ? jk : jp;
    if (js < 0) js = 0;  // unreachable: the threshold lies in the current range
    if (jb == js) {
      fs.sel_C = Cj;
      fs.sel_F = Fj;
      fs.sel_cnt = cnt;
      fs.sel_mass = mass;
    }
    __syncthreads();
    const uint64_t selC = fs.sel_C, selF = fs.sel_F, selc = fs.sel_cnt, selm = fs.sel_mass;
    prefix = (prefix << 8) | (uint32_t)js;
    above_c = selC - selc;
    above_m = selF - selm;
    const bool done = r == 3 || selc == 1 ||
                      (use_k && selC == (uint64_t)fk && (!use_p || selF + band <= P));
    if (done) {
      thr = key_floor_float(prefix << sh);
      if (use_p) {
        // P - (mass above t) > 0 always; (mass at or above t) - P matters
        // only when top-p chose the bucket
        // nothing above the largest logit: an exactly zero mass, which no
        // rounding can bring to P
        double mg = above_m > 0 ? (double)(P - above_m) / kMassOne : 1.0;
        if (js == jp) mg = fmin(mg, (double)(selF - P) / kMassOne);
        margin = mg;
      }
      return true;
    }
  }
}

// Read in place of a per-sequence array the call does not pass.
__device__ const int32_t kZeroI32 = 0;
__device__ const float kZeroF32 = 0.f;

// FILT: the sampling filters are compiled in (the variant used when the call
// passes top_k or top_p); without it every q is unfiltered.
template <int NG, int W, bool MAPPED, bool FILT>
__global__ __launch_bounds__(NT) void accept_kernel(AcceptArgs a) {
  // groups loaded together: four in the one-row passes, two when the
  // residual pass streams logits and draft rows side by side
  constexpr int BG1 = NG < 4 ? NG : 4;
  constexpr int BG2 = NG < 2 ? NG : 2;
  __shared__ int s_par[SPEC_MAX_NODES];
  __shared__ int s_tok[SPEC_MAX_NODES];
  __shared__ unsigned long long s_kids[SPEC_MAX_NODES];  // bit c set: node c is a child
  __shared__ int s_path[SPEC_MAX_NODES + 1];
  __shared__ int s_out[SPEC_MAX_NODES + 1];
  __shared__ double red[2 * (NT / 64)];
  __shared__ double xs[SPEC_MAX_NODES][2];
  __shared__ double cur_sums[SPEC_MAX_NODES];
  constexpr bool LOOK = !FILT && NG <= 2;  // first-child statistics in the parent's pass
  __shared__ double la_sums[LOOK ? SPEC_MAX_NODES : 1];  // first child's slice masses
  __shared__ double xs4[LOOK ? SPEC_MAX_NODES : 1][4];   // partials of exchange4
  // also the filters' histograms: [256][kCopies] uint64 masses in rows 0-3,
  // [256][kCopies] uint32 counts in rows 4-5
  __shared__ double scan[FILT && NG < 6 ? 6 : (NG < 2 ? 2 : NG)][NT];
  __shared__ FilterShared fsh;
  __shared__ double gsum_w[NG][NT / 64];   // wave sums of each group (ordered scan)
  // scan[g][t]: thread t's sum over group g of the last pass, kept for the
  // ordered scan of the terminal sample; after a statistics pass each sum is
  // relative to exp(mref[k][t]), k = g / BG1, the thread's running maximum of
  // z when it summed the batch holding group g
  __shared__ double mref[NG / BG1][NT];
  __shared__ double wtot[NT / 64];
  __shared__ int s_or, s_hit, s_first;
  __shared__ float s_kp[SPEC_MAX_NODES], s_kl[SPEC_MAX_NODES], s_ku[SPEC_MAX_NODES], s_us;
  __shared__ double s_tab[kTab];
  __shared__ double s_tab2[FILT ? 1 : kTab];  // s_tab for exp_fast
  // filtered rows: bit g * W + j set where this thread's entry j of group g is
  // kept (all bits once a negative draft entry is seen)
  __shared__ unsigned long long s_keep[FILT ? NT : 1];

  const int bl = blockIdx.x / a.KP;   // sequence within this launch's group
  const int b = a.b0 + bl;
  const int part = blockIdx.x % a.KP;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int lo = part * a.chunk;
  const int hi = min(a.V, lo + a.chunk);
  const bool writer0 = (part == 0);

  // Every per-sequence value the prologue checks, and the tree rows, are
  // requested at once, before the table is built: the loads are
  // unconditional (a missing array reads a zero word instead), so none waits
  // for another.
  const int n = a.n_nodes[b];
  const float T_b = *(a.temps ? a.temps + b : &kZeroF32);
  const int k_b = *(FILT && a.top_k ? a.top_k + b : &kZeroI32);
  const float p_b = *(FILT && a.top_p ? a.top_p + b : &kZeroF32);
  const int bad_map = *(MAPPED ? a.t2d_bad : &kZeroI32);
  const size_t tree_row = (size_t)b * a.n_max + (tid < a.n_max ? tid : a.n_max - 1);
  const int par_b = a.parents[tree_row];
  const int tok_b = a.tokens[tree_row];
  // The launch id of this sequence's exchange tags: the host's id of the
  // launch plus the sequence's counter in the workspace, which the sequence's
  // first workgroup advances once every workgroup has read it (after the
  // first exchange).  A launch replayed from a captured graph repeats the
  // host's id, and the counter still makes its tags new, so no word a
  // previous launch left in the workspace reads as current.
  const uint32_t ep = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)((uint32_t)a.epoch +
            (a.KP > 1 ? __hip_atomic_load(a.seq_epoch + b, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT)
                      : 0u)));

  for (int j = tid; j < kTab; j += NT) {
    const double tj = 2.0 * exp_nonpos((double)(j - kTab) / kTab * 0.6931471805599453);
    s_tab[j] = tj;
    if (!FILT)
      s_tab2[j] = __hiloint2double((int)((uint32_t)__double2hiint(tj) - ((uint32_t)j << 12)),
                                   __double2loint(tj));
  }

  // ---- validation (identical in every workgroup of the sequence) ----------
  int err = 0;
  bool greedy = a.greedy;
  double invT = a.inv_T;
  if (a.temps) {  // this sequence's temperature
    const float T = T_b;
    if (!(T >= 0.f) || !isfinite(T)) err = SPEC_DEVERR_NONFINITE;
    greedy = T == 0.f;
    invT = greedy ? 0.0 : 1.0 / (double)T;
  }
  int fk = 0;          // top-k, 0 = off
  uint64_t fP = 0;     // top-p in units of 2^-47, 0 = off
  if (FILT && a.top_k) {
    const int k = k_b;
    if (k > 0 && k < a.V) fk = k;
  }
  if (FILT && a.top_p) {
    const float pp = p_b;
    if (pp != pp) err = SPEC_DEVERR_NONFINITE;
    else if (pp > 0.f && pp < 1.f) fP = max((uint64_t)((double)pp * kMassOne), (uint64_t)1);
  }
  if (MAPPED && bad_map) err = SPEC_DEVERR_TOKEN;
  if (err) {
    // a bad temperature, top-p or draft map: nothing else is checked
  } else if (n < 1 || n > a.n_max) {
    err = SPEC_DEVERR_TREE;
  } else {
    int bad_tree = 0, bad_tok = 0;
    if (tid < n) {
      const int p = par_b;
      const int tk = tok_b;
      s_par[tid] = p;
      s_tok[tid] = tk;
      if (tid == 0) {
        bad_tree = (p != -1);
      } else {
        bad_tree = (p < 0 || p >= tid);
        bad_tok = (tk < 0 || tk >= a.V);
      }
    }
    __syncthreads();
    if (tid < n && !bad_tree) {
      int dep = 0, j = tid;
      while (j > 0 && dep <= a.max_depth) {
        const int p = s_par[j];
        if (p < 0 || p >= j) break;  // reported by thread j
        j = p;
        ++dep;
      }
      if (dep > a.max_depth) bad_tree = 1;
    }
    if (block_or(bad_tree, &s_or)) err = SPEC_DEVERR_TREE;
    else if (block_or(bad_tok, &s_or)) err = SPEC_DEVERR_TOKEN;
  }
  if (err) {
    if (writer0) write_failure(a, b, err);
    return;
  }
  // each node's children as a bit mask (lowest set bit = lowest id), so that a
  // visit walks its own children only
  static_assert(SPEC_MAX_NODES <= 64, "children masks are 64 bits");
  if (tid < SPEC_MAX_NODES) s_kids[tid] = 0ull;
  __syncthreads();
  if (tid > 0 && tid < n) atomicOr(&s_kids[s_par[tid]], 1ull << tid);
  __syncthreads();

  int gen = 0;
  int v = 0, depth = 0;
  if (tid == 0) s_path[0] = 0;
  // Statistics of node la_node (max, sum and slice masses of its q), computed
  // in its parent's pass: the first child is the one most often accepted.
  // Worth it for short slices (NG <= 2), whose passes are bound by latency
  // rather than by the float64 work or HBM, and not with the filters.
  int la_node = -1;
  double la_M = 0.0, la_S = 0.0;
  bool la_nf = false;
  const size_t rows_b = (size_t)b * a.n_max;

  for (;;) {
    const float* lrow = a.logits + (rows_b + v) * (size_t)a.V;
    const float* prow = a.draft_p + (rows_b + v) * (size_t)a.pstride;

    if (greedy) {
      float bv = -INFINITY;
      int bi = 0x7fffffff, nf = 0;
      stream_slice<NG, W, BG1, false>(lrow, -INFINITY, lrow, 0.f, lo, hi,
          [&](int g0, float (*xv)[W], float (*)[W]) {
#pragma unroll
            for (int gb = 0; gb < BG1; ++gb)
#pragma unroll
              for (int j = 0; j < W; ++j) {
                const int i = elem_index<W>(lo, (g0 + gb) * W + j);
                if (i < hi) {
                  nf |= !isfinite(xv[gb][j]);
                  amax_combine(bv, bi, xv[gb][j], i);
                }
              }
          });
      nf = block_or(nf, &s_or);
      block_argmax(bv, bi, red);
      if (!exchange(a, ep, bl, part, gen, (double)bv, nf ? -1.0 : (double)bi, xs, &s_or)) {
        fail_sync(a, b, writer0);
        return;
      }
      const bool has = lane < a.KP;
      float gv = has ? (float)xs[lane][0] : -INFINITY;
      int gi = has ? (int)xs[lane][1] : 0x7fffffff;
      const bool gnf = __any(has && xs[lane][1] < 0.0);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float v2 = __shfl_xor(gv, o);
        const int i2 = __shfl_xor(gi, o);
        amax_combine(gv, gi, v2, i2);
      }
      if (gnf) {
        if (writer0) write_failure(a, b, SPEC_DEVERR_NONFINITE);
        return;
      }
      int nxt = -1;
      for (unsigned long long m = s_kids[v]; m; m &= m - 1) {
        const int c = __ffsll(m) - 1;
        if (s_tok[c] == gi) {
          nxt = c;
          break;
        }
      }
      __syncthreads();
      if (tid == 0) s_out[depth] = gi;
      if (nxt >= 0) {
        ++depth;
        if (tid == 0) s_path[depth] = nxt;
        v = nxt;
        continue;
      }
      __syncthreads();
      if (writer0) write_outputs(a, b, depth, s_path, s_out);
      if (a.final_dist) {
        float* fd = a.final_dist + (size_t)b * a.V;
        for (int i = lo + tid; i < hi; i += NT) fd[i] = (i == gi) ? 1.f : 0.f;
      }
      return;
    }

    // What the child tests and the terminal sample read, loaded now so that
    // the loads overlap the statistics pass.
    // The loads are unconditional, at indices valid for every thread (token 0
    // and row 0 where the thread holds no child); only the children's values
    // are used.  Loads under a branch would be waited for at once.
    const bool kid = tid > v && tid < n && s_par[tid] == v;
    float k_p = 0.f, k_l, k_u, k_us;
    {
      const int xt = kid ? s_tok[tid] : 0;
      if constexpr (MAPPED) {
        if (kid) {
          const int dx = a.t2d[xt];
          k_p = dx >= 0 ? prow[dx] : 0.f;
        }
      } else {
        k_p = prow[xt];
      }
      k_l = lrow[xt];
      k_u = a.u_accept[rows_b + (tid < a.n_max ? tid : 0)];
      k_us = a.u_sample[rows_b + v];
    }

    // ---- T > 0: max M and sum S of exp(z - M) over the row ------------------
    const bool has = lane < a.KP;
    bool scan_ok = true, scan_rel = true;  // scan: this node's sums of exp(z - M) (rescaled by mref)
    double M, S, pterm;
    const int c1 = s_kids[v] ? __ffsll((unsigned long long)s_kids[v]) - 1 : -1;
    if (LOOK && v == la_node) {
      // computed in the parent's pass; no per-group sums of this row, so a
      // terminal sample here streams the row in the selected workgroup
      la_node = -1;
      if (la_nf) {
        if (writer0) write_failure(a, b, SPEC_DEVERR_NONFINITE);
        return;
      }
      M = la_M;
      S = la_S;
      pterm = has ? la_sums[lane] : 0.0;
      scan_ok = false;
    } else if (LOOK && c1 >= 0) {
      // One pass over this row and the first child's.  This node has
      // children, so its visit ends in an accepted child or after a
      // rejection, whose pass rewrites scan: no per-group sums are kept.
      la_node = -1;
      const float* lrow2 = a.logits + (rows_b + c1) * (size_t)a.V;
      double m = -INFINITY, es = 0.0, m2 = -INFINITY, es2 = 0.0;
      int nf = 0, nf2 = 0;
      stream_slice<NG, W, BG2, true>(lrow, -INFINITY, lrow2, -INFINITY, lo, hi,
          [&](int g0, float (*xv)[W], float (*yv)[W]) {
            batch_stats<W, BG2>(lo, hi, g0, xv, invT, m, es, nf, s_tab, s_tab2);
            batch_stats<W, BG2>(lo, hi, g0, yv, invT, m2, es2, nf2, s_tab, s_tab2);
          });
      // (block_or is a predicate: one per row)
      const int nfv = block_or(nf, &s_or);
      const int nfc = block_or(nf2, &s_or);
      block_lse(m, es, red, s_tab);
      block_lse(m2, es2, red, s_tab);
      if (!exchange4(a, ep, bl, part, gen, m, nfv ? -1.0 : es, m2, nfc ? -1.0 : es2, xs4,
                     &s_or)) {
        fail_sync(a, b, writer0);
        return;
      }
      const double pm = has ? xs4[lane][0] : -INFINITY;
      const double ps = has ? xs4[lane][1] : 0.0;
      if (__any(has && ps < 0.0)) {
        if (writer0) write_failure(a, b, SPEC_DEVERR_NONFINITE);
        return;
      }
      M = uni(wave_max_d(pm));
      pterm = (has && pm != -INFINITY) ? ps * exp_tab(pm - M, s_tab) : 0.0;
      S = uni(wave_sum_d(pterm));
      const double pm2 = has ? xs4[lane][2] : -INFINITY;
      const double ps2 = has ? xs4[lane][3] : 0.0;
      la_nf = __any(has && ps2 < 0.0);
      la_M = uni(wave_max_d(pm2));
      const double pt2 = (has && pm2 != -INFINITY && ps2 > 0.0) ? ps2 * exp_tab(pm2 - la_M, s_tab) : 0.0;
      la_S = uni(wave_sum_d(pt2));
      if (tid < a.KP) la_sums[tid] = pt2;  // wave 0: lane == tid
      la_node = c1;
      scan_ok = false;
    } else {
      la_node = -1;
      double m = -INFINITY, es = 0.0;
      int nf = 0;
      stream_slice<NG, W, BG1, false>(lrow, -INFINITY, lrow, 0.f, lo, hi,
          [&](int g0, float (*xv)[W], float (*)[W]) {
            float bmax = -INFINITY, bmin = INFINITY;
#pragma unroll
            for (int gb = 0; gb < BG1; ++gb)
#pragma unroll
              for (int j = 0; j < W; ++j) {
                const bool valid = elem_index<W>(lo, (g0 + gb) * W + j) < hi;
                nf |= valid && !isfinite(xv[gb][j]);
                bmax = fmaxf(bmax, xv[gb][j]);
                if (!FILT) bmin = fminf(bmin, xv[gb][j]);
              }
            if (bmax == -INFINITY) {  // nothing valid in this batch
#pragma unroll
              for (int gb = 0; gb < BG1; ++gb) scan[g0 + gb][tid] = 0.0;
              mref[g0 / BG1][tid] = -INFINITY;
              return;
            }
            const double zb = (double)bmax * invT;
            if (zb > m) {
              es *= exp_tab(m - zb, s_tab);  // m = -inf: es is still 0
              m = zb;
            }
            mref[g0 / BG1][tid] = m;
            // the terms are +0 or positive, so starting from the first one
            // gives the same sum as starting from 0
            if (!FILT && __all(fma((double)bmin, invT, -m) >= kFastFloor)) {
#pragma unroll
              for (int gb = 0; gb < BG1; ++gb) {
                double sg = exp_fast(fma((double)xv[gb][0], invT, -m), s_tab2);
#pragma unroll
                for (int j = 1; j < W; ++j) sg += exp_fast(fma((double)xv[gb][j], invT, -m), s_tab2);
                es += sg;
                scan[g0 + gb][tid] = sg;
              }
            } else {
#pragma unroll
              for (int gb = 0; gb < BG1; ++gb) {
                double sg = exp_tab(fma((double)xv[gb][0], invT, -m), s_tab);
#pragma unroll
                for (int j = 1; j < W; ++j) sg += exp_tab(fma((double)xv[gb][j], invT, -m), s_tab);
                es += sg;
                scan[g0 + gb][tid] = sg;
              }
            }
          });
      nf = block_or(nf, &s_or);
      block_lse(m, es, red, s_tab);
      if (!exchange(a, ep, bl, part, gen, m, nf ? -1.0 : es, xs, &s_or)) {
        fail_sync(a, b, writer0);
        return;
      }
      // combine the KP partials, lane k of every wave taking partial k
      const double pm = has ? xs[lane][0] : -INFINITY;
      const double ps = has ? xs[lane][1] : 0.0;
      if (__any(has && ps < 0.0)) {
        if (writer0) write_failure(a, b, SPEC_DEVERR_NONFINITE);
        return;
      }
      M = uni(wave_max_d(pm));
      pterm = (has && pm != -INFINITY) ? ps * exp_tab(pm - M, s_tab) : 0.0;
      S = uni(wave_sum_d(pterm));
    }

    // ---- sampling filters: threshold, then the kept mass per slice ----------
    float lcut = -INFINITY;  // q is restricted to logits >= lcut
    // kept(x): x passes the filters (always, in a variant without them)
    auto kept = [&](float x) { return !FILT || x >= lcut; };
    bool masks = false;  // s_keep holds this row's kept entries
    if (FILT && (fk > 0 || fP > 0)) {
      double fmargin;
      if (!filter_threshold<NG, W, BG2>(a, ep, bl, part, gen, lrow, lo, hi, invT, M, S, fk, fP, s_tab,
                                        reinterpret_cast<uint32_t*>(&scan[4][0]),
                                        reinterpret_cast<uint64_t*>(&scan[0][0]), fsh, &s_or, lcut,
                                        fmargin)) {
        fail_sync(a, b, writer0);
        return;
      }
      if (writer0 && tid == 0 && fmargin < kFilterBand)
        log_tie(a, b, v, 3, a.top_p[b], fmargin);
      double ek = 0.0;
      unsigned long long km = 0;
      stream_slice<NG, W, BG2, false>(lrow, -INFINITY, lrow, 0.f, lo, hi,
          [&](int g0, float (*xv)[W], float (*)[W]) {
#pragma unroll
            for (int gb = 0; gb < BG2; ++gb) {
              double sg = 0.0;
#pragma unroll
              for (int j = 0; j < W; ++j)
                if (kept(xv[gb][j])) {
                  sg += exp_tab(fma((double)xv[gb][j], invT, -M), s_tab);
                  if (elem_index<W>(lo, (g0 + gb) * W + j) < hi)
                    km |= 1ull << ((g0 + gb) * W + j);
                }
              ek += sg;
              scan[g0 + gb][tid] = sg;
            }
          });
      s_keep[tid] = km;
      masks = true;
      scan_rel = false;  // the filter's histograms overwrote scan; it now holds kept sums
      ek = block_sum(ek, red);
      if (!exchange(a, ep, bl, part, gen, ek, 0.0, xs, &s_or)) {
        fail_sync(a, b, writer0);
        return;
      }
      pterm = has ? xs[lane][0] : 0.0;
      S = uni(wave_sum_d(pterm));
    }
    // slice masses of q (in units of S) for the sample when no child is rejected
    if (tid < a.KP) cur_sums[tid] = pterm;
    if (kid) {
      s_kp[tid] = k_p;
      s_kl[tid] = k_l;
      s_ku[tid] = k_u;
    }
    if (tid == 0) s_us = k_us;
    __syncthreads();

    // r = max(0, exp(z - M) - CS p) for one group of W entries (exp(z - M)
    // taken as 0 below the filters' threshold)
    auto r_group = [&](int g, double CS, bool use_p, double* rv, int* pnf) {
      float xv[W], pv[W];
      load_group<W>(lrow, lo, hi, g, -INFINITY, xv);
      if (use_p) {
        load_group_p<W, MAPPED>(prow, a.t2d, lo, hi, g, 0.f, pv);
      } else {
#pragma unroll
        for (int j = 0; j < W; ++j) pv[j] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < W; ++j) {
        *pnf |= !isfinite(pv[j]);
        const double e = kept(xv[j]) ? exp_tab(fma((double)xv[j], invT, -M), s_tab) : 0.0;
        rv[j] = fmax(0.0, e - CS * (double)pv[j]);
      }
    };

    // ---- children in ascending id against the running residual ------------
    double C = 0.0, Z = 1.0;
    int nxt = -1;
    bool p_read = false;  // a residual pass has read (and checked) the draft row
    for (unsigned long long km = s_kids[v]; km; km &= km - 1) {
      const int c = __ffsll(km) - 1;
      const int xt = s_tok[c];
      const float pxf = s_kp[c];
      if (!isfinite(pxf)) {
        if (writer0) write_failure(a, b, SPEC_DEVERR_NONFINITE);
        return;
      }
      const double px = (double)pxf;
      if (px <= 0.0) {
        nxt = c;
        break;
      }
      // u < min(1, cur / px), cur = max(0, exp(z - M) / S - C px) / Z, tested
      // without divisions as u px Z S < max(0, exp(z - M) - C px S) (u < 1);
      // the ratio itself is formed only for a near tie's record
      const double e = kept(s_kl[c]) ? exp_tab((double)s_kl[c] * invT - M, s_tab) : 0.0;
      const double pzs = px * Z * S;
      const double rhs = fmax(0.0, e - C * px * S);
      const float uf = s_ku[c];
      const double u = (double)uf;
      const double lhs = u * pzs;
      if (writer0 && tid == 0 && fabs(lhs - fmin(rhs, pzs)) < 2.0 * kTieBand * pzs) {
        const double thr = fmin(1.0, rhs / pzs);
        if (fabs(u - thr) < kTieBand) log_tie(a, b, c, 0, uf, fabs(u - thr));
      }
      if (lhs < rhs) {
        nxt = c;
        break;
      }
      // rejected: residual mass for the next coefficient, in units of S
      const double Cn = C + Z;
      double zp = 0.0;
      int pnf = 0;
      const double CnS = Cn * S;
      if (FILT && masks && p_read && !__any(__popcll(s_keep[tid]) > kMaskMax)) {
        // A later rejection at a filtered node: only kept entries contribute
        // (q is 0 elsewhere and the draft row, already checked, has no
        // negative entry), so each thread gathers just those.  The group sums
        // are the streamed pass's bit for bit (its other terms are zeros).
        // The thread's (at most kMaskMax = 2) kept entries, both loaded at
        // once at valid indices (loads under a branch would be waited for one
        // by one); every other group sum is zero.
        static_assert(kMaskMax == 2, "two kept entries per thread");
        const unsigned long long km = s_keep[tid];
        const unsigned long long km1 = km & (km - 1);
        const int k0 = km ? __ffsll(km) - 1 : -1;
        const int k1 = km1 ? __ffsll(km1) - 1 : -1;
        const int i0 = k0 >= 0 ? elem_index<W>(lo, k0) : lo;
        const int i1 = k1 >= 0 ? elem_index<W>(lo, k1) : lo;
        float p0, p1;
        if constexpr (MAPPED) {
          const int t0 = a.t2d[i0], t1 = a.t2d[i1];
          const float q0 = prow[max(t0, 0)], q1 = prow[max(t1, 0)];
          p0 = t0 >= 0 ? q0 : 0.f;
          p1 = t1 >= 0 ? q1 : 0.f;
        } else {
          p0 = prow[i0];
          p1 = prow[i1];
        }
        const float z0 = lrow[i0], z1 = lrow[i1];
        const double r0 = k0 < 0 ? 0.0
            : fmax(0.0, exp_tab(fma((double)z0, invT, -M), s_tab) - CnS * (double)p0);
        const double r1 = k1 < 0 ? 0.0
            : fmax(0.0, exp_tab(fma((double)z1, invT, -M), s_tab) - CnS * (double)p1);
#pragma unroll
        for (int g = 0; g < NG; ++g) scan[g][tid] = 0.0;
        // the streamed pass adds the same terms in the same order (the others
        // are +0), so these are its sums bit for bit
        if (k0 >= 0) scan[k0 / W][tid] = r0;
        if (k1 >= 0) scan[k1 / W][tid] = k1 / W == k0 / W ? r0 + r1 : r1;
        zp = r0 + r1;
      } else {
        bool pneg = false;
        stream_slice<NG, W, BG2, true, MAPPED>(lrow, -INFINITY, prow, 0.f, lo, hi,
            [&](int g0, float (*xv)[W], float (*pv)[W]) {
              // one batch with the given exp (a separate loop for each, so
              // that only the chosen one runs)
              auto batch = [&](auto expf) {
#pragma unroll
                for (int gb = 0; gb < BG2; ++gb) {
                  double sg = 0.0;
#pragma unroll
                  for (int j = 0; j < W; ++j) {
                    pnf |= !isfinite(pv[gb][j]);
                    if (FILT) pneg |= pv[gb][j] < 0.f;
                    const double e =
                        kept(xv[gb][j]) ? expf(fma((double)xv[gb][j], invT, -M)) : 0.0;
                    sg += fmax(0.0, e - CnS * (double)pv[gb][j]);
                  }
                  zp += sg;
                  scan[g0 + gb][tid] = sg;
                }
              };
              bool fast = false;
              if (!FILT) {
                float bmin = INFINITY;
#pragma unroll
                for (int gb = 0; gb < BG2; ++gb)
#pragma unroll
                  for (int j = 0; j < W; ++j) bmin = fminf(bmin, xv[gb][j]);
                fast = __all(fma((double)bmin, invT, -M) >= kFastFloor);
              }
              if (fast) batch([&](double y) { return exp_fast(y, s_tab2); });
              else batch([&](double y) { return exp_tab(y, s_tab); });
            }, a.t2d);
        if (FILT && masks && pneg) s_keep[tid] = ~0ull;
      }
      p_read = true;
      pnf = block_or(pnf, &s_or);
      zp = block_sum(zp, red);
      if (!exchange(a, ep, bl, part, gen, zp, (double)pnf, xs, &s_or)) {
        fail_sync(a, b, writer0);
        return;
      }
      const bool has = lane < a.KP;
      const double Zs = uni(wave_sum_d(has ? xs[lane][0] : 0.0));
      if (__any(has && xs[lane][1] != 0.0)) {
        if (writer0) write_failure(a, b, SPEC_DEVERR_NONFINITE);
        return;
      }
      const double Zn = Zs / S;
      // scan now holds the sums for coefficient Cn: right for the terminal
      // sample only if Cn is taken
      scan_ok = Zn > 0.0;
      scan_rel = false;
      if (Zn > 0.0) {
        if (writer0 && tid == 0 && Zn < kDegenerate * Z) log_tie(a, b, c, 2, uf, Zn / Z);
        C = Cn;
        Z = Zn;
        if (tid < a.KP) cur_sums[tid] = xs[tid][0];
        __syncthreads();
      }
    }
    if (nxt >= 0) {
      __syncthreads();
      if (tid == 0) {
        s_out[depth] = s_tok[nxt];
        s_path[depth + 1] = nxt;
      }
      ++depth;
      v = nxt;
      continue;
    }

    // ---- terminal token: inverse CDF over r (slice masses in cur_sums) ----
    const bool use_p = (C != 0.0);
    const double CS = C * S;
    double Wt = 0.0;
    for (int k = 0; k < a.KP; ++k) Wt += cur_sums[k];
    const float usf = s_us;
    const double thr = (double)usf * Wt;
    int sel = -1, last_pos = -1;
    double off = 0.0, off_sel = 0.0;
    for (int k = 0; k < a.KP; ++k) {
      if (cur_sums[k] > 0.0) last_pos = k;
      if (sel < 0 && off + cur_sums[k] > thr) {
        sel = k;
        off_sel = off;
      }
      off += cur_sums[k];
    }
    if (sel < 0) {
      sel = last_pos;
      off_sel = off - cur_sums[last_pos];
    }
    int dummy = 0;
    // One streamed pass over r (loads pipelined as in the statistics
    // passes): final_dist entry by entry, and in the workgroup of the
    // selected slice each thread's sum of r per group for the ordered scan.
    const bool is_sel = part == sel;
    if (a.final_dist || (is_sel && !scan_ok)) {
      float* fd = a.final_dist ? a.final_dist + (size_t)b * a.V : nullptr;
      auto body = [&](int g0, float (*xv)[W], float (*pv)[W]) {
#pragma unroll
        for (int gb = 0; gb < BG2; ++gb) {
          double t = 0.0;
#pragma unroll
          for (int j = 0; j < W; ++j) {
            const double e =
                kept(xv[gb][j]) ? exp_tab(fma((double)xv[gb][j], invT, -M), s_tab) : 0.0;
            const double r = fmax(0.0, e - (use_p ? CS * (double)pv[gb][j] : 0.0));
            t += r;
            const int i = elem_index<W>(lo, (g0 + gb) * W + j);
            if (fd && i < hi) fd[i] = (float)(r / Wt);
          }
          if (g0 + gb < NG) scan[g0 + gb][tid] = t;
        }
      };
      if (use_p)
        stream_slice<NG, W, BG2, true, MAPPED>(lrow, -INFINITY, prow, 0.f, lo, hi, body, a.t2d);
      else
        stream_slice<NG, W, BG2, false>(lrow, -INFINITY, lrow, 0.f, lo, hi, body);
    }
    if (!is_sel) return;
    if (!a.final_dist && scan_ok && scan_rel) {
      // sums of the statistics pass: relative to each thread's running max
      for (int g = 0; g < NG; ++g) scan[g][tid] *= exp_tab(mref[g / BG1][tid] - M, s_tab);
    }

    // Ordered scan of this slice (entries in ascending id: group, then
    // thread, then a thread's W entries), in parallel: the group holding the
    // threshold from the group totals (wave sums), then the thread from an
    // exclusive scan over the threads' sums of that group, then the entry
    // within the thread.
    __syncthreads();
    const int lane_ = tid & 63, wv_ = tid >> 6;
    // group totals in four parts per group (one per 64 threads), each a
    // plain running sum over LDS by one thread: short dependent chains
    // instead of a shuffle reduction per group
    if (tid < NG * (NT / 64)) {
      const int g = tid / (NT / 64), k = tid % (NT / 64);
      double t = 0.0;
      for (int i = 0; i < 64; ++i) t += scan[g][k * 64 + i];
      gsum_w[g][k] = t;
    }
    if (tid == 0) {
      s_first = 0x7fffffff;
      s_hit = -1;
    }
    __syncthreads();
    double run = off_sel;
    int gs = -1;
    for (int g = 0; g < NG; ++g) {
      double gt = 0.0;
#pragma unroll
      for (int k = 0; k < NT / 64; ++k) gt += gsum_w[g][k];
      if (gs < 0) {
        if (run + gt > thr) gs = g;
        else run += gt;
      }
    }
    const double tsel = gs >= 0 ? scan[gs][tid] : 0.0;
    double incl = tsel;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const double y = __shfl_up(incl, o);
      if (lane_ >= o) incl += y;
    }
    double excl = __shfl_up(incl, 1);
    if (lane_ == 0) excl = 0.0;
    if (lane_ == 63) wtot[wv_] = incl;
    __syncthreads();
    double woff = 0.0;
    for (int k = 0; k < wv_; ++k) woff += wtot[k];
    const double start = run + (woff + excl);
    if (gs >= 0 && tsel > 0.0 && start + tsel > thr) atomicMin(&s_first, tid);
    __syncthreads();
    double margin = 0.0;
    if (gs >= 0 && tid == s_first) {
      double rv[W];
      r_group(gs, CS, use_p, rv, &dummy);
      double cum = start;
      int tok = -1, lastp = -1;
#pragma unroll
      for (int j = 0; j < W; ++j) {
        if (rv[j] > 0.0) {
          lastp = elem_index<W>(lo, gs * W + j);
          if (tok < 0 && cum + rv[j] > thr) {
            tok = lastp;
            margin = fmin(thr - cum, cum + rv[j] - thr) / Wt;
          }
        }
        cum += rv[j];
      }
      if (tok < 0) {  // rounding: the thread's own running sum stayed below
        tok = lastp;
        margin = 0.0;
      }
      s_hit = tok;
    }
    __syncthreads();
    if (s_hit < 0) {
      // rounding left the threshold past this slice: its last positive entry
      int lastpos = -1;
#pragma unroll 1
      for (int g = 0; g < NG; ++g) {
        double rv[W];
        r_group(g, CS, use_p, rv, &dummy);
#pragma unroll
        for (int j = 0; j < W; ++j)
          if (rv[j] > 0.0) lastpos = max(lastpos, elem_index<W>(lo, g * W + j));
      }
      if (lastpos >= 0) atomicMax(&s_hit, lastpos);
      __syncthreads();
      if (tid == 0) log_tie(a, b, v, 1, usf, 0.0);
    } else if (tid == s_first && margin < kSampleBand) {
      log_tie(a, b, v, 1, usf, margin);
    }
    __syncthreads();
    if (tid == 0) s_out[depth] = s_hit;
    __syncthreads();
    write_outputs(a, b, depth, s_path, s_out);
    return;
  }
}

// Clears the near-tie counter (only launched when the caller logs ties).
__global__ void accept_init_kernel(int32_t* tie_count) {
  if (threadIdx.x == 0) *tie_count = 0;
}

// Launch ids for exchange tags: 32 bits, never 0, distinct for 2^32 launches
// of this process; the start is drawn from the clock and the process id so
// that words left in reused memory by another process are unlikely to carry a
// current tag.
uint64_t next_epoch() {
  static std::atomic<uint64_t> counter{0};
  static const uint64_t start = [] {
    const uint64_t t = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
    return (t * 0x9E3779B97F4A7C15ull) ^ ((uint64_t)getpid() << 20);
  }();
  for (;;) {
    const uint64_t e = (start + counter.fetch_add(1, std::memory_order_relaxed)) & 0xFFFFFFFFull;
    if (e != 0) return e;
  }
}

typedef void (*accept_fn)(AcceptArgs);

template <bool MAPPED, bool FILT>
accept_fn pick_variant(int w, int ng) {
  if (w == 4) {
    switch (ng) {
      case 1: return accept_kernel<1, 4, MAPPED, FILT>;
      case 2: return accept_kernel<2, 4, MAPPED, FILT>;
      case 4: return accept_kernel<4, 4, MAPPED, FILT>;
      case 8: return accept_kernel<8, 4, MAPPED, FILT>;
      default: return accept_kernel<16, 4, MAPPED, FILT>;
    }
  }
  switch (ng) {
    case 1: return accept_kernel<1, 1, MAPPED, FILT>;
    case 2: return accept_kernel<2, 1, MAPPED, FILT>;
    case 4: return accept_kernel<4, 1, MAPPED, FILT>;
    case 8: return accept_kernel<8, 1, MAPPED, FILT>;
    default: return accept_kernel<16, 1, MAPPED, FILT>;
  }
}

accept_fn pick_kernel(int w, int ng, bool mapped = false, bool filt = false) {
  if (filt) return mapped ? pick_variant<true, true>(w, ng) : pick_variant<false, true>(w, ng);
  return mapped ? pick_variant<true, false>(w, ng) : pick_variant<false, false>(w, ng);
}

// Inverse of a draft-vocabulary map: t2d[x] = i where x = i + d2t[i], -1 for
// target tokens no draft id maps to; *bad set when the map leaves [0, V) or
// is not one-to-one.  Two launches: fill, then scatter.
// Zeroes the histogram exchange buffers of a filtered call.
__global__ void hist_clear_kernel(uint64_t* h, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    h[i] = 0;
}

__global__ void t2d_fill_kernel(int32_t* t2d, int V, int32_t* bad) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < V) t2d[i] = -1;
  if (i == 0) *bad = 0;
}
__global__ void t2d_scatter_kernel(const int32_t* d2t, int Vd, int V, int32_t* t2d, int32_t* bad) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= Vd) return;
  const long x = (long)i + d2t[i];
  if (x < 0 || x >= V) {
    atomicOr(bad, 1);
    return;
  }
  if (atomicCAS(t2d + x, -1, i) != -1) atomicOr(bad, 1);
}

// Groups per thread are capped so the sample scan's [NG][NT] float64 table
// stays at 32 KB of LDS.
constexpr int kMaxNG = 16;

struct AcceptPlan {
  int KP = 1;      // workgroups per sequence
  int NG = 1;      // element groups per thread
  int W = 1;       // entries per group: 4 when rows allow 16-byte loads
  int chunk = 0;   // entries per workgroup
  size_t ws = 0;   // workspace bytes: exchange words | inverse draft map | histograms |
                   // per-sequence launch counters
  size_t off_t2d = 0, off_hist = 0, off_seq = 0;
};

// Workgroups of the (W, NG) variant one compute unit holds at once, cached
// (relaxed atomics: concurrent first calls store the same value).
int resident_per_cu(int w, int ng, bool mapped, bool filt) {
  static std::atomic<int> cache[2][2][2][5];
  const int wi = w == 4 ? 1 : 0;
  const int mi = mapped ? 1 : 0;
  const int fi = filt ? 1 : 0;
  int ni = 0;
  while ((1 << ni) < ng) ++ni;
  const int c = cache[fi][mi][wi][ni].load(std::memory_order_relaxed);
  if (c > 0) return c;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(pick_kernel(w, ng, mapped, filt)), NT, 0) !=
      hipSuccess)
    per_cu = 1;
  if (per_cu < 1) per_cu = 1;
  cache[fi][mi][wi][ni].store(per_cu, std::memory_order_relaxed);
  return per_cu;
}

// KP workgroups of NT threads per sequence, each over NG groups of W entries.
// The largest KP (most parallel vocabulary passes) whose B * KP workgroups
// are all resident at once, so the whole batch walks in one launch; beyond
// that (very large batches) the fewest workgroups per
// sequence, walked in consecutive groups of sequences.
AcceptPlan make_accept_plan(int B, int V, bool mapped = false, bool filters = false) {
  AcceptPlan p;
  p.W = (V % 4) == 0 ? 4 : 1;
  const long per_group = (long)NT * p.W;
  const int cus = device_cu_count();
  long forced = 0;
  if (const char* env = getenv("SPEC_ACCEPT_PARTS")) {  // tuning sweeps
    const long e = atol(env);
    if (e >= 1 && e <= SPEC_MAX_NODES) forced = e;
  }
  int best_ng = kMaxNG;
  if (forced) {
    const long need = (V + forced * per_group - 1) / (forced * per_group);
    best_ng = 1;
    while (best_ng < need && best_ng < kMaxNG) best_ng *= 2;
  } else {
    for (int ng = 1; ng <= kMaxNG; ng *= 2) {
      const long kp = (V + per_group * ng - 1) / (per_group * ng);
      if (kp > SPEC_MAX_NODES) continue;
      if ((long)B * kp <= (long)resident_per_cu(p.W, ng, mapped, filters) * cus) {
        best_ng = ng;
        break;
      }
    }
  }
  p.NG = best_ng;
  p.chunk = (int)(per_group * best_ng);
  p.KP = (V + p.chunk - 1) / p.chunk;
  auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
  p.ws = p.KP > 1 ? (size_t)B * 2 * p.KP * kSlotWords * sizeof(uint64_t) : 256;
  if (mapped) {
    p.off_t2d = align(p.ws);
    p.ws = p.off_t2d + (size_t)V * sizeof(int32_t) + 256;
  }
  if (filters && p.KP > 1) {
    p.off_hist = align(p.ws);
    p.ws = p.off_hist + (size_t)B * 2 * p.KP * 512 * sizeof(uint64_t);
  }
  if (p.KP > 1) {
    p.off_seq = align(p.ws);
    p.ws = p.off_seq + (size_t)B * sizeof(uint32_t);
  }
  return p;
}

}  // namespace
}  // namespace specv

using namespace specv;

extern "C" size_t spec_accept_tree_workspace_size(int32_t B, int32_t n_max, int32_t V) {
  if (B <= 0 || n_max <= 0 || V <= 0) return 0;
  (void)n_max;
  return make_accept_plan(B, V).ws;
}

extern "C" size_t spec_accept_tree_ex_workspace_size(int32_t B, int32_t n_max, int32_t V,
                                                     int32_t Vd, int32_t filters) {
  if (B <= 0 || n_max <= 0 || V <= 0 || Vd < 0 || Vd > V) return 0;
  (void)n_max;
  return make_accept_plan(B, V, Vd > 0, filters != 0).ws;
}

extern "C" spec_status_t spec_accept_tree_ex(
    const int32_t* tokens, const int32_t* parents, const int32_t* n_nodes, const float* draft_p,
    const float* logits, int32_t B, int32_t n_max, int32_t V, int32_t max_depth,
    float temperature, const float* temperatures, const int32_t* top_k, const float* top_p,
    const int32_t* d2t, int32_t Vd, const float* u_accept, const float* u_sample,
    int32_t* accept_len, int32_t* path, int32_t* out_tokens, int32_t* n_out, float* final_dist,
    spec_tie_t* tie_log, int32_t tie_cap, int32_t* tie_count, void* workspace,
    size_t workspace_bytes, int32_t launch, int32_t* dev_error, void* stream) {
  if (!tokens || !parents || !n_nodes || !draft_p || !logits || !u_accept || !u_sample ||
      !accept_len || !path || !out_tokens || !n_out)
    return SPEC_E_NULL;
  if (launch != SPEC_LAUNCH_ORDINARY && launch != SPEC_LAUNCH_COOPERATIVE) return SPEC_E_VALUE;
  const bool mapped = d2t != nullptr;
  if (mapped && (Vd <= 0 || Vd > V)) return SPEC_E_SHAPE;
  if (tie_log && !tie_count) return SPEC_E_NULL;
  if (B <= 0 || n_max <= 0 || n_max > SPEC_MAX_NODES || V <= 0 ||
      V > SPEC_MAX_NODES * NT * kMaxNG * (V % 4 == 0 ? 4 : 1) || max_depth < 0 || max_depth >= SPEC_MAX_NODES ||
      (tie_log && tie_cap < 0))
    return SPEC_E_SHAPE;
  if (!temperatures && (!(temperature >= 0.f) || !isfinite(temperature))) return SPEC_E_VALUE;
  const bool filters = top_k != nullptr || top_p != nullptr;
  AcceptPlan p = make_accept_plan(B, V, mapped, filters);
  if (p.KP > SPEC_MAX_NODES) return SPEC_E_SHAPE;
  if (!workspace || workspace_bytes < p.ws) return SPEC_E_WORKSPACE;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);

  AcceptArgs a;
  a.tokens = tokens; a.parents = parents; a.n_nodes = n_nodes;
  a.draft_p = draft_p; a.logits = logits;
  a.B = B; a.n_max = n_max; a.V = V; a.max_depth = max_depth;
  a.greedy = temperature == 0.f ? 1 : 0;
  a.inv_T = a.greedy || temperatures ? 0.0 : 1.0 / (double)temperature;
  a.temps = temperatures;
  a.pstride = mapped ? Vd : V;
  a.t2d = nullptr;
  a.t2d_bad = nullptr;
  a.top_k = top_k;
  a.top_p = top_p;
  a.hist = filters && p.KP > 1
               ? reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + p.off_hist)
               : nullptr;
  a.u_accept = u_accept; a.u_sample = u_sample;
  a.accept_len = accept_len; a.path = path; a.out_tokens = out_tokens; a.n_out = n_out;
  a.final_dist = final_dist; a.tie_log = tie_log; a.tie_cap = tie_cap; a.tie_count = tie_count;
  a.KP = p.KP;
  a.chunk = p.chunk;
  a.slots = static_cast<uint64_t*>(workspace);
  a.seq_epoch = p.KP > 1 ? reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + p.off_seq)
                         : nullptr;
  a.dev_error = dev_error;
  // bound on the polls of one inter-workgroup wait; tests set a negative
  // bound, which makes every wait give up at once, to drive the failure path
  a.spin_limit = 1 << 22;
  if (const char* env = getenv("SPEC_ACCEPT_SPIN_LIMIT")) a.spin_limit = atoi(env);
  const accept_fn fn = pick_kernel(p.W, p.NG, mapped, filters);
  const bool cooperative = launch == SPEC_LAUNCH_COOPERATIVE;

  // Sequences per launch: all of them, unless the KP > 1 workgroups of every
  // sequence cannot be resident together (their exchanges need that).
  int group = B;
  if (p.KP > 1) {
    const long resident = (long)resident_per_cu(p.W, p.NG, mapped, filters) * device_cu_count();
    if (resident < p.KP) return SPEC_E_UNSUPPORTED;
    group = (int)(resident / p.KP < B ? resident / p.KP : B);
  }
  if (tie_count) {
    hipLaunchKernelGGL(accept_init_kernel, dim3(1), dim3(64), 0, strm, tie_count);
    SPEC_HIP_TRY(hipGetLastError());
  }
  if (a.hist) {
    const size_t n = (size_t)B * 2 * p.KP * 512;
    const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(hist_clear_kernel, dim3(blocks), dim3(256), 0, strm, a.hist, n);
    SPEC_HIP_TRY(hipGetLastError());
  }
  if (mapped) {  // inverse map in the workspace, after the exchange words
    int32_t* t2d = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + p.off_t2d);
    int32_t* bad = t2d + V;
    hipLaunchKernelGGL(t2d_fill_kernel, dim3((V + 255) / 256), dim3(256), 0, strm, t2d, V, bad);
    SPEC_HIP_TRY(hipGetLastError());
    hipLaunchKernelGGL(t2d_scatter_kernel, dim3((Vd + 255) / 256), dim3(256), 0, strm, d2t, Vd, V,
                       t2d, bad);
    SPEC_HIP_TRY(hipGetLastError());
    a.t2d = t2d;
    a.t2d_bad = bad;
  }
  for (int b0 = 0; b0 < B; b0 += group) {
    const int nb = B - b0 < group ? B - b0 : group;
    a.b0 = b0;
    a.epoch = next_epoch();
    const unsigned grid = (unsigned)((long)nb * p.KP);
    if (p.KP == 1) {
      hipLaunchKernelGGL(fn, dim3(grid), dim3(NT), 0, strm, a);
      SPEC_HIP_TRY(hipGetLastError());
    } else {
      // The plan keeps every workgroup of the launch resident at once on an
      // otherwise idle GPU, so the ordinary launch suffices there (a
      // cooperative one costs about 17 us more per call); the cooperative
      // launch has the runtime guarantee residency where the GPU is shared.
      if (cooperative) {
        void* args[] = {&a};
        SPEC_HIP_TRY(hipLaunchCooperativeKernel(reinterpret_cast<const void*>(fn), dim3(grid),
                                                dim3(NT), args, 0, strm));
      } else {
        hipLaunchKernelGGL(fn, dim3(grid), dim3(NT), 0, strm, a);
        SPEC_HIP_TRY(hipGetLastError());
      }
    }
  }
  return SPEC_OK;
}

extern "C" spec_status_t spec_accept_tree(
    const int32_t* tokens, const int32_t* parents, const int32_t* n_nodes, const float* draft_p,
    const float* logits, int32_t B, int32_t n_max, int32_t V, int32_t max_depth,
    float temperature, const float* u_accept, const float* u_sample, int32_t* accept_len,
    int32_t* path, int32_t* out_tokens, int32_t* n_out, float* final_dist, spec_tie_t* tie_log,
    int32_t tie_cap, int32_t* tie_count, void* workspace, size_t workspace_bytes,
    int32_t* dev_error, void* stream) {
  return spec_accept_tree_ex(tokens, parents, n_nodes, draft_p, logits, B, n_max, V, max_depth,
                             temperature, nullptr, nullptr, nullptr, nullptr, 0, u_accept,
                             u_sample, accept_len, path, out_tokens, n_out, final_dist, tie_log,
                             tie_cap, tie_count, workspace, workspace_bytes, SPEC_LAUNCH_ORDINARY,
                             dev_error, stream);
}

// ---- the allocation-free form ------------------------------------------------
namespace specv {
namespace {

// Scratch of spec_accept_tree_noalloc: the exchange words of one call, in a
// fixed array of the code object (one copy per GPU, zero at load, held until
// the process ends).  Host code must not pass `scratch` itself to a kernel:
// its host-side name is not the device address, which noalloc_scratch()
// looks up per device.
__device__ __align__(256) uint8_t scratch[SPEC_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];

// The device address of the current GPU's copy of `scratch`, looked up with
// hipGetSymbolAddress on the first call with that GPU current and kept.
spec_status_t noalloc_scratch(void** addr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SPEC_E_HIP;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return SPEC_E_HIP;
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *addr = p;
  return SPEC_OK;
}

}  // namespace
}  // namespace specv

extern "C" spec_status_t spec_accept_tree_noalloc(
    const int32_t* tokens, const int32_t* parents, const int32_t* n_nodes, const float* draft_p,
    const float* logits, int32_t B, int32_t n_max, int32_t V, int32_t max_depth,
    float temperature, const float* u_accept, const float* u_sample, int32_t* accept_len,
    int32_t* path, int32_t* out_tokens, int32_t* n_out, float* final_dist, spec_tie_t* tie_log,
    int32_t tie_cap, int32_t* tie_count, int32_t* dev_error, void* stream) {
  // the argument checks of spec_accept_tree come first, so that a bad
  // argument reports the same status as there, without touching a device
  if (!tokens || !parents || !n_nodes || !draft_p || !logits || !u_accept || !u_sample ||
      !accept_len || !path || !out_tokens || !n_out || (tie_log && !tie_count))
    return SPEC_E_NULL;
  if (B <= 0 || n_max <= 0 || n_max > SPEC_MAX_NODES || V <= 0 || max_depth < 0 ||
      max_depth >= SPEC_MAX_NODES || (tie_log && tie_cap < 0))
    return SPEC_E_SHAPE;
  if (!(temperature >= 0.f) || !isfinite(temperature)) return SPEC_E_VALUE;
  if (make_accept_plan(B, V).ws > SPEC_NOALLOC_SCRATCH_BYTES) return SPEC_E_SCRATCH;
  void* ws = nullptr;
  const spec_status_t st = noalloc_scratch(&ws);
  if (st != SPEC_OK) return st;
  return spec_accept_tree_ex(tokens, parents, n_nodes, draft_p, logits, B, n_max, V, max_depth,
                             temperature, nullptr, nullptr, nullptr, nullptr, 0, u_accept,
                             u_sample, accept_len, path, out_tokens, n_out, final_dist, tie_log,
                             tie_cap, tie_count, ws, SPEC_NOALLOC_SCRATCH_BYTES,
                             SPEC_LAUNCH_ORDINARY, dev_error, stream);
}
