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
// Z_{k+1} = sum(max(0, q - C_{k+1} p)), so each rejection costs one vocab pass
// and no row is materialised.  Temperature 0 is greedy decoding (accept iff
// the token is the verifier's argmax; emit the argmax).
//
// Shape on the GPU.  The walk is serial along the tree but each step is a
// vocab-wide reduction over 32k-128k entries, so every sequence gets KP
// workgroups, each owning a contiguous slice of the vocabulary.  They run
// the same control flow and meet at a per-sequence barrier (one atomic
// counter) after every pass, exchanging one or two float64 partials; the
// combined values are formed in slice order, so every workgroup takes the
// same decisions.  KP > 1 uses a cooperative launch so that all workgroups
// are resident; every wait is bounded.  All vocab arithmetic is float64: the
// verifier row is read once per visited node (max and sum of exp), once more
// per rejected child (residual mass), and the terminal sample reads the final
// row again (slice masses, then one workgroup scans its slice).
#include <math.h>
#include <stdlib.h>

#include "common.hpp"

namespace specv {
namespace {

constexpr int NT = 256;   // threads per workgroup
constexpr double kTieBand = 1e-6;
constexpr double kSampleBand = 1e-9;
constexpr double kDegenerate = 1e-12;

struct AcceptArgs {
  const int32_t* tokens;
  const int32_t* parents;
  const int32_t* n_nodes;
  const float* draft_p;
  const float* logits;
  int B, n_max, V, max_depth, greedy;
  double T;
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
  int KP;       // workgroups per sequence
  int chunk;    // vocabulary entries per workgroup
  int* bar;     // [B] arrival counters (zeroed before the launch)
  double* part; // [B][KP][2 slots][2]
  int32_t* dev_error;
  int spin_limit;
};

// ---- block reductions (fixed order, so results are deterministic) ---------
__device__ double block_sum(double v, double* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int wv = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wv] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) t += red[k];
  return t;
}

__device__ __forceinline__ void lse_combine(double& m, double& s, double m2, double s2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) {
    m = m2;
    s = s2;
    return;
  }
  if (m2 > m) {
    s = s * exp(m - m2) + s2;
    m = m2;
  } else {
    s += s2 * exp(m2 - m);
  }
}

__device__ void block_lse(double& m, double& s, double* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const double m2 = __shfl_xor(m, o);
    const double s2 = __shfl_xor(s, o);
    lse_combine(m, s, m2, s2);
  }
  const int wv = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    red[2 * wv] = m;
    red[2 * wv + 1] = s;
  }
  __syncthreads();
  double mm = -INFINITY, ss = 0.0;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) lse_combine(mm, ss, red[2 * k], red[2 * k + 1]);
  m = mm;
  s = ss;
}

// argmax with lowest index on ties; NaN-free inputs (NaN is flagged separately)
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

__device__ int block_or(int f, int* s_or) {
  __syncthreads();
  if (threadIdx.x == 0) *s_or = 0;
  __syncthreads();
  if (f) atomicOr(s_or, 1);
  __syncthreads();
  return *s_or;
}

// ---- inter-workgroup exchange ---------------------------------------------
// Publishes this workgroup's two partials, waits until all KP workgroups of
// the sequence have published theirs, and loads every partial into xs.
__device__ bool exchange(const AcceptArgs& a, int b, int part, int& gen, double v0, double v1,
                         double (*xs)[2], int* s_ok) {
  if (a.KP == 1) {
    __syncthreads();
    if (threadIdx.x == 0) {
      xs[0][0] = v0;
      xs[0][1] = v1;
    }
    __syncthreads();
    return true;
  }
  const int slot = gen & 1;
  ++gen;
  __syncthreads();
  if (threadIdx.x == 0) {
    double* dst = a.part + (((size_t)b * a.KP + part) * 2 + slot) * 2;
    __hip_atomic_store(dst, v0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(dst + 1, v1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(a.bar + b, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    const int target = gen * a.KP;
    int ok = 1, spins = 0;
    while (__hip_atomic_load(a.bar + b, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > a.spin_limit) {
        ok = 0;
        break;
      }
    }
    *s_ok = ok;
  }
  __syncthreads();
  if (!*s_ok) return false;
  if ((int)threadIdx.x < a.KP) {
    const double* src = a.part + (((size_t)b * a.KP + threadIdx.x) * 2 + slot) * 2;
    xs[threadIdx.x][0] = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    xs[threadIdx.x][1] = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return true;
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

// Load one element group of the slice: 4 entries with VEC, else 1.
template <bool VEC>
__device__ __forceinline__ int load_group(const float* row, int i, int hi, float* x) {
  if (VEC) {
    const float4 f = *reinterpret_cast<const float4*>(row + i);
    x[0] = f.x; x[1] = f.y; x[2] = f.z; x[3] = f.w;
    return 4;
  }
  x[0] = row[i];
  return 1;
}

template <bool VEC>
__global__ __launch_bounds__(NT) void accept_kernel(AcceptArgs a) {
  constexpr int W = VEC ? 4 : 1;
  __shared__ int s_par[SPEC_MAX_NODES];
  __shared__ int s_tok[SPEC_MAX_NODES];
  __shared__ int s_path[SPEC_MAX_NODES + 1];
  __shared__ int s_out[SPEC_MAX_NODES + 1];
  __shared__ double red[2 * (NT / 64)];
  __shared__ double xs[SPEC_MAX_NODES][2];
  __shared__ double scan[NT];
  __shared__ int s_ok, s_or, s_hit;

  const int b = blockIdx.x / a.KP;
  const int part = blockIdx.x % a.KP;
  const int tid = threadIdx.x;
  const int lo = part * a.chunk;
  const int hi = min(a.V, lo + a.chunk);
  const bool writer0 = (part == 0);

  // ---- validation (identical in every workgroup of the sequence) ----------
  const int n = a.n_nodes[b];
  int err = 0;
  if (n < 1 || n > a.n_max) {
    err = SPEC_DEVERR_TREE;
  } else {
    int bad_tree = 0, bad_tok = 0;
    if (tid < n) {
      const int p = a.parents[(size_t)b * a.n_max + tid];
      const int tk = a.tokens[(size_t)b * a.n_max + tid];
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
        if (p < 0 || p >= j) break;  // reported above by thread j
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

  int gen = 0;
  int v = 0, depth = 0;
  if (tid == 0) s_path[0] = 0;
  const double T = a.T;
  const size_t rows_b = (size_t)b * a.n_max;

  for (;;) {
    const float* lrow = a.logits + (rows_b + v) * (size_t)a.V;
    const float* prow = a.draft_p + (rows_b + v) * (size_t)a.V;

    if (a.greedy) {
      float bv = -INFINITY;
      int bi = 0x7fffffff, nf = 0;
      for (int i = lo + tid * W; i < hi; i += NT * W) {
        float x[4];
        const int cnt = load_group<VEC>(lrow, i, hi, x);
        for (int k = 0; k < cnt; ++k) {
          if (!isfinite(x[k])) nf = 1;
          amax_combine(bv, bi, x[k], i + k);
        }
      }
      nf = block_or(nf, &s_or);
      block_argmax(bv, bi, red);
      if (!exchange(a, b, part, gen, (double)bv, (double)bi + (nf ? 0.5 : 0.0), xs, &s_ok)) {
        if (writer0) write_failure(a, b, SPEC_DEVERR_SYNC);
        return;
      }
      float gv = -INFINITY;
      int gi = 0x7fffffff, gnf = 0;
      for (int k = 0; k < a.KP; ++k) {
        const double enc = xs[k][1];
        const int ik = (int)enc;
        if (enc != (double)ik) gnf = 1;
        amax_combine(gv, gi, (float)xs[k][0], ik);
      }
      if (gnf) {
        if (writer0) write_failure(a, b, SPEC_DEVERR_NONFINITE);
        return;
      }
      int nxt = -1;
      for (int c = v + 1; c < n; ++c)
        if (s_par[c] == v && s_tok[c] == gi) {
          nxt = c;
          break;
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

    // ---- T > 0: max and sum of exp of the verifier row (float64) ----------
    double m = -INFINITY, ssum = 0.0;
    int nf = 0;
    for (int i = lo + tid * W; i < hi; i += NT * W) {
      float x[4];
      const int cnt = load_group<VEC>(lrow, i, hi, x);
      for (int k = 0; k < cnt; ++k) {
        if (!isfinite(x[k])) nf = 1;
        const double z = (double)x[k] / T;
        if (z > m) {
          ssum = ssum * exp(m - z) + 1.0;
          m = z;
        } else {
          ssum += exp(z - m);
        }
      }
    }
    nf = block_or(nf, &s_or);
    block_lse(m, ssum, red);
    if (!exchange(a, b, part, gen, m, nf ? -1.0 : ssum, xs, &s_ok)) {
      if (writer0) write_failure(a, b, SPEC_DEVERR_SYNC);
      return;
    }
    double M = -INFINITY, S = 0.0;
    int gnf = 0;
    for (int k = 0; k < a.KP; ++k) {
      if (xs[k][1] < 0.0) gnf = 1;
      lse_combine(M, S, xs[k][0], xs[k][1]);
    }
    if (gnf) {
      if (writer0) write_failure(a, b, SPEC_DEVERR_NONFINITE);
      return;
    }

    // ---- children in ascending id against the running residual ------------
    double C = 0.0, Z = 1.0;
    int nxt = -1;
    for (int c = v + 1; c < n && nxt < 0; ++c) {
      if (s_par[c] != v) continue;
      const int x = s_tok[c];
      const float pxf = prow[x];
      if (!isfinite(pxf)) {
        if (writer0) write_failure(a, b, SPEC_DEVERR_NONFINITE);
        return;
      }
      const double px = (double)pxf;
      if (px <= 0.0) {
        nxt = c;
        break;
      }
      const double qx = exp((double)lrow[x] / T - M) / S;
      const double cur = fmax(0.0, qx - C * px) / Z;
      const double thr = fmin(1.0, cur / px);
      const float uf = a.u_accept[rows_b + c];
      const double u = (double)uf;
      if (writer0 && tid == 0 && fabs(u - thr) < kTieBand) log_tie(a, b, c, 0, uf, fabs(u - thr));
      if (u < thr) {
        nxt = c;
        break;
      }
      // rejected: residual mass for the next coefficient
      const double Cn = C + Z;
      double zp = 0.0;
      int pnf = 0;
      for (int i = lo + tid * W; i < hi; i += NT * W) {
        float xl[4], xp[4];
        const int cnt = load_group<VEC>(lrow, i, hi, xl);
        load_group<VEC>(prow, i, hi, xp);
        for (int k = 0; k < cnt; ++k) {
          if (!isfinite(xp[k])) pnf = 1;
          const double q = exp((double)xl[k] / T - M) / S;
          zp += fmax(0.0, q - Cn * (double)xp[k]);
        }
      }
      pnf = block_or(pnf, &s_or);
      zp = block_sum(zp, red);
      if (!exchange(a, b, part, gen, zp, (double)pnf, xs, &s_ok)) {
        if (writer0) write_failure(a, b, SPEC_DEVERR_SYNC);
        return;
      }
      double Zn = 0.0;
      int gp = 0;
      for (int k = 0; k < a.KP; ++k) {
        Zn += xs[k][0];
        gp |= (xs[k][1] != 0.0);
      }
      if (gp) {
        if (writer0) write_failure(a, b, SPEC_DEVERR_NONFINITE);
        return;
      }
      if (Zn > 0.0) {
        if (writer0 && tid == 0 && Zn < kDegenerate * Z) log_tie(a, b, c, 2, uf, Zn / Z);
        C = Cn;
        Z = Zn;
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

    // ---- terminal token: inverse CDF over r = max(0, q - C p) ------------
    const bool use_p = (C != 0.0);
    double wp = 0.0;
    for (int i = lo + tid * W; i < hi; i += NT * W) {
      float xl[4], xp[4] = {0.f, 0.f, 0.f, 0.f};
      const int cnt = load_group<VEC>(lrow, i, hi, xl);
      if (use_p) load_group<VEC>(prow, i, hi, xp);
      for (int k = 0; k < cnt; ++k) {
        const double q = exp((double)xl[k] / T - M) / S;
        wp += fmax(0.0, q - C * (double)xp[k]);
      }
    }
    wp = block_sum(wp, red);
    if (!exchange(a, b, part, gen, wp, 0.0, xs, &s_ok)) {
      if (writer0) write_failure(a, b, SPEC_DEVERR_SYNC);
      return;
    }
    double Wt = 0.0;
    for (int k = 0; k < a.KP; ++k) Wt += xs[k][0];
    const float usf = a.u_sample[rows_b + v];
    const double thr = (double)usf * Wt;
    // the slice holding the threshold (running sum in slice order)
    int sel = -1, last_pos = -1;
    double off = 0.0, off_sel = 0.0;
    for (int k = 0; k < a.KP; ++k) {
      if (xs[k][0] > 0.0) last_pos = k;
      if (sel < 0 && off + xs[k][0] > thr) {
        sel = k;
        off_sel = off;
      }
      off += xs[k][0];
    }
    if (sel < 0) {
      sel = last_pos;
      off_sel = off - xs[last_pos][0];
    }
    if (a.final_dist) {
      float* fd = a.final_dist + (size_t)b * a.V;
      for (int i = lo + tid; i < hi; i += NT) {
        const double q = exp((double)lrow[i] / T - M) / S;
        fd[i] = (float)(fmax(0.0, q - C * (use_p ? (double)prow[i] : 0.0)) / Wt);
      }
    }
    if (part != sel) return;

    // scan of this slice: each thread sums a contiguous run, then the thread
    // whose run holds the threshold walks it element by element, comparing
    // run-local sums so that the walk repeats the run total's rounding.
    const int len = hi - lo;
    const int per = (len + NT - 1) / NT;
    const int r0 = min(hi, lo + tid * per);
    const int r1 = min(hi, r0 + per);
    double tsum = 0.0;
    for (int i = r0; i < r1; ++i) {
      const double q = exp((double)lrow[i] / T - M) / S;
      tsum += fmax(0.0, q - C * (use_p ? (double)prow[i] : 0.0));
    }
    scan[tid] = tsum;
    __syncthreads();
    if (tid == 0) {
      double run = off_sel;
      for (int k = 0; k < NT; ++k) {
        const double t = scan[k];
        scan[k] = run;  // exclusive prefix in slice order
        run += t;
      }
      s_hit = 0x7fffffff;
    }
    __syncthreads();
    const double target = thr - scan[tid];
    double margin = 0.0;
    int tok = -1;
    if (r0 < r1 && target >= 0.0 && target < tsum) {
      double run = 0.0;
      for (int i = r0; i < r1; ++i) {
        const double q = exp((double)lrow[i] / T - M) / S;
        const double r = fmax(0.0, q - C * (use_p ? (double)prow[i] : 0.0));
        if (run + r > target) {
          tok = i;
          margin = fmin(target - run, run + r - target) / Wt;
          break;
        }
        run += r;
      }
      if (tok >= 0) atomicMin(&s_hit, tok);
    }
    __syncthreads();
    if (s_hit == 0x7fffffff) {
      // rounding left the threshold past this slice: its last positive entry
      int lastpos = -1;
      for (int i = r0; i < r1; ++i) {
        const double q = exp((double)lrow[i] / T - M) / S;
        const double r = fmax(0.0, q - C * (use_p ? (double)prow[i] : 0.0));
        if (r > 0.0) lastpos = i;
      }
      __syncthreads();
      if (tid == 0) s_hit = -1;
      __syncthreads();
      if (lastpos >= 0) atomicMax(&s_hit, lastpos);
      __syncthreads();
      if (tid == 0) log_tie(a, b, v, 1, usf, 0.0);
    } else if (tok >= 0 && tok == s_hit && margin < kSampleBand) {
      log_tie(a, b, v, 1, usf, margin);
    }
    __syncthreads();
    if (tid == 0) s_out[depth] = s_hit;
    __syncthreads();
    write_outputs(a, b, depth, s_path, s_out);
    return;
  }
}

__global__ void accept_init_kernel(int* bar, int B, int32_t* tie_count) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < B) bar[i] = 0;
  if (i == 0 && tie_count) *tie_count = 0;
}

struct AcceptPlan {
  int KP = 1;
  int chunk = 0;
  bool vec = false;
  size_t ws = 0;
  size_t bar_bytes = 0;
};

AcceptPlan make_accept_plan(int B, int n_max, int V) {
  AcceptPlan p;
  p.vec = (V % 4) == 0;
  const int cus = device_cu_count();
  long kp = (2L * cus + B - 1) / B;
  const long by_v = (V + 2047) / 2048;
  if (kp > by_v) kp = by_v;
  if (kp > SPEC_MAX_NODES) kp = SPEC_MAX_NODES;
  if (const char* env = getenv("SPEC_ACCEPT_PARTS")) {
    const long e = atol(env);
    if (e >= 1 && e <= SPEC_MAX_NODES) kp = e;
  }
  if (kp < 1) kp = 1;
  int chunk = (int)((V + kp - 1) / kp);
  if (p.vec) chunk = (chunk + 3) / 4 * 4;
  p.chunk = chunk;
  p.KP = (V + chunk - 1) / chunk;
  p.bar_bytes = ((size_t)B * sizeof(int) + 255) / 256 * 256;
  p.ws = p.bar_bytes + (size_t)B * p.KP * 4 * sizeof(double);
  return p;
}

}  // namespace
}  // namespace specv

using namespace specv;

extern "C" size_t spec_accept_tree_workspace_size(int32_t B, int32_t n_max, int32_t V) {
  if (B <= 0 || n_max <= 0 || V <= 0) return 0;
  return make_accept_plan(B, n_max, V).ws;
}

extern "C" spec_status_t spec_accept_tree(
    const int32_t* tokens, const int32_t* parents, const int32_t* n_nodes, const float* draft_p,
    const float* logits, int32_t B, int32_t n_max, int32_t V, int32_t max_depth,
    float temperature, const float* u_accept, const float* u_sample, int32_t* accept_len,
    int32_t* path, int32_t* out_tokens, int32_t* n_out, float* final_dist, spec_tie_t* tie_log,
    int32_t tie_cap, int32_t* tie_count, void* workspace, size_t workspace_bytes,
    int32_t* dev_error, void* stream) {
  if (!tokens || !parents || !n_nodes || !draft_p || !logits || !u_accept || !u_sample ||
      !accept_len || !path || !out_tokens || !n_out)
    return SPEC_E_NULL;
  if (tie_log && !tie_count) return SPEC_E_NULL;
  if (B <= 0 || n_max <= 0 || n_max > SPEC_MAX_NODES || V <= 0 || max_depth < 0 ||
      max_depth >= SPEC_MAX_NODES || (tie_log && tie_cap < 0))
    return SPEC_E_SHAPE;
  if (!(temperature >= 0.f) || !isfinite(temperature)) return SPEC_E_VALUE;
  AcceptPlan p = make_accept_plan(B, n_max, V);
  if (!workspace || workspace_bytes < p.ws) return SPEC_E_WORKSPACE;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);

  AcceptArgs a;
  a.tokens = tokens; a.parents = parents; a.n_nodes = n_nodes;
  a.draft_p = draft_p; a.logits = logits;
  a.B = B; a.n_max = n_max; a.V = V; a.max_depth = max_depth;
  a.greedy = temperature == 0.f ? 1 : 0;
  a.T = (double)temperature;
  a.u_accept = u_accept; a.u_sample = u_sample;
  a.accept_len = accept_len; a.path = path; a.out_tokens = out_tokens; a.n_out = n_out;
  a.final_dist = final_dist; a.tie_log = tie_log; a.tie_cap = tie_cap; a.tie_count = tie_count;
  a.chunk = p.chunk;
  a.bar = static_cast<int*>(workspace);
  a.part = reinterpret_cast<double*>(static_cast<char*>(workspace) + p.bar_bytes);
  a.dev_error = dev_error;
  a.spin_limit = 1 << 22;

  // Cooperative launches need every workgroup resident: shrink KP to fit.
  int kp = p.KP;
  if (kp > 1) {
    int per_cu = 0;
    const void* fn = p.vec ? reinterpret_cast<const void*>(accept_kernel<true>)
                           : reinterpret_cast<const void*>(accept_kernel<false>);
    SPEC_HIP_TRY(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, NT, 0));
    const long resident = (long)per_cu * device_cu_count();
    if ((long)B * kp > resident) {
      kp = (int)(resident / B);
      if (kp < 1) kp = 1;
      int chunk = (V + kp - 1) / kp;
      if (p.vec) chunk = (chunk + 3) / 4 * 4;
      a.chunk = chunk;
      kp = (V + chunk - 1) / chunk;
    }
  }
  a.KP = kp;

  const int ib = (B + 255) / 256;
  hipLaunchKernelGGL(accept_init_kernel, dim3(ib), dim3(256), 0, strm, a.bar, B, tie_count);
  SPEC_HIP_TRY(hipGetLastError());
  const unsigned grid = (unsigned)((long)B * kp);
  if (kp == 1) {
    if (p.vec)
      hipLaunchKernelGGL(accept_kernel<true>, dim3(grid), dim3(NT), 0, strm, a);
    else
      hipLaunchKernelGGL(accept_kernel<false>, dim3(grid), dim3(NT), 0, strm, a);
    SPEC_HIP_TRY(hipGetLastError());
  } else {
    void* args[] = {&a};
    const void* fn = p.vec ? reinterpret_cast<const void*>(accept_kernel<true>)
                           : reinterpret_cast<const void*>(accept_kernel<false>);
    SPEC_HIP_TRY(hipLaunchCooperativeKernel(fn, dim3(grid), dim3(NT), args, 0, strm));
  }
  return SPEC_OK;
}
