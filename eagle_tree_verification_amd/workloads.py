"""Seeded synthetic workloads for tree verification.

This module draws inputs only.  It holds none of the verification arithmetic
(no tree attention, no acceptance rule, no KV commit); both the HIP path and
the CPU oracle consume what it produces, which is the only thing they share.

Shapes follow the verify settings the pages give:
  * draft-tree budgets of 60 / 50 / 48 draft tokens for 8B / 13B / 70B
    targets, tree depth 6 (EAGLE-2) raised to 8 (EAGLE-3), ten nodes expanded
    per level -- page "EAGLE-3 完全拆解", section on how EAGLE-3 and the
    EAGLE-2 dynamic tree fit together; page "EAGLE-1/2/3 拆解", section
    "两阶段，而不是按置信度决定深度" (the two stages of EAGLE-2);
  * a chain of N drafts verified in one pass that returns N+1 distributions
    -- page "推测解码与 EAGLE-3", section "不变量：Leviathan 拒绝采样".
The pages measure on public chat/code/math suites with trained models; none of
that is available, so seeded random tensors of the same shapes stand in.

Conventions (shared with the C ABI):
  * node 0 of every tree is the pending root (the last emitted token, whose KV
    row is not yet committed); parents[b][0] = -1 and 0 <= parents[b][j] < j;
  * the tree has n_nodes[b] = drafts + 1 rows; tree node j's K/V sit in cache
    row prefix_len[b] + j;
  * draft_p[b][v] is the distribution the children of node v were drawn from;
    logits[b][v] is the verifier's next-token logits after node v.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

# Purpose streams spawned from one SeedSequence per workload.
_S_QKV, _S_LOGITS, _S_NOISE, _S_SHAPE, _S_TOKENS, _S_UACC, _S_USAMP, _S_PREFIX, _S_CALIB = range(9)


@dataclass(frozen=True)
class Config:
    name: str
    batch: int
    hq: int
    hkv: int
    head_dim: int
    prefix: tuple          # (lo, hi) inclusive range of committed prefix lengths
    drafts: int            # draft nodes per tree; the tree has drafts + 1 rows
    depth: int             # exact maximum depth of every tree
    vocab: int
    kv_dtype: str          # "f32" or "bf16"
    logit_std: float       # verifier logits ~ N(0, logit_std)
    alpha: Optional[tuple]  # per-sequence target acceptance rate range, or None
    noise_std: Optional[float]  # literal draft-logit noise when alpha is None
    temperatures: tuple
    chain: bool
    seed: int


CONFIGS = {
    1: Config("tiny-chain", 1, 4, 4, 16, (32, 32), 5, 5, 1000, "f32", 2.0,
              None, 0.5, (0.0, 1.0), True, 1001),
    2: Config("llama3-8b-b1", 1, 32, 8, 128, (2048, 2048), 60, 6, 128256, "bf16", 3.0,
              (0.8, 0.8), None, (1.0,), False, 1002),
    3: Config("vicuna-13b-b1", 1, 40, 40, 128, (4096, 4096), 50, 8, 32000, "bf16", 3.0,
              (0.9, 0.9), None, (0.0, 1.0), False, 1003),
    4: Config("serving-b64", 64, 32, 8, 128, (512, 4096), 60, 8, 128256, "bf16", 3.0,
              (0.6, 0.95), None, (1.0,), False, 1004),
    5: Config("llama3.3-70b-b16", 16, 64, 8, 128, (8192, 8192), 48, 8, 128256, "bf16", 3.0,
              (0.8, 0.8), None, (1.0,), False, 1005),
}


# ----------------------------------------------------------------------------
# bf16 storage helpers (data conversion only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite values cannot wrap in uint32 (largest: 0xFF7FFFFF + 0x8000); NaNs are patched below
    r = ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def storage_to_f64(a: np.ndarray, kv_dtype: str) -> np.ndarray:
    """Exact float64 value of stored K/V/Q elements."""
    if kv_dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def _to_storage(x32: np.ndarray, kv_dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if kv_dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


# ----------------------------------------------------------------------------
# Workload container
# ----------------------------------------------------------------------------
@dataclass
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    L_cap: int
    n_max: int
    V: int
    max_depth: int
    T: float
    kv_dtype: str
    q: np.ndarray            # [B][n_max][Hq][d]  storage (f32 or bf16 bits)
    k_cache: np.ndarray      # [B][Hkv][L_cap][d] storage
    v_cache: np.ndarray      # [B][Hkv][L_cap][d] storage
    prefix_len: np.ndarray   # int32 [B]
    n_nodes: np.ndarray      # int32 [B]
    parents: np.ndarray      # int32 [B][n_max], -1 padded
    tokens: np.ndarray       # int32 [B][n_max]; node 0 holds the root token
    logits: np.ndarray       # float32 [B][n_max][V]
    draft_p: np.ndarray      # float32 [B][n_max][V]
    u_accept: np.ndarray     # float32 [B][n_max] in [0,1)
    u_sample: np.ndarray     # float32 [B][n_max] in [0,1)
    alpha_target: np.ndarray  # float64 [B] (nan when literal noise was used)
    noise_std: np.ndarray    # float64 [B]

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    @property
    def verified_tokens(self) -> int:
        """Draft nodes verified per step (tree rows minus the roots)."""
        return int((self.n_nodes - 1).sum())

    def q_f64(self, b: int) -> np.ndarray:
        return storage_to_f64(self.q[b, : self.n_nodes[b]], self.kv_dtype)

    def kv_f64(self, b: int):
        rows = int(self.prefix_len[b] + self.n_nodes[b])
        return (storage_to_f64(self.k_cache[b, :, :rows], self.kv_dtype),
                storage_to_f64(self.v_cache[b, :, :rows], self.kv_dtype))


# ----------------------------------------------------------------------------
# Tree shapes
# ----------------------------------------------------------------------------
def tree_shape(drafts: int, depth: int, rng: np.random.Generator,
               max_children: int = 10, max_expand: int = 10) -> np.ndarray:
    """Parents of a random draft tree with exactly `depth` levels below the root.

    Level sizes are grown from one node per level by adding nodes to levels
    chosen at random with weight falling with depth, within the capacity that
    `max_expand` expanded parents with at most `max_children` children each
    allow.  At each level up to `max_expand` nodes of the previous level are
    expanded (chosen at random, weighted to lower ids, i.e. the higher-valued
    candidates) and the level's nodes are dealt among them.  Ids are assigned
    level by level, then by parent, then by rank, so parents[j] < j.
    """
    if depth < 1 or drafts < depth:
        raise ValueError("need drafts >= depth >= 1")
    sizes = [1] * depth
    remaining = drafts - depth

    def cap(lv):
        prev = 1 if lv == 0 else sizes[lv - 1]
        return max_children * min(max_expand, prev)

    w_level = 0.75 ** np.arange(depth)
    while remaining > 0:
        ok = np.array([sizes[lv] < cap(lv) for lv in range(depth)])
        if not ok.any():
            raise ValueError("tree budget exceeds the expansion capacity")
        w = np.where(ok, w_level, 0.0)
        lv = int(rng.choice(depth, p=w / w.sum()))
        sizes[lv] += 1
        remaining -= 1

    parents = [-1]
    prev_ids = [0]
    next_id = 1
    for lv in range(depth):
        k = min(max_expand, len(prev_ids), sizes[lv])
        wr = 1.0 / (1.0 + np.arange(len(prev_ids)))
        chosen = np.sort(rng.choice(len(prev_ids), size=k, replace=False, p=wr / wr.sum()))
        counts = np.ones(k, dtype=np.int64)
        extra = sizes[lv] - k
        wc = 1.0 / (1.0 + np.arange(k))
        while extra > 0:
            okc = counts < max_children
            ww = np.where(okc, wc, 0.0)
            i = int(rng.choice(k, p=ww / ww.sum()))
            counts[i] += 1
            extra -= 1
        level_ids = []
        for ci, c in zip(chosen, counts):
            for _ in range(int(c)):
                parents.append(prev_ids[ci])
                level_ids.append(next_id)
                next_id += 1
        prev_ids = level_ids
    return np.asarray(parents, dtype=np.int32)


def chain_parents(drafts: int) -> np.ndarray:
    return np.arange(-1, drafts, dtype=np.int32)


def node_depths(parents: np.ndarray) -> np.ndarray:
    dep = np.zeros(len(parents), dtype=np.int32)
    for j in range(1, len(parents)):
        dep[j] = dep[parents[j]] + 1
    return dep


# ----------------------------------------------------------------------------
# Draft distributions (input synthesis only)
# ----------------------------------------------------------------------------
def _softmax_rows64(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    x = x - x.max(axis=-1, keepdims=True)
    e = np.exp(x)
    return e / e.sum(axis=-1, keepdims=True)


def _overlap(p: np.ndarray, q: np.ndarray) -> float:
    return float(np.minimum(p, q).sum(axis=-1).mean())


def calibrate_noise(targets: Sequence[float], vocab: int, logit_std: float,
                    rng: np.random.Generator, rows: int = 16) -> np.ndarray:
    """Draft-logit noise std giving mean overlap sum_x min(p(x), q(x)) = target.

    The overlap is the per-token acceptance rate of the rejection rule at T=1
    (page "推测解码与 EAGLE-3", key-terms table entry on the acceptance rate).
    Measured on `rows` calibration rows over a grid of noise levels and
    inverted by interpolation (the overlap falls monotonically with noise).
    """
    l = rng.normal(0.0, logit_std, size=(rows, vocab))
    z = rng.standard_normal(size=(rows, vocab))
    q = _softmax_rows64(l)
    grid = np.concatenate([np.linspace(0.0, 0.5, 21)[:-1], np.linspace(0.5, 3.0, 26)])
    alphas = np.array([_overlap(_softmax_rows64(l + s * z), q) for s in grid])
    alphas = np.minimum.accumulate(alphas)  # enforce monotone for interp
    t = np.clip(np.asarray(targets, dtype=np.float64), alphas[-1], 1.0)
    return np.interp(-t, -alphas, grid)


# ----------------------------------------------------------------------------
# Main generator
# ----------------------------------------------------------------------------
def make_workload(cfg, *, T: Optional[float] = None, token_mode: Optional[str] = None,
                  batch: Optional[int] = None, prefix: Optional[tuple] = None,
                  vocab: Optional[int] = None, drafts=None, depth: Optional[int] = None,
                  hq: Optional[int] = None, hkv: Optional[int] = None,
                  head_dim: Optional[int] = None, kv_dtype: Optional[str] = None,
                  parents: Optional[Sequence[np.ndarray]] = None,
                  seed: Optional[int] = None, poison: bool = False,
                  l_cap: Optional[int] = None,
                  prefix_lens: Optional[Sequence[int]] = None,
                  threads: Optional[int] = None) -> Workload:
    """Draw one workload from a named config with optional overrides.

    drafts: int, or a per-sequence list for ragged trees.
    token_mode: "iid" draws each child token from its parent's draft
      distribution (siblings independent); "topk" gives the children of a node
      the distinct highest-probability tokens of its draft distribution.
      Default: "topk" at T == 0, else "iid".
    poison: fill every element the path must never read (cache rows past the
      tree, logits/p/q rows past n_nodes) with NaN.
    prefix_lens: explicit per-sequence prefix lengths (within `prefix`'s hi).
    """
    if isinstance(cfg, int):
        cfg = CONFIGS[cfg]
    over = {}
    for k, v in dict(batch=batch, prefix=prefix, vocab=vocab, depth=depth, hq=hq, hkv=hkv,
                     head_dim=head_dim, kv_dtype=kv_dtype, seed=seed).items():
        if v is not None:
            over[k] = v
    if drafts is not None and np.isscalar(drafts):
        over["drafts"] = int(drafts)
    cfg = dataclasses.replace(cfg, **over)
    if T is None:
        T = cfg.temperatures[-1]
    if token_mode is None:
        token_mode = "topk" if T == 0 else "iid"
    B, V = cfg.batch, cfg.vocab
    if drafts is not None and not np.isscalar(drafts):
        drafts_b = np.asarray(drafts, dtype=np.int64)
        assert drafts_b.shape == (B,)
    else:
        drafts_b = np.full(B, cfg.drafts, dtype=np.int64)
    if parents is not None:
        drafts_b = np.array([len(p) - 1 for p in parents], dtype=np.int64)
    n_max = int(drafts_b.max()) + 1

    ss = np.random.SeedSequence(cfg.seed)
    subs = ss.spawn(9)
    rngs = [np.random.Generator(np.random.Philox(s)) for s in subs]

    # prefix lengths
    lo, hi = cfg.prefix
    if prefix_lens is not None:
        prefix_len = np.asarray(prefix_lens, dtype=np.int32)
        assert prefix_len.shape == (B,) and prefix_len.max() <= hi
    elif lo == hi:
        prefix_len = np.full(B, lo, dtype=np.int32)
    else:
        prefix_len = rngs[_S_PREFIX].integers(lo, hi, endpoint=True, size=B).astype(np.int32)
    L_cap = l_cap if l_cap is not None else int(-(-(hi + n_max) // 64) * 64)

    # tree shapes
    par = np.full((B, n_max), -1, dtype=np.int32)
    n_nodes = (drafts_b + 1).astype(np.int32)
    for b in range(B):
        if parents is not None:
            pb = np.asarray(parents[b], dtype=np.int32)
        elif drafts_b[b] == 0:
            pb = np.array([-1], dtype=np.int32)
        elif cfg.chain:
            pb = chain_parents(int(drafts_b[b]))
        else:
            dep = min(cfg.depth, int(drafts_b[b]))
            pb = tree_shape(int(drafts_b[b]), dep, rngs[_S_SHAPE])
        par[b, : len(pb)] = pb
    max_depth = int(max(node_depths(par[b, : n_nodes[b]]).max() for b in range(B)))
    max_depth = max(max_depth, 1)

    # per-sequence data, each sequence from its own child streams
    d, Hq, Hkv = cfg.head_dim, cfg.hq, cfg.hkv
    dt = cfg.kv_dtype
    fill = np.float32(np.nan) if poison else np.float32(0.0)
    fill_st = _to_storage(np.array([fill], np.float32), dt)[0]
    sdt = np.uint16 if dt == "bf16" else np.float32
    q = np.empty((B, n_max, Hq, d), dtype=sdt)
    k_cache = np.empty((B, Hkv, L_cap, d), dtype=sdt)
    v_cache = np.empty((B, Hkv, L_cap, d), dtype=sdt)
    logits = np.empty((B, n_max, V), dtype=np.float32)
    draft_p = np.empty((B, n_max, V), dtype=np.float32)
    tokens = np.full((B, n_max), -1, dtype=np.int32)

    rn = rngs[_S_NOISE]
    if cfg.alpha is not None:
        a_lo, a_hi = cfg.alpha
        alpha_t = (np.full(B, a_lo) if a_lo == a_hi else rn.uniform(a_lo, a_hi, size=B))
        uniq, inv = np.unique(alpha_t, return_inverse=True)
        sig_u = calibrate_noise(uniq, V, cfg.logit_std, rngs[_S_CALIB])
        noise = sig_u[inv]
    else:
        alpha_t = np.full(B, np.nan)
        noise = np.full(B, cfg.noise_std)
    root_tok = rngs[_S_TOKENS].integers(V, size=B)
    kids_ss = [subs[_S].spawn(B) for _S in (_S_QKV, _S_LOGITS, _S_NOISE, _S_TOKENS)]

    def one(b):
        rq, rl, rn_b, rt = (np.random.Generator(np.random.Philox(k[b])) for k in kids_ss)
        nb = int(n_nodes[b])
        rows = int(prefix_len[b] + nb)
        qb = np.full((n_max, Hq, d), fill, dtype=np.float32)
        qb[:nb] = rq.standard_normal(size=(nb, Hq, d), dtype=np.float32)
        q[b] = _to_storage(qb, dt)
        for cache in (k_cache, v_cache):
            cache[b, :, :rows] = _to_storage(
                rq.standard_normal(size=(Hkv, rows, d), dtype=np.float32), dt)
            cache[b, :, rows:] = fill_st
        lb = rl.standard_normal(size=(nb, V), dtype=np.float32) * np.float32(cfg.logit_std)
        eps = rn_b.standard_normal(size=(nb, V), dtype=np.float32)
        x = lb + np.float32(noise[b]) * eps
        x -= x.max(axis=-1, keepdims=True)
        np.exp(x, out=x)
        x /= x.sum(axis=-1, keepdims=True, dtype=np.float64).astype(np.float32)
        logits[b, :nb] = lb
        draft_p[b, :nb] = x
        logits[b, nb:] = fill
        draft_p[b, nb:] = fill
        pb = par[b, :nb]
        tokens[b, 0] = root_tok[b]
        for v in range(nb):
            kids = np.nonzero(pb == v)[0]
            if len(kids) == 0:
                continue
            prow = draft_p[b, v].astype(np.float64)
            if token_mode == "topk":
                order = np.argsort(-prow, kind="stable")
                tokens[b, kids] = order[: len(kids)]
            elif token_mode == "iid":
                cdf = np.cumsum(prow)
                u = rt.random(size=len(kids)) * cdf[-1]
                tokens[b, kids] = np.minimum(np.searchsorted(cdf, u, side="right"), V - 1)
            else:
                raise ValueError(token_mode)

    workers = max(1, min(B, threads or len(os.sched_getaffinity(0)), 16))
    if workers == 1:
        for b in range(B):
            one(b)
    else:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(one, range(B)))

    u_accept = rngs[_S_UACC].random(size=(B, n_max), dtype=np.float32)
    u_sample = rngs[_S_USAMP].random(size=(B, n_max), dtype=np.float32)

    return Workload(name=cfg.name, B=B, Hq=Hq, Hkv=Hkv, d=d, L_cap=L_cap, n_max=n_max, V=V,
                    max_depth=max_depth, T=float(T), kv_dtype=dt, q=q, k_cache=k_cache,
                    v_cache=v_cache, prefix_len=prefix_len, n_nodes=n_nodes, parents=par,
                    tokens=tokens, logits=logits, draft_p=draft_p, u_accept=u_accept,
                    u_sample=u_sample, alpha_target=alpha_t.astype(np.float64),
                    noise_std=noise.astype(np.float64))


def small_cases():
    """Reduced shapes of the five configs that the oracle finishes in seconds.

    Each keeps its config's head layout, head dim and dtype and still spans
    several KV tiles with a ragged tail.
    """
    return {
        "c1-t0": dict(cfg=1, T=0.0),
        "c1-t1": dict(cfg=1, T=1.0),
        "c2-mini": dict(cfg=2, prefix=(333, 333), vocab=6007),
        "c3-mini-t0": dict(cfg=3, prefix=(517, 517), vocab=3001, T=0.0),
        "c3-mini-t1": dict(cfg=3, prefix=(517, 517), vocab=3001, T=1.0),
        "c4-mini": dict(cfg=4, batch=5, prefix=(1, 700), vocab=5003),
        "c5-mini": dict(cfg=5, batch=2, prefix=(190, 190), vocab=4099),
    }


@dataclass
class TreeInputs:
    """Draft outputs for building trees level by level (inputs only).

    levels[l] holds the draft logits of level l + 1: [B][1][Vd] for the root
    row, [B][top_k][Vd] afterwards (row r standing for the r-th node expanded
    at the level before).  `store[l]` is the same in storage form (float32, or
    bf16 bits as uint16); `levels[l]` is its exact float32 value.
    """
    B: int
    top_k: int
    depth: int
    Vd: int
    total_tokens: int
    dtype: str
    levels: list
    store: list
    d2t: Optional[np.ndarray]
    root_token: np.ndarray
    prefix_len: np.ndarray


def make_tree_inputs(B, top_k, depth, Vd, total_tokens, *, dtype="f32", seed=0,
                     logit_std=3.0, target_vocab=None, threads=None):
    """Seeded draft logits ~ N(0, logit_std) for a tree of `depth` levels.

    target_vocab: if given, d2t maps the Vd draft ids onto a sorted random
    subset of range(target_vocab) (draft id i -> token i + d2t[i]), the shape
    of an EAGLE-3 head with its own smaller vocabulary (page "EAGLE-1/2/3
    拆解", section "代码里能直接读到的三处改动": 32000 draft ids into 128256).
    """
    ss = np.random.SeedSequence([2000, seed])
    kids = ss.spawn(depth + 1)
    aux = np.random.Generator(np.random.Philox(kids[depth]))

    def one(lv):
        rg = np.random.Generator(np.random.Philox(kids[lv]))
        R = 1 if lv == 0 else top_k
        x = rg.standard_normal(size=(B, R, Vd), dtype=np.float32) * np.float32(logit_std)
        st = _to_storage(x, dtype)
        val = bf16_bits_to_f32(st) if dtype == "bf16" else st
        return val, st

    workers = max(1, min(depth, threads or len(os.sched_getaffinity(0)), 16))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        out = list(ex.map(one, range(depth)))
    d2t = None
    if target_vocab is not None:
        ids = np.sort(aux.choice(int(target_vocab), size=Vd, replace=False))
        d2t = (ids - np.arange(Vd)).astype(np.int32)
    root = aux.integers(0, target_vocab or Vd, size=B).astype(np.int32)
    prefix = aux.integers(0, 4096, size=B).astype(np.int32)
    return TreeInputs(B=B, top_k=top_k, depth=depth, Vd=Vd, total_tokens=total_tokens,
                      dtype=dtype, levels=[o[0] for o in out], store=[o[1] for o in out],
                      d2t=d2t, root_token=root, prefix_len=prefix)


def to_device(w: Workload, device="cuda"):
    """Copy a workload's arrays into device tensors (dict keyed like the fields)."""
    import torch

    def kv(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if w.kv_dtype == "bf16":
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.to(device)

    def plain(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    return {
        "q": kv(w.q), "k_cache": kv(w.k_cache), "v_cache": kv(w.v_cache),
        "prefix_len": plain(w.prefix_len), "n_nodes": plain(w.n_nodes),
        "parents": plain(w.parents), "tokens": plain(w.tokens), "logits": plain(w.logits),
        "draft_p": plain(w.draft_p), "u_accept": plain(w.u_accept), "u_sample": plain(w.u_sample),
    }
