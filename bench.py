"""Benchmark of one verify step on one MI355X.

A step is the whole hot path over one batch: spec_verify_tree_attn (one
layer), spec_accept_tree and spec_kv_commit, back to back on one stream, with
every input resident in HBM.  Between steps the committed lengths are restored
from a pristine copy (outside the timed events) so every step does the same
work; the commit's row moves leave tree K/V rows permuted, which changes
values but not the amount of work.

Prints one JSON line.  `value` is verified tree tokens per second (draft nodes
per step / mean step time); committed tokens per second are reported beside
it.  The step is timed as the three calls captured once into a HIP graph and
replayed, with HIP events only at its start and end; the per-call times
(`kernels_ms`) come from as many eagerly issued steps with events between the
calls, whose own step time is `ms_per_step_with_call_events`.  `roofline`
covers the attention kernel, the dominant one, with algorithmic bytes (what
the method must move) over its mean event-timed duration.  `configs` holds the same step timed on every other configuration
(tiny chain at T=0 and T=1, Llama-3-8B-shaped batch 1, Vicuna-13B-shaped
batch 1 at T=0 and T=1, Llama-3.3-70B-shaped batch 16), each with its
verified and committed tokens/s, per-kernel times and algorithmic rates.
`cpu_baseline` times the oracle on a bounded sample of the headline workload
on the host cores.

    python bench.py [--steps K] [--warmup W] [--config 4] [--gpus 1]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
PROFILE_PMC = os.path.join(ROOT, "profiles", "attention_pmc.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def node_depths(parents, n):
    d = np.zeros(n, np.int64)
    for j in range(1, n):
        d[j] = d[parents[j]] + 1
    return d


def attention_cost(w):
    """Algorithmic HBM bytes and flops of one tree-attention launch."""
    s = 2 if w.kv_dtype == "bf16" else 4
    n = w.n_nodes.astype(np.int64)
    L = w.prefix_len.astype(np.int64)
    bytes_ = (L.sum() * w.Hkv * w.d * 2 * s          # prefix K and V
              + n.sum() * w.Hkv * w.d * 2 * s        # tree K and V
              + n.sum() * w.Hq * w.d * s             # Q
              + n.sum() * w.Hq * w.d * 4             # fp32 output
              + 4 * n.sum() + 8 * w.B)               # parents, lengths
    keys = 0
    for b in range(w.B):
        keys += (L[b] * n[b] + (node_depths(w.parents[b], int(n[b])) + 1).sum())
    flops = 4 * w.d * w.Hq * keys
    return int(bytes_), int(flops)


def accept_bytes(w, accept_len, path):
    """Algorithmic bytes of the acceptance walk: one logits row per visited
    node, one draft row per visited node with a rejected child, tokens,
    parents and uniforms, outputs."""
    total = 0
    for b in range(w.B):
        a = int(accept_len[b])
        pb = w.parents[b, : w.n_nodes[b]]
        total += (a + 1) * w.V * 4
        if w.T > 0:
            for i in range(a + 1):
                v = int(path[b, i])
                kids = np.nonzero(pb == v)[0]
                if i < a:
                    rejected = (kids < int(path[b, i + 1])).sum()
                else:
                    rejected = len(kids)
                if rejected:
                    total += w.V * 4
        total += 16 * int(w.n_nodes[b]) + 8 * (w.max_depth + 1) + 8
    return total


def commit_bytes(w, accept_len, path):
    s = 2 if w.kv_dtype == "bf16" else 4
    total = 0
    for b in range(w.B):
        a = int(accept_len[b])
        if a > 0 and any(int(path[b, i]) != i for i in range(a + 1)):
            total += 2 * a * w.Hkv * w.d * 2 * s
        total += 8 + 4 * (a + 1)
    return total


def pmc_traffic(per_launch_algo):
    """HBM bytes per attention launch from the committed counter summary, if
    it was taken on the current attention source."""
    if not os.path.exists(PROFILE_PMC):
        return None
    with open(PROFILE_PMC) as f:
        rec = json.load(f)
    src = os.path.join(ROOT, "eagle_tree_verification_amd", "csrc", "attention.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if rec.get("attention_source_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, budget_s=12.0):
    """The oracle (as it stands) on a bounded sample of sequences of the same
    workload: attention of every node and head, the walk and the commit."""
    import oracle
    from threadpoolctl import threadpool_limits

    host_cores = os.cpu_count()
    avail = len(os.sched_getaffinity(0))
    cores = min(avail, 16)
    t0 = time.perf_counter()
    c0 = time.process_time()
    drafts = 0
    done = 0
    with threadpool_limits(limits=cores):
        for b in range(w.B):
            n = int(w.n_nodes[b])
            k, v = w.kv_f64(b)
            oracle.tree_attention(w.q_f64(b), k, v, int(w.prefix_len[b]), w.parents[b, :n],
                                  scale=w.scale)
            r = oracle.accept_tree(w.tokens[b], w.parents[b], n, w.draft_p[b], w.logits[b], w.T,
                                   w.u_accept[b], w.u_sample[b], w.max_depth, n_max=w.n_max)
            oracle.kv_commit(w.k_cache[b], w.v_cache[b], int(w.prefix_len[b]), r.path,
                             r.accept_len)
            drafts += n - 1
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
    dt = time.perf_counter() - t0
    busy = (time.process_time() - c0) / dt
    return {"value": drafts / dt, "unit": "verified tree tokens/s", "cores": cores,
            "host_cores": host_cores, "host_cores_available": avail,
            "cpu_seconds_per_second": round(busy, 2),
            "kind": "oracle",
            "sample": f"first {done} of {w.B} sequences of the same workload (all nodes and heads "
                      f"of tree attention in float64, the acceptance walk and the commit), "
                      f"{dt:.1f} s; numpy's thread pools capped at {cores} of the "
                      f"{avail} cores this process may use ({host_cores} on the host); "
                      f"{busy:.2f} CPU-seconds per second on average (the Python walk "
                      f"runs on one thread)"}


def time_steps(w, dev, steps, warmup):
    """Warm-up, then two timed phases of `steps` verify steps of workload w
    (attention, walk, commit on one stream):

    - the step: the three calls captured once as a HIP graph and replayed,
      with HIP events only at the step's start and end (eagerly issued calls
      with the same two events if capture fails);
    - the per-call breakdown: eagerly issued steps with events between the
      calls (each event in the stream adds a few microseconds to the step,
      which is why the step itself is timed without them).

    Returns the per-call times (breakdown), the step times (graph), the last
    step's walk outputs and the workspaces."""
    import torch

    from eagle_tree_verification_amd import api

    kv_dt = api.SPEC_BF16 if w.kv_dtype == "bf16" else api.SPEC_F32
    ws_attn = torch.empty(max(1, api.verify_tree_attn_workspace_size(
        w.B, w.n_max, w.Hq, w.Hkv, w.d, w.L_cap, kv_dt)), dtype=torch.uint8, device="cuda")
    ws_acc = torch.empty(api.accept_tree_workspace_size(w.B, w.n_max, w.V), dtype=torch.uint8,
                         device="cuda")
    out = torch.empty((w.B, w.n_max, w.Hq, w.d), dtype=torch.float32, device="cuda")
    outs = {"accept_len": torch.empty(w.B, dtype=torch.int32, device="cuda"),
            "path": torch.empty((w.B, w.max_depth + 1), dtype=torch.int32, device="cuda"),
            "out_tokens": torch.empty((w.B, w.max_depth + 1), dtype=torch.int32, device="cuda"),
            "n_out": torch.empty(w.B, dtype=torch.int32, device="cuda")}
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    plen0 = dev["prefix_len"].clone()

    def calls(ev=None):
        api.verify_tree_attn(dev["q"], dev["k_cache"], dev["v_cache"], dev["prefix_len"],
                             dev["n_nodes"], dev["parents"], out=out, workspace=ws_attn,
                             dev_error=err)
        if ev:
            ev[1].record()
        api.accept_tree(dev["tokens"], dev["parents"], dev["n_nodes"], dev["draft_p"],
                        dev["logits"], w.T, dev["u_accept"], dev["u_sample"], w.max_depth,
                        workspace=ws_acc, dev_error=err, outputs=outs)
        if ev:
            ev[2].record()
        api.kv_commit(dev["k_cache"], dev["v_cache"], dev["prefix_len"], outs["path"],
                      outs["accept_len"], w.max_depth, dev_error=err)

    for _ in range(warmup):
        dev["prefix_len"].copy_(plen0)
        calls()
    torch.cuda.synchronize()

    # per-call breakdown
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for k in range(steps):
        dev["prefix_len"].copy_(plen0)
        events[k][0].record()
        calls(events[k])
        events[k][3].record()
    torch.cuda.synchronize()

    # the step as a replayed graph
    graph = None
    try:
        dev["prefix_len"].copy_(plen0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            calls()
        torch.cuda.synchronize()
        graph = g
    except RuntimeError as exc:  # capture refused: time eagerly issued calls
        log(f"[bench] graph capture failed ({exc}); timing eagerly issued calls")
        torch.cuda.synchronize()
    run = graph.replay if graph is not None else calls
    for _ in range(2):
        dev["prefix_len"].copy_(plen0)
        run()
    torch.cuda.synchronize()
    step_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    t0 = time.perf_counter()
    for k in range(steps):
        dev["prefix_len"].copy_(plen0)
        step_ev[k][0].record()
        run()
        step_ev[k][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if int(err.item()) != 0:
        raise RuntimeError(f"device error bits {int(err.item())}")
    dev["prefix_len"].copy_(plen0)
    torch.cuda.synchronize()
    return {"attn": np.array([e[0].elapsed_time(e[1]) for e in events]),
            "accept": np.array([e[1].elapsed_time(e[2]) for e in events]),
            "commit": np.array([e[2].elapsed_time(e[3]) for e in events]),
            "step_with_call_events": np.array([e[0].elapsed_time(e[3]) for e in events]),
            "step": np.array([e[0].elapsed_time(e[1]) for e in step_ev]),
            "step_timing": "hip graph replay" if graph is not None else "eager calls",
            "wall": wall, "outs": outs, "plen0": plen0, "ws_attn": ws_attn, "ws_acc": ws_acc}


def step_summary(w, t):
    """Throughput, per-kernel times and algorithmic rates of timed steps."""
    ms = float(t["step"].mean())
    accept_len = t["outs"]["accept_len"].cpu().numpy()
    path = t["outs"]["path"].cpu().numpy()
    committed = int((accept_len + 1).sum())
    a_bytes, a_flops = attention_cost(w)
    acc_b = accept_bytes(w, accept_len, path)
    com_b = commit_bytes(w, accept_len, path)
    km = {k: float(t[k].mean()) for k in ("attn", "accept", "commit")}
    gbps = lambda nbytes, m: round(nbytes / (m * 1e-3) / 1e9, 1)
    return {
        "verified_tokens_per_s": round(w.verified_tokens / (ms * 1e-3), 1),
        "committed_tokens_per_s": round(committed / (ms * 1e-3), 1),
        "ms_per_step": round(ms, 4),
        "step_timing": t["step_timing"],
        "ms_per_step_with_call_events": round(float(t["step_with_call_events"].mean()), 4),
        "tokens_per_step": {"verified": int(w.verified_tokens), "committed": committed},
        "kernels_ms": {"verify_tree_attn": round(km["attn"], 4),
                       "accept_tree": round(km["accept"], 4),
                       "kv_commit": round(km["commit"], 4)},
        "algorithmic_bytes": {"verify_tree_attn": a_bytes, "accept_tree": int(acc_b),
                              "kv_commit": int(com_b)},
        "algorithmic_GBps": {"verify_tree_attn": gbps(a_bytes, km["attn"]),
                             "accept_tree": gbps(acc_b, km["accept"]),
                             "kv_commit": gbps(com_b, km["commit"]),
                             "step": gbps(a_bytes + acc_b + com_b, ms)},
        "attn_frac_hbm_peak": round(a_bytes / (km["attn"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "attn_mfma_tflops": round(a_flops / (km["attn"] * 1e-3) / 1e12, 2),
        "attn_frac_mfma_peak": round(a_flops / (km["attn"] * 1e-3) / 1e12
                                     / BF16_MFMA_PEAK_TFLOPS, 4),
        "mean_accept_len": round(float(accept_len.mean()), 3),
    }


# The configurations besides the headline one, each timed as its own step:
# (config id, temperature)
OTHER_CONFIGS = [(1, 0.0), (1, 1.0), (2, 1.0), (3, 0.0), (3, 1.0), (5, 1.0)]


def configs_bench(steps=20, warmup=3):
    """Every other configuration's step, timed like the headline one."""
    import torch

    from eagle_tree_verification_amd.workloads import CONFIGS, make_workload, to_device

    res = {}
    for cfg_id, T in OTHER_CONFIGS:
        cfg = CONFIGS[cfg_id]
        w = make_workload(cfg_id, T=T)
        dev = to_device(w)
        t = time_steps(w, dev, steps, warmup)
        rec = {"workload": f"{cfg.name}: batch {w.B}, {w.Hq} q / {w.Hkv} kv heads, head_dim "
                           f"{w.d}, {w.kv_dtype} KV, prefix {cfg.prefix[0]}-{cfg.prefix[1]}, "
                           f"{cfg.drafts}-draft depth-{cfg.depth} trees, vocab {w.V}, T={T:g}",
               "steps": steps, "warmup": warmup}
        rec.update(step_summary(w, t))
        res[f"{cfg.name}-T{T:g}"] = rec
        log(f"[bench] {cfg.name} T={T:g}: {rec['ms_per_step']} ms/step, "
            f"{rec['verified_tokens_per_s']} verified tokens/s")
        del dev, t
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return res


def commit_layers_bench(w, dev, outs, plen0, layers, reps=20):
    """The all-layer commit on this step's accepted paths, over `layers`
    caches of the workload's shape, in place and from scratch rows.  Cache
    contents are left as allocated: the commit moves bytes."""
    import torch

    from eagle_tree_verification_amd import api

    kv_t = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    s = 2 if w.kv_dtype == "bf16" else 4
    shape = (w.B, w.Hkv, w.L_cap, w.d)
    kl = [torch.empty(shape, dtype=kv_t, device="cuda") for _ in range(layers)]
    vl = [torch.empty(shape, dtype=kv_t, device="cuda") for _ in range(layers)]
    tshape = (w.B, w.Hkv, w.n_max, w.d)
    kt = [torch.empty(tshape, dtype=kv_t, device="cuda") for _ in range(layers)]
    vt = [torch.empty(tshape, dtype=kv_t, device="cuda") for _ in range(layers)]
    acc = outs["accept_len"].cpu().numpy()
    path = outs["path"].cpu().numpy()
    row = w.Hkv * w.d * s * 2 * layers                    # K and V of one cache row, all layers
    moved = sum(int(acc[b]) for b in range(w.B)
                if acc[b] > 0 and any(int(path[b, i]) != i for i in range(acc[b] + 1)))
    res = {"layers": layers}
    for form, tree in (("in_place", (None, None)), ("scratch", (kt, vt))):
        pl = plen0.clone()

        def call():
            pl.copy_(plen0)
            return api.kv_commit_layers(kl, vl, pl, outs["path"], outs["accept_len"], w.max_depth,
                                        k_tree=tree[0], v_tree=tree[1])
        call()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            pl.copy_(plen0)
            keep = api._pointer_table(kl, "k_layers"), api._pointer_table(vl, "v_layers")
            tk = (api._pointer_table(kt, "k_tree"), api._pointer_table(vt, "v_tree")) \
                if tree[0] is not None else (None, None)
            torch.cuda.synchronize()
            e0.record()
            st = api.load().spec_kv_commit_layers(
                api._ptr(keep[0]), api._ptr(keep[1]), api._ptr(tk[0]), api._ptr(tk[1]), layers,
                api._ptr(pl), api._ptr(outs["path"]), api._ptr(outs["accept_len"]), w.B,
                w.n_max if tree[0] is not None else 0, w.Hkv, w.d, w.L_cap, w.max_depth,
                api.SPEC_BF16 if w.kv_dtype == "bf16" else api.SPEC_F32, None,
                api._stream(None))
            e1.record()
            torch.cuda.synchronize()
            if st != 0:
                raise RuntimeError(f"spec_kv_commit_layers status {st}")
            ms.append(e0.elapsed_time(e1))
        t = float(np.median(ms))
        nbytes = 2 * row * (moved if form == "in_place" else int((acc + 1).sum()))
        res[form] = {"ms": round(t, 4), "algorithmic_bytes": nbytes,
                     "GBps": round(nbytes / (t * 1e-3) / 1e9, 1)}
    return res


def accept_variants_bench(w, dev, reps=20):
    """The walk's input variants at the workload's shape: per-sequence
    temperatures (seeded from {0, 0.8, 1, 1.5}), and draft rows over a
    32000-id draft vocabulary mapped into the target one (EAGLE-3's shape:
    a sorted seeded subset, rows restricted and renormalised, children
    redrawn from their parent's draft row), and the sampling filters on q
    (top-k 50, top-p 0.9, both).  Each is timed with the plain call on the
    same inputs beside it."""
    import torch

    from eagle_tree_verification_amd import api

    gen = torch.Generator(device="cuda")
    gen.manual_seed(99)
    temps = torch.tensor([0.0, 0.8, 1.0, 1.5], device="cuda")[
        torch.randint(0, 4, (w.B,), generator=gen, device="cuda")]
    Vd = min(32000, w.V)
    ids = torch.sort(torch.randperm(w.V, generator=gen, device="cuda")[:Vd]).values
    d2t = (ids - torch.arange(Vd, device="cuda")).to(torch.int32)
    pd = dev["draft_p"][:, :, ids]
    pd = (pd / pd.sum(-1, keepdim=True).clamp_min(1e-30)).contiguous()
    par = dev["parents"].long().clamp_min(0)
    rows = torch.gather(pd, 1, par[:, :, None].expand(-1, -1, Vd)).reshape(-1, Vd)
    draw = torch.multinomial(rows.nan_to_num(0.0).clamp_min(0) + 1e-30, 1, generator=gen)
    tokens = dev["tokens"].clone()
    child = torch.arange(w.n_max, device="cuda")[None, :] >= 1
    tokens = torch.where(child, ids[draw.reshape(w.B, w.n_max)].to(torch.int32), tokens)
    full = torch.zeros_like(dev["draft_p"])
    full[:, :, ids] = pd
    ws = torch.empty(api.accept_tree_ex_workspace_size(w.B, w.n_max, w.V, Vd, filters=True),
                     dtype=torch.uint8, device="cuda")
    k50 = torch.full((w.B,), 50, dtype=torch.int32, device="cuda")
    p09 = torch.full((w.B,), 0.9, dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return round(float(np.median(ms)), 4)

    def walk(draft_p, toks, **kw):
        return lambda: api.accept_tree(toks, dev["parents"], dev["n_nodes"], draft_p,
                                       dev["logits"], w.T, dev["u_accept"], dev["u_sample"],
                                       w.max_depth, workspace=ws, dev_error=err, **kw)
    res = {"draft_vocab": Vd,
           "scalar_T_ms": timed(walk(dev["draft_p"], dev["tokens"])),
           "per_seq_T_ms": timed(walk(dev["draft_p"], dev["tokens"], temperatures=temps)),
           "expanded_rows_ms": timed(walk(full, tokens)),
           "draft_vocab_ms": timed(walk(pd, tokens, d2t=d2t)),
           "top_k50_ms": timed(walk(dev["draft_p"], dev["tokens"], top_k=k50)),
           "top_p09_ms": timed(walk(dev["draft_p"], dev["tokens"], top_p=p09)),
           "top_k50_p09_ms": timed(walk(dev["draft_p"], dev["tokens"], top_k=k50, top_p=p09))}
    if int(err.item()) != 0:
        raise RuntimeError(f"walk variants device error bits {int(err.item())}")
    del full, pd, rows
    return res


def model_verify_bench(w, dev, outs, plen0, layers, ws_attn, ws_acc, reps=10):
    """One verify step of a whole `layers`-layer model's tree part: per layer,
    the tree's K/V written into that layer's cache with rotated keys
    (spec_tree_kv_write) and the rotated-query tree attention over it
    (spec_verify_tree_attn_rope); then the acceptance walk and the all-layer
    commit.  Each layer has its own seeded cache, queries and new K/V (so no
    layer finds another's data in cache).  Frequencies: base 500000 with the
    lower half of the planes slowed 8x (a rescaled schedule)."""
    import torch

    from eagle_tree_verification_amd import api

    kv_t = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    gen = torch.Generator(device="cuda")
    gen.manual_seed(777)
    shape = (w.B, w.Hkv, w.L_cap, w.d)
    kl = [torch.randn(shape, generator=gen, device="cuda").to(kv_t) for _ in range(layers)]
    vl = [torch.randn(shape, generator=gen, device="cuda").to(kv_t) for _ in range(layers)]
    ql = [torch.randn((w.B, w.n_max, w.Hq, w.d), generator=gen, device="cuda").to(kv_t)
          for _ in range(layers)]
    kn = [torch.randn((w.B, w.n_max, w.Hkv, w.d), generator=gen, device="cuda").to(kv_t)
          for _ in range(layers)]
    vn = [torch.randn((w.B, w.n_max, w.Hkv, w.d), generator=gen, device="cuda").to(kv_t)
          for _ in range(layers)]
    f = 500000.0 ** (-np.arange(w.d // 2) * 2.0 / w.d)
    f[w.d // 4:] /= 8.0
    inv_freq = torch.tensor(f, dtype=torch.float32, device="cuda")
    out = torch.empty((w.B, w.n_max, w.Hq, w.d), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pl = plen0.clone()

    def step(ev=None):
        pl.copy_(plen0)
        if ev:
            ev[0].record()
        for l in range(layers):
            api.tree_kv_write(kn[l], vn[l], kl[l], vl[l], pl, dev["n_nodes"], dev["parents"],
                              inv_freq=inv_freq, dev_error=err)
            api.verify_tree_attn(ql[l], kl[l], vl[l], pl, dev["n_nodes"], dev["parents"], out=out,
                                 workspace=ws_attn, dev_error=err, inv_freq=inv_freq)
        if ev:
            ev[1].record()
        api.accept_tree(dev["tokens"], dev["parents"], dev["n_nodes"], dev["draft_p"],
                        dev["logits"], w.T, dev["u_accept"], dev["u_sample"], w.max_depth,
                        workspace=ws_acc, dev_error=err, outputs=outs)
        if ev:
            ev[2].record()
        st = lib.spec_kv_commit_layers(
            api._ptr(ktab), api._ptr(vtab), None, None, layers, api._ptr(pl),
            api._ptr(outs["path"]), api._ptr(outs["accept_len"]), w.B, 0, w.Hkv, w.d, w.L_cap,
            w.max_depth, api.SPEC_BF16 if w.kv_dtype == "bf16" else api.SPEC_F32,
            api._ptr(err), api._stream(None))
        if st != 0:
            raise RuntimeError(f"spec_kv_commit_layers status {st}")
        if ev:
            ev[3].record()

    lib = api.load()
    ktab = api._pointer_table(kl, "k_layers")   # built once, outside the timed steps
    vtab = api._pointer_table(vl, "v_layers")
    step()
    torch.cuda.synchronize()
    rows = []
    for _ in range(reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        step(ev)
        torch.cuda.synchronize()
        rows.append([ev[0].elapsed_time(ev[3]), ev[0].elapsed_time(ev[1]),
                     ev[1].elapsed_time(ev[2]), ev[2].elapsed_time(ev[3])])
    # the two per-layer calls alone (layer 0), for the breakdown
    part = []
    for _ in range(reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record()
        api.tree_kv_write(kn[0], vn[0], kl[0], vl[0], pl, dev["n_nodes"], dev["parents"],
                          inv_freq=inv_freq, dev_error=err)
        ev[1].record()
        api.verify_tree_attn(ql[0], kl[0], vl[0], pl, dev["n_nodes"], dev["parents"], out=out,
                             workspace=ws_attn, dev_error=err, inv_freq=inv_freq)
        ev[2].record()
        torch.cuda.synchronize()
        part.append([ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2])])
    t_kvw, t_attn = (float(x) for x in np.median(np.asarray(part), axis=0))
    if int(err.item()) != 0:
        raise RuntimeError(f"model verify device error bits {int(err.item())}")
    t, t_layers, t_acc, t_com = (float(x) for x in np.median(np.asarray(rows), axis=0))
    verified = w.verified_tokens
    committed = int((outs["accept_len"].cpu().numpy() + 1).sum())
    res = {"layers": layers, "rope": "half, base 500000, lower planes / 8",
           "ms": round(t, 4), "layers_ms": round(t_layers, 4),
           "per_layer_ms": round(t_layers / layers, 4),
           "kv_write_ms": round(t_kvw, 4), "attn_rope_ms": round(t_attn, 4),
           "accept_ms": round(t_acc, 4),
           "commit_layers_ms": round(t_com, 4),
           "verified_tokens_per_s": round(verified / (t * 1e-3), 1),
           "committed_tokens_per_s": round(committed / (t * 1e-3), 1)}
    del kl, vl, ql, kn, vn, ktab, vtab
    torch.cuda.synchronize()
    return res


def tree_build_bench(B, top_k, depth, Vd, total, reps=20):
    """EAGLE-2 tree construction at the workload's batch, tree budget and
    vocabulary: `depth` calls of spec_tree_expand on seeded N(0, 3) draft
    logits (a separate buffer per level) and one spec_tree_finalize, timed
    with HIP events on the launch stream; per dtype of the draft logits."""
    import torch

    from eagle_tree_verification_amd import api

    res = {"batch": B, "top_k": top_k, "depth": depth, "draft_vocab": Vd, "drafts": total}
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    for name, tdt, s in (("bf16", torch.bfloat16, 2), ("f32", torch.float32, 4)):
        levels = [(torch.randn((B, 1 if lv == 0 else top_k, Vd), generator=gen, device="cuda")
                   * 3.0).to(tdt) for lv in range(depth)]
        state = api.tree_state(B, top_k, depth, "cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        et = torch.empty((B, top_k), dtype=torch.int32, device="cuda")
        ei = torch.empty((B, top_k), dtype=torch.int32, device="cuda")
        n_max = total + 1
        outs = {key: torch.empty((B, n_max), dtype=dt_, device="cuda")
                for key, dt_ in (("tokens", torch.int32), ("parents", torch.int32),
                                 ("depth", torch.int32), ("positions", torch.int32),
                                 ("anc_mask", torch.int64), ("draft_row", torch.int32),
                                 ("value", torch.float32))}
        outs["n_nodes"] = torch.empty(B, dtype=torch.int32, device="cuda")

        def build(ev=None):
            for lv in range(depth):
                api.tree_expand(levels[lv], state, lv + 1, top_k, depth, expanded_tokens=et,
                                expanded_ids=ei, dev_error=err)
                if ev:
                    ev[lv + 1].record()
            api.tree_finalize(state, B, top_k, depth, total, n_max, dev_error=err, outputs=outs)

        build()
        torch.cuda.synchronize()
        tot, lev = [], []
        for _ in range(reps):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(depth + 2)]
            ev[0].record()
            build(ev)
            ev[depth + 1].record()
            torch.cuda.synchronize()
            tot.append(ev[0].elapsed_time(ev[depth + 1]))
            lev.append([ev[i].elapsed_time(ev[i + 1]) for i in range(1, depth)])
        if int(err.item()) != 0:
            raise RuntimeError(f"tree construction device error bits {int(err.item())}")
        if (outs["n_nodes"] != total + 1).any():
            raise RuntimeError("tree construction emitted a short tree")
        t = float(np.median(tot))
        t_lv = float(np.median(np.asarray(lev)))             # one full level (rows = top_k)
        nbytes = B * Vd * s * (1 + (depth - 1) * top_k)       # every draft logit read once
        lv_bytes = B * top_k * Vd * s
        res[name] = {"ms": round(t, 4), "algorithmic_bytes": nbytes,
                     "GBps": round(nbytes / (t * 1e-3) / 1e9, 1),
                     "level_ms": round(t_lv, 4),
                     "level_GBps": round(lv_bytes / (t_lv * 1e-3) / 1e9, 1),
                     "level_frac_hbm_peak": round(lv_bytes / (t_lv * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        del levels, state
        torch.cuda.synchronize()
    return res


def paged_bench(w, dev, ws_attn, block_size=16, reps=20):
    """Tree attention over a paged cache: the workload's K/V scattered to a
    shuffled pool of block_size-row blocks (plus spare blocks), timed against
    the contiguous call on the same logical contents, interleaved."""
    import torch
    from eagle_tree_verification_amd import api

    if w.L_cap % block_size:
        return {"skipped": f"L_cap {w.L_cap} not a multiple of {block_size}"}
    mb = w.L_cap // block_size
    spare = 64
    gen = torch.Generator(device="cuda").manual_seed(6)
    perm = torch.randperm(w.B * mb + spare, generator=gen, device="cuda")
    table = perm[: w.B * mb].reshape(w.B, mb).to(torch.int32).contiguous()

    def to_pool(c):
        blocks = c.reshape(w.B, w.Hkv, mb, block_size, w.d).permute(0, 2, 1, 3, 4)
        pool = torch.zeros((w.B * mb + spare, w.Hkv, block_size, w.d), dtype=c.dtype, device="cuda")
        pool[table.reshape(-1).long()] = blocks.reshape(w.B * mb, w.Hkv, block_size, w.d)
        return pool

    kp, vp = to_pool(dev["k_cache"]), to_pool(dev["v_cache"])
    out_c = torch.empty((w.B, w.n_max, w.Hq, w.d), dtype=torch.float32, device="cuda")
    out_p = torch.empty_like(out_c)
    fc = lambda: api.verify_tree_attn(dev["q"], dev["k_cache"], dev["v_cache"], dev["prefix_len"],
                                      dev["n_nodes"], dev["parents"], out=out_c, workspace=ws_attn)
    fp = lambda: api.verify_tree_attn_paged(dev["q"], kp, vp, table, dev["prefix_len"],
                                            dev["n_nodes"], dev["parents"], out=out_p,
                                            workspace=ws_attn)
    fc(); fp()
    torch.cuda.synchronize()
    tc, tp = [], []
    for _ in range(reps):
        for fn, acc in ((fc, tc), (fp, tp)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            acc.append(e0.elapsed_time(e1))
    same = all(torch.equal(out_c[b, : int(w.n_nodes[b])], out_p[b, : int(w.n_nodes[b])])
               for b in range(w.B))
    res = {"block_size": block_size, "pool_blocks": int(w.B * mb + spare),
           "contiguous_attn_ms": round(float(np.median(tc)), 4),
           "paged_attn_ms": round(float(np.median(tp)), 4), "bit_identical": bool(same)}
    del kp, vp
    return res


def shard_bench(cfg_id, shards=8, reps=20):
    """One GPU's share of an 8-way tensor-parallel target, at the workload's
    batch, prefixes and trees.  Attention shards by KV head with no exchange:
    the share is Hq/8 query heads over Hkv/8 KV heads (one, here).  The walk
    shards the vocabulary: the share is a V/8 slice, walked here as a whole
    vocabulary of that size; the small per-pass exchanges between shards are
    not part of it."""
    import torch

    from eagle_tree_verification_amd import api
    from eagle_tree_verification_amd.workloads import CONFIGS, make_workload, to_device

    cfg = CONFIGS[cfg_id]

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return float(np.median(ms))

    res = {"shards": shards}
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    if cfg.kv_dtype == "bf16" and cfg.hkv % shards == 0:
        wa = make_workload(cfg_id, hq=cfg.hq // shards, hkv=cfg.hkv // shards, vocab=64)
        da = to_device(wa)
        out = torch.empty((wa.B, wa.n_max, wa.Hq, wa.d), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(1, api.verify_tree_attn_workspace_size(
            wa.B, wa.n_max, wa.Hq, wa.Hkv, wa.d, wa.L_cap, api.SPEC_BF16)) * 4,
            dtype=torch.uint8, device="cuda")
        ms = timed(lambda: api.verify_tree_attn(da["q"], da["k_cache"], da["v_cache"],
                                                da["prefix_len"], da["n_nodes"], da["parents"],
                                                out=out, workspace=ws, dev_error=err))
        nbytes, flops = attention_cost(wa)
        res["attention"] = {"hq": wa.Hq, "hkv": wa.Hkv, "ms": round(ms, 4),
                            "algorithmic_bytes": nbytes, "GBps": round(nbytes / ms / 1e6, 1),
                            "frac_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBPS, 3),
                            "mfma_tflops": round(flops / ms / 1e9, 1)}
        del da, out, ws
    Vs = -(-cfg.vocab // shards)
    wv = make_workload(cfg_id, vocab=Vs, hq=4, hkv=1)
    dv = to_device(wv)
    acc = {}

    def walk():
        acc.update(api.accept_tree(dv["tokens"], dv["parents"], dv["n_nodes"], dv["draft_p"],
                                   dv["logits"], wv.T, dv["u_accept"], dv["u_sample"],
                                   wv.max_depth, dev_error=err))
    ms = timed(walk)
    al, path = acc["accept_len"].cpu().numpy(), acc["path"].cpu().numpy()
    nbytes = accept_bytes(wv, al, path)
    res["walk"] = {"vocab": Vs, "T": wv.T, "ms": round(ms, 4), "algorithmic_bytes": int(nbytes),
                   "GBps": round(nbytes / ms / 1e6, 1), "mean_accept_len": round(float(al.mean()), 3)}
    if int(err.item()) != 0:
        raise RuntimeError(f"shard bench device error bits {int(err.item())}")
    del dv
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--commit-layers", type=int, default=32,
                    help="also time spec_kv_commit_layers over this many layers (0: skip)")
    ap.add_argument("--model-layers", type=int, default=32,
                    help="also time a whole model's verify step over this many layers, with "
                         "rotary embedding (0: skip)")
    ap.add_argument("--no-walk-variants", action="store_true",
                    help="skip timing the walk with per-sequence temperatures and a draft vocabulary")
    ap.add_argument("--no-tree-build", action="store_true",
                    help="skip timing the EAGLE-2 tree construction")
    ap.add_argument("--no-paged", action="store_true",
                    help="skip timing tree attention over a paged (block-table) cache")
    ap.add_argument("--no-shard", action="store_true",
                    help="skip timing one GPU's share of an 8-way tensor-parallel target")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing the other configurations' steps")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="run one plain device copy of this size first (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the verify path is per-sequence independent and would shard by sequence "
              "with no exchange).", file=sys.stderr)
        sys.exit(2)

    import torch

    from eagle_tree_verification_amd import api
    from eagle_tree_verification_amd.workloads import CONFIGS, make_workload, to_device

    api.load()
    cfg = CONFIGS[args.config]
    t_gen = time.perf_counter()
    w = make_workload(args.config)
    log(f"[bench] generated {cfg.name} in {time.perf_counter() - t_gen:.1f} s")
    dev = to_device(w)
    torch.cuda.synchronize()
    if args.copy_probe_mb:
        a = torch.empty(args.copy_probe_mb << 20, dtype=torch.uint8, device="cuda")
        b_ = torch.empty_like(a)
        b_.copy_(a)
        torch.cuda.synchronize()
        del a, b_

    t = time_steps(w, dev, args.steps, args.warmup)
    outs, plen0, ws_attn, ws_acc = t["outs"], t["plen0"], t["ws_attn"], t["ws_acc"]
    summ = step_summary(w, t)
    ms = summ["ms_per_step"]
    a_bytes, a_flops = attention_cost(w)
    attn_ms = float(t["attn"].mean())
    achieved = a_bytes / (attn_ms * 1e-3) / 1e9
    intensity = a_flops / a_bytes
    ridge = BF16_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    traffic = pmc_traffic(a_bytes)
    roof = {"bound": "hbm" if intensity < ridge else "mfma",
            "kernel": "attn_mfma_kernel" if (w.kv_dtype == "bf16" and w.d == 128) else "attn_valu_kernel",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": a_bytes, "flops_per_launch": a_flops,
            "mean_launch_ms": round(attn_ms, 4),
            "mfma_tflops": round(a_flops / (attn_ms * 1e-3) / 1e12, 1),
            "mfma_frac": round(a_flops / (attn_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)}
    if roof["bound"] == "mfma":
        roof.update({"achieved": roof["mfma_tflops"], "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": roof["mfma_frac"]})
    rec = {
        "metric": "verified tree tokens/s + committed tokens/s at 1 GPU; % peak HBM GB/s",
        "value": summ["verified_tokens_per_s"],
        "unit": "verified tree tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "step_timing": summ["step_timing"],
        "ms_per_step_with_call_events": summ["ms_per_step_with_call_events"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.kv_dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: batch {w.B}, {w.Hq} q / {w.Hkv} kv heads, head_dim "
                               f"{w.d}, {w.kv_dtype} KV, prefix {cfg.prefix[0]}-{cfg.prefix[1]}, "
                               f"{cfg.drafts}-draft depth-{cfg.depth} trees, vocab {w.V}, T={w.T}",
                   "global_batch": w.B, "prefix_mean": float(w.prefix_len.mean()),
                   "tree_drafts": cfg.drafts, "tree_depth": cfg.depth, "vocab": w.V,
                   "temperature": w.T, "parallelism": "single GPU"},
        "committed_tokens_per_s": summ["committed_tokens_per_s"],
        "tokens_per_step": summ["tokens_per_step"],
        "kernels_ms": summ["kernels_ms"],
        "algorithmic_GBps": summ["algorithmic_GBps"],
        "step_algorithmic_GBps": summ["algorithmic_GBps"]["step"],
        "accept_algorithmic_GBps": summ["algorithmic_GBps"]["accept_tree"],
        "mean_accept_len": summ["mean_accept_len"],
        "ms_per_step_wall_incl_length_restore": round(t["wall"] / args.steps * 1e3, 4),
        "roofline": roof,
    }
    if args.commit_layers > 0:
        rec["commit_layers"] = commit_layers_bench(w, dev, outs, plen0, args.commit_layers)
    if not args.no_walk_variants:
        rec["walk_variants"] = accept_variants_bench(w, dev)
    if args.model_layers > 0:
        rec["model_verify"] = model_verify_bench(w, dev, outs, plen0, args.model_layers, ws_attn,
                                                 ws_acc)
    if not args.no_tree_build:
        rec["tree_build"] = tree_build_bench(w.B, 10, cfg.depth, w.V, cfg.drafts)
    if not args.no_paged:
        rec["paged"] = paged_bench(w, dev, ws_attn)
    if not args.no_shard:
        rec["shard"] = shard_bench(args.config)
    if not args.no_configs:
        rec["configs"] = configs_bench()
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
