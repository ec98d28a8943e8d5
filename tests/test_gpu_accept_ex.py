"""GPU parity of spec_accept_tree_ex: per-sequence temperatures, top-k /
top-p filters on q, and a draft distribution held over an EAGLE-3 draft
vocabulary (d2t), against the oracle (oracle.accept_tree with each sequence's
temperature and filters; oracle.draft_p_to_target for the draft vocabulary).

Bars as for spec_accept_tree: accepted lengths, paths and tokens bit-exact
except a near tie the oracle confirms (at most one sequence per case, itself
checked for a valid walk); residual distributions within 1e-5.
The mapped call is also compared with the unmapped call on the explicitly
expanded draft rows: same kernel arithmetic, so every output is bit-identical.
"""
import numpy as np
import pytest
import torch

import oracle
from eagle_tree_verification_amd.workloads import make_workload, small_cases, to_device
from gpu_helpers import compare_walks, say

pytestmark = pytest.mark.gpu


def _run(api, w, dev, draft_p, *, temperatures=None, d2t=None, T=None, tokens=None, top_k=None,
         top_p=None, logits=None, launch="ordinary"):
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    res = api.accept_tree(tokens if tokens is not None else dev["tokens"], dev["parents"],
                          dev["n_nodes"], draft_p, dev["logits"] if logits is None else logits,
                          w.T if T is None else T, dev["u_accept"], dev["u_sample"], w.max_depth,
                          final_dist=True, tie_cap=4096, dev_error=err, temperatures=temperatures,
                          d2t=d2t, top_k=top_k, top_p=top_p, launch=launch)
    torch.cuda.synchronize()
    host = {k: v.cpu().numpy() for k, v in res.items() if isinstance(v, torch.Tensor) and k != "tie_log"}
    host["ties"] = api.decode_ties(res["tie_log"], res["tie_count"])
    host["dev_error"] = int(err.item())
    return host


def _compare(w, host, temps, p_rows, tokens, seqs=None, top_k=None, top_p=None, logits=None):
    """Oracle per sequence at its own temperature and filters (compare_walks);
    returns the excluded (near-tie) sequences."""
    return compare_walks(w, host, seqs=seqs, tokens=tokens, logits=logits, p_rows=p_rows,
                         temps=temps, top_k=top_k, top_p=top_p)


@pytest.mark.parametrize("name", ["c4-mini", "c2-mini", "c1-t1"])
def test_per_sequence_temperatures(hip_lib, name):
    api = hip_lib
    w = make_workload(poison=True, **small_cases()[name])
    rng = np.random.default_rng(17)
    temps = rng.choice(np.array([0.0, 0.6, 1.0, 1.7, 3.0], np.float32), size=w.B)
    if w.B >= 2:
        temps[0], temps[1] = 0.0, 1.0
    say(f"[gpu] per-sequence temperatures {name}: {temps.tolist()}")
    dev = to_device(w)
    host = _run(api, w, dev, dev["draft_p"], temperatures=torch.from_numpy(temps).to("cuda"))
    assert host["dev_error"] == 0
    excluded = _compare(w, host, temps, lambda b: w.draft_p[b], w.tokens)
    say(f"[gpu]   near-tie sequences excluded: {excluded}")
    assert len(excluded) <= max(1, w.B // 4)
    # all equal to the call's scalar: bit-identical to the scalar form
    same = _run(api, w, dev, dev["draft_p"],
                temperatures=torch.full((w.B,), w.T, dtype=torch.float32, device="cuda"))
    base = _run(api, w, dev, dev["draft_p"])
    for k in ("accept_len", "path", "out_tokens", "n_out", "final_dist"):
        np.testing.assert_array_equal(same[k], base[k], err_msg=k)


def test_bad_temperature_fails_only_its_sequence(hip_lib):
    api = hip_lib
    w = make_workload(poison=True, **small_cases()["c4-mini"])
    dev = to_device(w)
    temps = np.full(w.B, 1.0, np.float32)
    temps[2] = -0.5
    temps[3] = np.nan
    host = _run(api, w, dev, dev["draft_p"], temperatures=torch.from_numpy(temps).to("cuda"))
    assert host["dev_error"] == api.DEVERR_NONFINITE
    assert host["accept_len"][2] == -1 and host["accept_len"][3] == -1
    assert (host["path"][2] == -1).all() and host["n_out"][3] == 0
    _compare(w, host, temps, lambda b: w.draft_p[b], w.tokens, seqs=[0, 1, 4])


def _draft_vocab(w, Vd, seed):
    """A draft vocabulary of Vd target ids: d2t, draft rows restricted to it
    and renormalised, and child tokens redrawn from the parent's draft row."""
    rng = np.random.default_rng(seed)
    ids = np.sort(rng.choice(w.V, size=Vd, replace=False))
    d2t = (ids - np.arange(Vd)).astype(np.int32)
    pd = w.draft_p[:, :, ids].astype(np.float64)
    pd /= np.where(pd.sum(-1, keepdims=True) > 0, pd.sum(-1, keepdims=True), 1.0)
    pd = np.ascontiguousarray(pd, dtype=np.float32)
    tokens = w.tokens.copy()
    for b in range(w.B):
        n = int(w.n_nodes[b])
        for j in range(1, n):
            row = pd[b, w.parents[b, j]].astype(np.float64)
            cdf = np.cumsum(row)
            i = min(int(np.searchsorted(cdf, rng.random() * cdf[-1], side="right")), Vd - 1)
            tokens[b, j] = ids[i]
    return d2t, pd, tokens


@pytest.mark.parametrize("name,Vd", [("c4-mini", 1201), ("c2-mini", 1500), ("c1-t1", 250)])
def test_draft_vocabulary(hip_lib, name, Vd):
    api = hip_lib
    w = make_workload(poison=True, **small_cases()[name])
    d2t, pd, tokens = _draft_vocab(w, Vd, 23)
    say(f"[gpu] draft vocabulary {name}: V={w.V} Vd={Vd} T={w.T}")
    dev = to_device(w)
    tok_dev = torch.from_numpy(tokens).to("cuda")
    host = _run(api, w, dev, torch.from_numpy(pd).to("cuda"), d2t=torch.from_numpy(d2t).to("cuda"),
                tokens=tok_dev)
    assert host["dev_error"] == 0
    temps = np.full(w.B, w.T)
    excluded = _compare(w, host, temps, lambda b: oracle.draft_p_to_target(pd[b], d2t, w.V), tokens)
    say(f"[gpu]   near-tie sequences excluded: {excluded}")
    assert len(excluded) <= max(1, w.B // 4)
    # the unmapped call on the expanded rows: bit-identical outputs
    full = np.zeros((w.B, w.n_max, w.V), np.float32)
    full[:, :, np.arange(Vd) + d2t] = pd
    base = _run(api, w, dev, torch.from_numpy(full).to("cuda"), tokens=tok_dev)
    for k in ("accept_len", "path", "out_tokens", "n_out", "final_dist"):
        np.testing.assert_array_equal(host[k], base[k], err_msg=k)


def test_bad_draft_map_fails_every_sequence(hip_lib):
    api = hip_lib
    w = make_workload(poison=True, **small_cases()["c4-mini"])
    d2t, pd, tokens = _draft_vocab(w, 600, 5)
    d2t_dup = d2t.copy()
    d2t_dup[7] = d2t[8] + 1          # ids 7 and 8 land on one token
    dev = to_device(w)
    for bad in (d2t_dup, np.where(np.arange(600) == 599, w.V, d2t).astype(np.int32)):
        host = _run(api, w, dev, torch.from_numpy(pd).to("cuda"),
                    d2t=torch.from_numpy(bad).to("cuda"), tokens=torch.from_numpy(tokens).to("cuda"))
        assert host["dev_error"] == api.DEVERR_TOKEN
        assert (host["accept_len"] == -1).all()


@pytest.mark.timeout(900)
def test_draft_vocabulary_full_size(hip_lib):
    """The EAGLE-3 shape at the serving batch: a 32000-id draft vocabulary in
    the 128256-id target vocabulary, batch 64, per-sequence temperatures.
    Every sequence is compared with the unmapped call on expanded rows (bit
    for bit); a sample of sequences with the oracle."""
    api = hip_lib
    w = make_workload(4)
    d2t, pd, tokens = _draft_vocab(w, 32000, 31)
    temps = np.random.default_rng(2).choice(np.array([0.0, 0.8, 1.0, 1.5], np.float32), size=w.B)
    dev = to_device(w)
    tok_dev = torch.from_numpy(tokens).to("cuda")
    t_dev = torch.from_numpy(temps).to("cuda")
    host = _run(api, w, dev, torch.from_numpy(pd).to("cuda"), d2t=torch.from_numpy(d2t).to("cuda"),
                tokens=tok_dev, temperatures=t_dev)
    assert host["dev_error"] == 0
    full = torch.zeros((w.B, w.n_max, w.V), dtype=torch.float32, device="cuda")
    full[:, :, torch.from_numpy(np.arange(32000) + d2t).long().cuda()] = torch.from_numpy(pd).cuda()
    base = _run(api, w, dev, full, tokens=tok_dev, temperatures=t_dev)
    del full
    for k in ("accept_len", "path", "out_tokens", "n_out", "final_dist"):
        np.testing.assert_array_equal(host[k], base[k], err_msg=k)
    sample = sorted(np.random.default_rng(3).choice(w.B, size=6, replace=False).tolist())
    excluded = _compare(w, host, temps, lambda b: oracle.draft_p_to_target(pd[b], d2t, w.V),
                        tokens, seqs=sample)
    say(f"[gpu]   sampled {sample}; near-tie excluded {excluded}")
    assert len(excluded) <= 2


# ----------------------------------------------------------------------------
# top-k / top-p filters on q
# ----------------------------------------------------------------------------
K_CHOICES = np.array([0, 1, 2, 7, 40, 1000, -3], np.int32)
P_CHOICES = np.array([0.0, 0.3, 0.6, 0.8, 0.9, 1e-30, 1.0], np.float32)


def _filters(B, V, seed):
    rng = np.random.default_rng(seed)
    k = rng.choice(np.append(K_CHOICES, [V - 1, V, V + 5]).astype(np.int32), size=B)
    p = rng.choice(P_CHOICES, size=B)
    return k.astype(np.int32), p.astype(np.float32)


FILTER_CASES = {
    # name: (make_workload kwargs, logit rounding step or None)
    "c1-kp1": (dict(cfg=1, T=1.0), None),                                   # V 1000: one workgroup
    "c4-w1": (dict(cfg=4, batch=12, prefix=(1, 64), vocab=5003), None),     # ragged V, KP > 1
    "c4-w4": (dict(cfg=4, batch=16, prefix=(1, 64), vocab=20000), None),    # 16-byte loads, KP > 1
    "c4-ties": (dict(cfg=4, batch=16, prefix=(1, 64), vocab=20000), 0.25),  # many equal logits
    "c3-t07": (dict(cfg=3, batch=8, prefix=(1, 64), vocab=3001, T=0.7), None),
}


@pytest.mark.parametrize("name", list(FILTER_CASES))
def test_sampling_filters(hip_lib, name):
    api = hip_lib
    kw, step = FILTER_CASES[name]
    w = make_workload(poison=True, **kw)
    logits = w.logits if step is None else (np.round(w.logits / step) * step).astype(np.float32)
    k, p = _filters(w.B, w.V, 41 + w.V)
    k[0], p[0] = 2, 0.0           # top-k alone
    p[1 % w.B], k[1 % w.B] = 0.9, 0   # top-p alone
    temps = np.full(w.B, w.T, np.float32)
    say(f"[gpu] filters {name}: B={w.B} V={w.V} T={w.T} k={k.tolist()} p={p.tolist()}")
    dev = to_device(w)
    lg = torch.from_numpy(logits).to("cuda")
    host = _run(api, w, dev, dev["draft_p"], logits=lg, top_k=torch.from_numpy(k).to("cuda"),
                top_p=torch.from_numpy(p).to("cuda"))
    assert host["dev_error"] == 0
    excluded = _compare(w, host, temps, lambda b: w.draft_p[b], w.tokens, top_k=k, top_p=p,
                        logits=logits)
    say(f"[gpu]   near-tie sequences excluded: {excluded}; "
        f"top-p boundary logs {sum(int(t['kind']) == 3 for t in host['ties'])}")
    assert len(excluded) <= max(1, w.B // 4)
    # a filtered final distribution is zero outside the kept set
    for b in range(w.B):
        if b in excluded or host["accept_len"][b] < 0:
            continue
        v = int(host["path"][b, host["accept_len"][b]])
        keep, _ = oracle.filter_keep(logits[b, v], float(w.T), int(k[b]), float(p[b]))
        assert np.all(host["final_dist"][b][~keep] == 0.0), b


def test_filters_off_are_bit_identical(hip_lib):
    """k <= 0 or k >= V and p <= 0 or p >= 1 turn the filters off: outputs
    bit-identical to the unfiltered call (same kernels, threshold -inf)."""
    api = hip_lib
    w = make_workload(poison=True, cfg=4, batch=8, prefix=(1, 64), vocab=20000)
    dev = to_device(w)
    base = _run(api, w, dev, dev["draft_p"])
    k = np.array([0, -1, w.V, w.V + 9, 0, 0, -7, w.V], np.int32)
    p = np.array([0.0, 1.0, 0.0, 2.5, -0.5, 1.0, 0.0, 0.0], np.float32)
    off = _run(api, w, dev, dev["draft_p"], top_k=torch.from_numpy(k).to("cuda"),
               top_p=torch.from_numpy(p).to("cuda"))
    for key in ("accept_len", "path", "out_tokens", "n_out", "final_dist"):
        np.testing.assert_array_equal(off[key], base[key], err_msg=key)


def test_filters_at_greedy_and_with_a_nan_top_p(hip_lib):
    api = hip_lib
    w = make_workload(poison=True, cfg=4, batch=6, prefix=(1, 64), vocab=5003)
    dev = to_device(w)
    temps = np.array([0.0, 0.0, 1.0, 1.0, 0.8, 1.2], np.float32)
    k = np.array([1, 3, 5, 0, 2, 9], np.int32)
    p = np.array([0.1, 0.5, 0.7, np.nan, 0.9, 0.2], np.float32)
    host = _run(api, w, dev, dev["draft_p"], temperatures=torch.from_numpy(temps).to("cuda"),
                top_k=torch.from_numpy(k).to("cuda"), top_p=torch.from_numpy(p).to("cuda"))
    assert host["dev_error"] == api.DEVERR_NONFINITE
    assert host["accept_len"][3] == -1 and host["n_out"][3] == 0
    # greedy sequences ignore the filters: same as greedy without them
    plain = _run(api, w, dev, dev["draft_p"], temperatures=torch.from_numpy(temps).to("cuda"))
    for b in (0, 1):
        for key in ("accept_len", "path", "out_tokens"):
            np.testing.assert_array_equal(host[key][b], plain[key][b], err_msg=key)
    _compare(w, host, temps, lambda b: w.draft_p[b], w.tokens, seqs=[0, 1, 2, 4, 5], top_k=k,
             top_p=p)


def test_filters_with_a_draft_vocabulary(hip_lib):
    api = hip_lib
    w = make_workload(poison=True, cfg=4, batch=10, prefix=(1, 64), vocab=20000)
    d2t, pd, tokens = _draft_vocab(w, 6000, 77)
    k, p = _filters(w.B, w.V, 5)
    dev = to_device(w)
    host = _run(api, w, dev, torch.from_numpy(pd).to("cuda"), d2t=torch.from_numpy(d2t).to("cuda"),
                tokens=torch.from_numpy(tokens).to("cuda"), top_k=torch.from_numpy(k).to("cuda"),
                top_p=torch.from_numpy(p).to("cuda"))
    assert host["dev_error"] == 0
    excluded = _compare(w, host, np.full(w.B, w.T), lambda b: oracle.draft_p_to_target(pd[b], d2t, w.V),
                        tokens, top_k=k, top_p=p)
    assert len(excluded) <= max(1, w.B // 4)


@pytest.mark.timeout(900)
def test_filters_full_size(hip_lib):
    """Batch 64 over the 128256-token vocabulary with a per-sequence mix of
    top-k, top-p and temperature, a sample of sequences against the oracle."""
    api = hip_lib
    w = make_workload(4)
    k, p = _filters(w.B, w.V, 9)
    k[:4] = [50, 0, 1, 20]
    p[:4] = [0.0, 0.95, 0.0, 0.8]
    temps = np.random.default_rng(8).choice(np.array([0.6, 1.0, 1.3], np.float32), size=w.B)
    dev = to_device(w)
    host = _run(api, w, dev, dev["draft_p"], temperatures=torch.from_numpy(temps).to("cuda"),
                top_k=torch.from_numpy(k).to("cuda"), top_p=torch.from_numpy(p).to("cuda"))
    assert host["dev_error"] == 0
    sample = sorted(set([0, 1, 2, 3]) | set(np.random.default_rng(4).choice(w.B, size=4,
                                                                           replace=False).tolist()))
    excluded = _compare(w, host, temps, lambda b: w.draft_p[b], w.tokens, seqs=sample, top_k=k,
                        top_p=p)
    say(f"[gpu]   sampled {sample}; near-tie excluded {excluded}")
    assert len(excluded) <= 2


@pytest.mark.parametrize("name", ["c1-kp1", "c4-w1", "c4-ties", "c4-w4"])
def test_top_k_alone(hip_lib, name):
    """Top-k with top-p off, k from 1 to 1000, against the oracle on distinct
    and on heavily tied logits (the search may stop early on a bucket holding
    exactly the entries top-k needs, or run all four rounds)."""
    api = hip_lib
    kw, step = FILTER_CASES[name]
    w = make_workload(poison=True, **kw)
    logits = w.logits if step is None else (np.round(w.logits / step) * step).astype(np.float32)
    ks = np.array([1, 2, 3, 17, 50, 63, 64, 65, 200, 1000], np.int32)
    k = ks[np.arange(w.B) % len(ks)]
    say(f"[gpu] top-k alone {name}: B={w.B} V={w.V} k={k.tolist()}")
    dev = to_device(w)
    host = _run(api, w, dev, dev["draft_p"], logits=torch.from_numpy(logits).to("cuda"),
                top_k=torch.from_numpy(k).to("cuda"))
    assert host["dev_error"] == 0
    excluded = _compare(w, host, np.full(w.B, w.T, np.float32), lambda b: w.draft_p[b], w.tokens,
                        top_k=k, logits=logits)
    assert len(excluded) <= max(1, w.B // 4)
    for b in range(w.B):
        if b in excluded:
            continue
        v = int(host["path"][b, host["accept_len"][b]])
        keep, _ = oracle.filter_keep(logits[b, v], float(w.T), int(k[b]), 0.0)
        assert np.all(host["final_dist"][b][~keep] == 0.0), b


@pytest.mark.parametrize("cfg,variant", [(4, "plain"), (4, "filters"), (5, "plain"),
                                         (2, "draft-vocab")])
def test_cooperative_launch_same_bits(hip_lib, cfg, variant):
    """The cooperative launch of the walk gives the ordinary launch's outputs
    bit for bit at full size (the same kernel, only the launch differs), and
    both match the oracle."""
    api = hip_lib
    w = make_workload(cfg, T=1.0)
    dev = to_device(w)
    kw = {}
    p_rows, draft_p = (lambda b: w.draft_p[b]), dev["draft_p"]
    top_k = top_p = None
    if variant == "filters":
        rng = np.random.default_rng(91)
        top_k = rng.choice(np.array([0, 1, 20, 1000], np.int32), size=w.B)
        # (0.99 lies in the 128k vocabulary's flat tail, where token masses
        # are ~1e-7 and many boundaries fall inside the near-tie band)
        top_p = rng.choice(np.array([0.0, 0.5, 0.8, 0.9], np.float32), size=w.B)
        kw = dict(top_k=torch.from_numpy(top_k).to("cuda"), top_p=torch.from_numpy(top_p).to("cuda"))
    tokens = w.tokens
    if variant == "draft-vocab":
        d2t, pd, tokens = _draft_vocab(w, 32000, 92)
        draft_p = torch.from_numpy(pd).to("cuda")
        kw = dict(d2t=torch.from_numpy(d2t).to("cuda"), tokens=torch.from_numpy(tokens).to("cuda"))
        p_rows = lambda b: oracle.draft_p_to_target(pd[b], d2t, w.V)
    say(f"[gpu] cooperative launch {variant}: B={w.B} V={w.V} n_max={w.n_max}")
    ordinary = _run(api, w, dev, draft_p, launch="ordinary", **kw)
    coop = _run(api, w, dev, draft_p, launch="cooperative", **kw)
    assert ordinary["dev_error"] == 0 and coop["dev_error"] == 0
    for k in ("accept_len", "path", "out_tokens", "n_out", "final_dist", "tie_count"):
        np.testing.assert_array_equal(coop[k], ordinary[k], err_msg=k)
    compare_walks(w, coop, p_rows=p_rows, tokens=tokens, top_k=top_k, top_p=top_p)
