"""Shared driver code for the GPU parity tests: run the HIP path through the C
ABI binding and the oracle on the same seeded inputs, and compare."""
import os
import sys

import numpy as np
import torch

import oracle
from eagle_tree_verification_amd import api
from eagle_tree_verification_amd.workloads import bf16_bits_to_f32, storage_to_f64, to_device

ATOL = {"f32": 1e-5, "bf16": 2e-2}
SENTINEL = -12345.0


def say(*args):
    print(*args, file=sys.stderr, flush=True)


def run_gpu_step(w, dev, *, final_dist=True, tie_cap=4096, commit=True):
    """The three calls on one stream; returns host copies of every output."""
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.full((w.B, w.n_max, w.Hq, w.d), SENTINEL, dtype=torch.float32, device="cuda")
    api.verify_tree_attn(dev["q"], dev["k_cache"], dev["v_cache"], dev["prefix_len"],
                         dev["n_nodes"], dev["parents"], out=out, dev_error=err)
    acc = api.accept_tree(dev["tokens"], dev["parents"], dev["n_nodes"], dev["draft_p"],
                          dev["logits"], w.T, dev["u_accept"], dev["u_sample"], w.max_depth,
                          final_dist=final_dist, tie_cap=tie_cap, dev_error=err)
    res = {"attn": out, **acc}
    if commit:
        api.kv_commit(dev["k_cache"], dev["v_cache"], dev["prefix_len"], acc["path"],
                      acc["accept_len"], w.max_depth, dev_error=err)
    torch.cuda.synchronize()
    host = {}
    for k, v in res.items():
        if isinstance(v, torch.Tensor) and k not in ("tie_log",):
            host[k] = v.cpu().numpy()
    host["ties"] = api.decode_ties(acc["tie_log"], acc["tie_count"])
    host["dev_error"] = int(err.item())
    return host


def oracle_accept(w, b):
    return oracle.accept_tree(w.tokens[b], w.parents[b], w.n_nodes[b], w.draft_p[b], w.logits[b],
                              w.T, w.u_accept[b], w.u_sample[b], w.max_depth, n_max=w.n_max)


def compare_attention(w, attn, nodes_per_seq=None, heads=None, seqs=None, rng=None):
    """Element-wise comparison with the oracle on every (or a sample of) rows."""
    tol = ATOL[w.kv_dtype]
    worst = 0.0
    seqs = range(w.B) if seqs is None else seqs
    for b in seqs:
        n = int(w.n_nodes[b])
        nodes = range(n) if nodes_per_seq is None else sorted(set(
            [0, n - 1] + list(rng.choice(n, size=min(n, nodes_per_seq), replace=False))))
        hs = range(w.Hq) if heads is None else heads
        k, v = w.kv_f64(b)
        ref = oracle.tree_attention(w.q_f64(b), k, v, int(w.prefix_len[b]),
                                    w.parents[b, :n], scale=w.scale, nodes=nodes, heads=hs)
        for i in nodes:
            for h in hs:
                d = np.abs(attn[b, i, h].astype(np.float64) - ref[i, h]).max()
                worst = max(worst, d)
                assert d <= tol, (b, i, h, d)
        # rows past the tree are never written
        assert np.all(attn[b, n:] == SENTINEL)
    return worst


# Near-tie bands of the oracle by the kind a GPU tie record carries:
# 0 child test, 1 terminal sample, 2 degenerate residual, 3 top-p boundary.
TIE_BANDS = {0: oracle.TIE_BAND, 1: oracle.SAMPLE_BAND, 2: oracle.DEGENERATE_BAND,
             3: oracle.FILTER_BAND}
CONFIRM = 10.0   # a GPU tie record counts only if the oracle's margin is under 10x its band
# (test id, sequences compared, excluded sequences) of every walk comparison,
# printed in the session's terminal summary
EXCLUSIONS = []


def _oracle_margin(r, tie):
    """The oracle's margin at the decision a GPU tie record names, or None
    when the oracle made no such decision."""
    kind, node = int(tie["kind"]), int(tie["node"])
    for (v, c, k, _u, _val, margin, _acc) in r.decisions:
        if ((kind == 0 and k == "accept-test" and c == node)
                or (kind == 1 and k == "sample" and v == node)
                or (kind == 2 and k == "residual" and c == node)
                or (kind == 3 and k == "filter" and v == node)):
            return margin
    return None


def _check_valid_walk(b, host, tokens_b, parents_b, n, term_dist, fd_tol, degenerate):
    """What every walk must satisfy, whichever of several correct results a
    near tie gave: a root-to-node path down the tree, the path's tokens
    emitted, then a terminal token with positive mass under the distribution
    the walk stops in (and that distribution as final_dist)."""
    a = int(host["accept_len"][b])
    assert a >= 0 and int(host["n_out"][b]) == a + 1, (b, a, host["n_out"][b])
    path = [int(x) for x in host["path"][b]]
    out = [int(x) for x in host["out_tokens"][b]]
    assert path[0] == 0, (b, path)
    for i in range(1, a + 1):
        assert 0 < path[i] < n and int(parents_b[path[i]]) == path[i - 1], (b, path)
    assert all(x == -1 for x in path[a + 1:]) and all(x == -1 for x in out[a + 1:]), b
    assert out[:a] == [int(tokens_b[path[i]]) for i in range(1, a + 1)], (b, out, path)
    if degenerate:
        return  # the residual left at the last node is itself decided by rounding
    dist = term_dist(path[a])
    assert dist[out[a]] > 0.0, (b, out[a])
    if host.get("final_dist") is not None:
        np.testing.assert_allclose(host["final_dist"][b], dist / dist.sum(), rtol=0, atol=fd_tol)


def compare_walks(w, host, *, seqs=None, tokens=None, logits=None, p_rows=None, temps=None,
                  top_k=None, top_p=None, fd_tol=1e-5, max_excluded=1):
    """The GPU's acceptance walks against the oracle's.

    Bit-exact accepted lengths, paths, emitted tokens and error results, and
    final distributions within fd_tol, on every sequence except near ties.  A
    sequence is excluded only when the oracle flags a near tie on it, or when
    a GPU tie record names a decision whose oracle margin is under CONFIRM
    times its band; a GPU tie record the oracle does not confirm fails the
    test.  Every excluded sequence is still checked for a valid walk
    (_check_valid_walk).  At most max_excluded sequences may be excluded;
    the count is recorded for the session summary.  Returns the excluded
    sequences."""
    tokens = w.tokens if tokens is None else tokens
    logits = w.logits if logits is None else logits
    p_rows = (lambda b: w.draft_p[b]) if p_rows is None else p_rows
    seqs = range(w.B) if seqs is None else seqs
    ties = {}
    for t in host["ties"]:
        ties.setdefault(int(t["b"]), []).append(t)
    excluded = []
    compared = 0
    for b in seqs:
        compared += 1
        T = w.T if temps is None else float(temps[b])
        fk = 0 if top_k is None else int(top_k[b])
        fp = 0.0 if top_p is None else float(top_p[b])
        pr = p_rows(b)
        r = oracle.accept_tree(tokens[b], w.parents[b], w.n_nodes[b], pr, logits[b], T,
                               w.u_accept[b], w.u_sample[b], w.max_depth, n_max=w.n_max,
                               top_k=fk, top_p=fp)
        if r.error:
            assert int(host["accept_len"][b]) == -1, (b, host["accept_len"][b])
            continue
        confirmed = False
        degenerate = False
        if not r.near_tie:
            for t in ties.get(b, []):
                m = _oracle_margin(r, t)
                assert m is not None and m < CONFIRM * TIE_BANDS[int(t["kind"])], (
                    f"sequence {b}: GPU near-tie record {t} is not confirmed by the oracle "
                    f"(oracle margin {m})")
                confirmed = True
                degenerate |= int(t["kind"]) == 2
        if r.near_tie or confirmed:
            excluded.append(b)
            degenerate |= any(d[2] == "residual" and 0.0 <= d[5] < CONFIRM * oracle.DEGENERATE_BAND
                              for d in r.decisions)
            n = int(w.n_nodes[b])
            _check_valid_walk(
                b, host, tokens[b], w.parents[b], n,
                lambda v: oracle.terminal_distribution(v, tokens[b], w.parents[b], n, pr,
                                                       logits[b], T, fk, fp),
                fd_tol, degenerate)
            continue
        a = r.accept_len
        assert host["accept_len"][b] == a, (b, host["accept_len"][b], a)
        assert host["n_out"][b] == a + 1
        np.testing.assert_array_equal(host["path"][b, : a + 1], r.path)
        np.testing.assert_array_equal(host["out_tokens"][b, : a + 1], r.out_tokens)
        assert np.all(host["path"][b, a + 1:] == -1) and np.all(host["out_tokens"][b, a + 1:] == -1)
        if host.get("final_dist") is not None:
            np.testing.assert_allclose(host["final_dist"][b], r.final_dist / r.final_dist.sum(),
                                       rtol=0, atol=fd_tol)
    case = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    EXCLUSIONS.append((case, compared, list(excluded)))
    say(f"[gpu]   walks compared: {compared}; near-tie sequences excluded: {len(excluded)} "
        f"{excluded}")
    assert len(excluded) <= max_excluded, (
        f"{len(excluded)} near-tie exclusions in one case (at most {max_excluded}): {excluded}")
    return excluded


def compare_accept(w, host, seqs=None, fd_tol=1e-5, max_excluded=1):
    """compare_walks on the workload's own inputs."""
    return compare_walks(w, host, seqs=seqs, fd_tol=fd_tol, max_excluded=max_excluded)


def compare_commit(w, host, k_after, v_after, len_after, seqs=None):
    """Committed KV rows and lengths are bit-exact against the oracle."""
    for b in (range(w.B) if seqs is None else seqs):
        a = int(host["accept_len"][b])
        path = host["path"][b, : a + 1] if a >= 0 else []
        k2, v2, new_len = oracle.kv_commit(w.k_cache[b], w.v_cache[b], int(w.prefix_len[b]), path, a)
        assert len_after[b] == new_len, (b, len_after[b], new_len)
        rows = int(w.prefix_len[b]) + int(w.n_nodes[b])
        np.testing.assert_array_equal(k_after[b, :, :rows], k2[:, :rows])
        np.testing.assert_array_equal(v_after[b, :, :rows], v2[:, :rows])


def kv_host(t, kv_dtype):
    """Device cache tensor -> numpy storage array (bf16 bits or float32)."""
    if kv_dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()
