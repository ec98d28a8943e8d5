"""Shared driver code for the GPU parity tests: run the HIP path through the C
ABI binding and the oracle on the same seeded inputs, and compare."""
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


def compare_accept(w, host, seqs=None, fd_tol=1e-5):
    """Bit-exact tokens/lengths/paths except sequences with a near tie."""
    gpu_tie_b = set(int(t["b"]) for t in host["ties"])
    excluded = []
    for b in (range(w.B) if seqs is None else seqs):
        r = oracle_accept(w, b)
        if r.near_tie or b in gpu_tie_b:
            excluded.append(b)
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
    return excluded


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
