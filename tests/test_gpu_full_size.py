"""GPU parity at the five configs' full sizes, in the launch configuration the
benchmark times (the library's default plan for each shape).

Attention is compared with the oracle on every sequence and every query head,
at the root, the last node and random nodes of each tree (every node of a
small tree); every other output is checked to be finite.  The acceptance walk is compared on
every sequence (bit-exact except a near tie the oracle confirms, at most one
per case, itself checked for a valid walk) and the commit on every sequence
(bit-exact).

A second test runs 50,000 independent tiny-chain steps in one launch and
checks the Leviathan invariant on the GPU's own output: the first emitted
token of each step must be distributed as its own verifier distribution q,
and so must the second emitted token under the next q when the first draft
was accepted.  Two statistics: the randomised probability integral transform
under q must be uniform (chi-square over 20 bins), and the summed log
likelihood ratio log q(t) - log p(t) must match its exact mean and variance
under t ~ q (|z| < 4).  The first draft token itself, drawn from p, is the
negative control and must fail the second statistic by a wide margin.
"""
import numpy as np
import pytest

import oracle
from eagle_tree_verification_amd.workloads import CONFIGS, make_workload, to_device
from gpu_helpers import (compare_accept, compare_attention, compare_commit, kv_host, run_gpu_step,
                         say)

pytestmark = pytest.mark.gpu

FULL = [(1, 0.0), (1, 1.0), (2, 1.0), (3, 0.0), (3, 1.0), (4, 1.0), (5, 1.0)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg,T", FULL, ids=[f"cfg{c}-T{t:g}" for c, t in FULL])
def test_full_size_step(hip_lib, cfg, T):
    w = make_workload(cfg, T=T)
    say(f"[gpu] full size {CONFIGS[cfg].name} T={T}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} d={w.d} "
        f"L={w.prefix_len.min()}..{w.prefix_len.max()} n_max={w.n_max} V={w.V}")
    dev = to_device(w)
    host = run_gpu_step(w, dev)
    assert host["dev_error"] == 0

    attn = host["attn"]
    for b in range(w.B):
        assert np.isfinite(attn[b, : w.n_nodes[b]]).all(), b
    rng = np.random.default_rng(1000 + cfg)
    # every sequence and every query head (so every KV head and, in a large
    # batch, the longest-first order of the sequences); the root, the last
    # node and random nodes of each tree (all of a small tree; six random
    # ones at batch 1, one in a batch)
    nodes = None if w.n_max <= 8 else (6 if w.B <= 2 else 1)
    worst = compare_attention(w, attn, nodes_per_seq=nodes, rng=rng)

    excluded = compare_accept(w, host)
    say(f"[gpu]   attention max|diff|={worst:.3g} on all {w.B} sequences and {w.Hq} heads; "
        f"accepted {int(host['accept_len'].sum())} drafts; near-tie sequences excluded: {excluded}")
    compare_commit(w, host, kv_host(dev["k_cache"], w.kv_dtype),
                   kv_host(dev["v_cache"], w.kv_dtype), dev["prefix_len"].cpu().numpy())


def _pit_chi2(dists, tokens, rng, bins=20):
    """Chi-square statistic of the randomised PIT of tokens under dists."""
    u = np.empty(len(tokens))
    for i, (q, t) in enumerate(zip(dists, tokens)):
        c = np.cumsum(q)
        lo = c[t - 1] if t > 0 else 0.0
        u[i] = lo + rng.random() * q[t]
    u = np.clip(u / np.array([q.sum() for q in dists]), 0.0, np.nextafter(1.0, 0.0))
    counts = np.bincount((u * bins).astype(int), minlength=bins)
    expected = len(tokens) / bins
    return float(((counts - expected) ** 2 / expected).sum())


def _llr_z(dists, refs, tokens):
    """z-score of sum log(q(t) / r(t)) against its exact law under t ~ q."""
    total = mean = var = 0.0
    for q, r, t in zip(dists, refs, tokens):
        lr = np.log(np.maximum(q, 1e-300)) - np.log(np.maximum(r.astype(np.float64), 1e-300))
        m = float((q * lr).sum())
        total += lr[t]
        mean += m
        var += float((q * lr * lr).sum()) - m * m
    return (total - mean) / np.sqrt(var)


@pytest.mark.timeout(900)
def test_leviathan_marginals_50k_steps(hip_lib):
    B = 50_000
    w = make_workload(1, batch=B, T=1.0, seed=CONFIGS[1].seed + 77)
    say(f"[gpu] Leviathan check: {B} tiny-chain steps, V={w.V}, n={w.n_max}")
    dev = to_device(w)
    host = run_gpu_step(w, dev, final_dist=False, commit=False)
    assert host["dev_error"] == 0
    # the GPU's steps agree with the oracle's (first 500 sequences)
    compare_accept(w, host, seqs=range(500))

    rng = np.random.default_rng(20240501)
    q0 = [oracle.target_distribution(w.logits[b, 0], w.T) for b in range(B)]
    first = host["out_tokens"][:, 0]
    stat_first = _pit_chi2(q0, first, rng)
    # second emitted token of the steps that accepted the first draft
    acc = np.nonzero(host["accept_len"] >= 1)[0]
    q1 = [oracle.target_distribution(w.logits[b, 1], w.T) for b in acc]
    stat_second = _pit_chi2(q1, host["out_tokens"][acc, 1], rng)
    # negative control: the first draft token is drawn from p, not q
    stat_draft = _pit_chi2(q0, w.tokens[:, 1], rng)
    z_first = _llr_z(q0, w.draft_p[:, 0], first)
    z_second = _llr_z(q1, w.draft_p[acc, 1], host["out_tokens"][acc, 1])
    z_draft = _llr_z(q0, w.draft_p[:, 0], w.tokens[:, 1])
    crit = 43.82  # chi-square 0.999 quantile, 19 degrees of freedom
    say(f"[gpu]   PIT chi2 first={stat_first:.1f} second={stat_second:.1f} (n={len(acc)}) "
        f"draft control={stat_draft:.1f} (critical {crit}); LLR z first={z_first:.2f} "
        f"second={z_second:.2f} draft control={z_draft:.1f}")
    assert stat_first < crit and stat_second < crit
    assert abs(z_first) < 4 and abs(z_second) < 4
    assert z_draft < -20
