"""Pins for the oracle's EAGLE-2 tree construction (CPU only).

Fixed by page "EAGLE-1/2/3 拆解", sections "一个可核对的经验性质" (value =
product of draft confidences along the root path) and "两阶段" (expand the
top-k nodes of each level, then take the global top N of all nodes):
  * a tree worked out by hand (tests/golden/tree_build_small.json);
  * a brute-force restatement over the complete draft tree of a tiny
    vocabulary, with values as products of probabilities and every level's
    expansion and the final choice checked from their definitions;
  * top_k = 1, which is greedy decoding of the draft;
  * structural invariants on random trees of the papers' sizes.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from oracle import tree as otree

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "tree_build_small.json")) as f:
        return json.load(f)


def _grow(g, d2t=None):
    tb = otree.TreeBuilder(g["top_k"], d2t)
    for rows in g["levels"]:
        tb.expand(np.log(np.asarray(rows, dtype=np.float64)))
    return tb


def test_golden_pool_and_expansion():
    g = _golden()
    tb = _grow(g)
    pool = g["pool"]
    assert [e["draft_id"] for e in tb.pool] == pool["draft_id"]
    assert [e["parent"] for e in tb.pool] == pool["parent"]
    np.testing.assert_allclose([np.exp(e["value"]) for e in tb.pool], pool["prob"],
                               rtol=1e-12)
    assert tb.expanded == g["expanded"]


@pytest.mark.parametrize("case", range(4))
def test_golden_rerank(case):
    g = _golden()
    c = g["cases"][case]
    tb = _grow(g, c["d2t"])
    res = tb.finalize(c["total_tokens"], g["root_token"], g["prefix_len"])
    assert res["pool_ids"] == c["pool_ids"]
    for key in ("tokens", "parents", "depth", "positions", "draft_row", "anc_mask"):
        assert res[key] == c[key], key
    assert res["n_nodes"] == len(c["tokens"])
    np.testing.assert_allclose(np.exp(res["value"]), c["prob"], rtol=1e-12)


# ---- brute force over the complete draft tree -------------------------------

def _draft_fn(seed, vd, spread):
    """A synthetic draft model: the probabilities at a node are a seeded
    function of its root path (a tuple of draft ids)."""
    cache = {}

    def f(path):
        if path not in cache:
            h = abs(hash((seed,) + path)) % (2 ** 32)
            rng = np.random.default_rng([seed, h])
            cache[path] = rng.normal(0.0, spread, size=vd)
        return cache[path]
    return f


def _probs(z):
    e = np.exp(np.asarray(z, dtype=np.float64))
    return e / e.sum()


def _pool_path(tb, pid):
    path = []
    while pid != -1:
        path.append(tb.pool[pid]["draft_id"])
        pid = tb.pool[pid]["parent"]
    return tuple(reversed(path))


def _drive(f, k, depth, total):
    """Run the oracle the way a draft model would: each level's rows are the
    draft's outputs at the previous level's expanded nodes, in their order."""
    tb = otree.TreeBuilder(k)
    tb.expand(f(()))
    for _ in range(depth - 1):
        tb.expand(np.stack([f(_pool_path(tb, p)) for p in tb.expanded[-1]]))
    return tb, tb.finalize(total, root_token=0)


def _brute(f, vd, k, depth, total):
    """Definition-level restatement: value(path) = product of probabilities
    along the path; level l's pool = the k most probable children of each of
    the k best pool nodes of level l-1 (level 1: of the root); the result =
    the `total` best nodes of the pool."""
    value = {(): 1.0}
    level_nodes = [()]
    pool = []
    for lv in range(1, depth + 1):
        cand = []
        for par in level_nodes:
            p = _probs(f(par))
            best = sorted(range(vd), key=lambda i: -p[i])[:k]
            for i in best:
                value[par + (i,)] = value[par] * p[i]
                cand.append(par + (i,))
        pool += cand
        level_nodes = sorted(cand, key=lambda q: -value[q])[:k]
    chosen = set(sorted(pool, key=lambda q: -value[q])[:total])
    return value, pool, chosen


@pytest.mark.parametrize("seed,vd,k,depth,total", [
    (1, 5, 2, 3, 5), (2, 6, 3, 3, 9), (3, 4, 2, 4, 7), (4, 7, 3, 4, 14),
    (5, 5, 1, 4, 4), (6, 8, 4, 3, 20), (7, 6, 2, 5, 9), (8, 5, 5, 2, 30)])
def test_brute_force_small(seed, vd, k, depth, total):
    f = _draft_fn(seed, vd, 1.5)
    tb, res = _drive(f, k, depth, total)
    value, pool, chosen = _brute(f, vd, k, depth, total)
    # the pool is the same set of root paths, with product values
    got_pool = {_pool_path(tb, p): np.exp(tb.pool[p]["value"]) for p in range(len(tb.pool))}
    assert set(got_pool) == set(pool)
    for q, v in got_pool.items():
        assert v == pytest.approx(value[q], rel=1e-12)
    # the emitted drafts are the chosen paths, each once, parents first
    paths = [()]
    for j in range(1, res["n_nodes"]):
        paths.append(paths[res["parents"][j]] + (res["tokens"][j],))
    assert set(paths[1:]) == chosen and len(paths) == len(chosen) + 1
    # a sanity margin so that float ordering is not what decides
    vals = sorted(value[q] for q in pool)
    assert min(b - a for a, b in zip(vals, vals[1:])) > 1e-12


@pytest.mark.parametrize("seed", range(4))
def test_top1_is_greedy_decoding(seed):
    vd, depth = 50, 6
    f = _draft_fn(100 + seed, vd, 2.0)
    tb, res = _drive(f, 1, depth, depth)
    path, logv = (), 0.0
    for _ in range(depth):
        p = _probs(f(path))
        i = int(np.argmax(p))
        path, logv = path + (i,), logv + np.log(p[i])
    assert res["n_nodes"] == depth + 1
    assert res["parents"] == [-1] + list(range(depth))
    assert tuple(res["tokens"][1:]) == path
    assert res["value"][-1] == pytest.approx(logv, rel=1e-12)


@pytest.mark.parametrize("seed,k,depth,total", [(0, 10, 6, 60), (1, 10, 8, 60),
                                                (2, 8, 5, 62), (3, 10, 8, 48)])
def test_structure_at_paper_sizes(seed, k, depth, total):
    rng = np.random.default_rng(seed)
    vd = 300
    levels = [rng.normal(0, 3, size=(1, vd))]
    levels += [rng.normal(0, 3, size=(k, vd)) for _ in range(depth - 1)]
    res, err, tb = otree.build_tree(levels, k, total, root_token=5, prefix_len=17)
    assert err == 0
    n = res["n_nodes"]
    assert n == total + 1
    assert len(tb.pool) == k + (depth - 1) * k * k
    ok, dep = oracle.validate_tree(np.asarray(res["parents"]), n, 64, depth)
    assert ok and list(dep) == res["depth"]
    assert res["positions"] == [17 + d for d in res["depth"]]
    chosen = set(res["pool_ids"])
    thr = min(tb.pool[p]["value"] for p in chosen)
    assert all(tb.pool[p]["value"] <= thr for p in range(len(tb.pool)) if p not in chosen)
    for j in range(1, n):
        assert res["value"][j] <= res["value"][res["parents"][j]]
        m = res["anc_mask"][j]
        anc = {i for i in range(n) if m >> i & 1}
        walk, x = set(), j
        while x != -1:
            walk.add(x)
            x = res["parents"][x]
        assert anc == walk
    # every expanded set is the top of its own level
    for lv, ids in enumerate(tb.expanded):
        level_ids = [p for p in range(len(tb.pool)) if tb.pool[p]["depth"] == lv + 1]
        cut = min(tb.pool[p]["value"] for p in ids)
        assert all(tb.pool[p]["value"] <= cut for p in level_ids if p not in ids)
        assert len(ids) == min(k, len(level_ids))


def test_invalid_rows_and_zero_probability_nodes():
    k, vd = 3, 8
    good = np.zeros((1, vd))
    bad = good.copy()
    bad[0, 4] = np.nan
    assert otree.build_tree([bad], k, 5)[1] == oracle.ERR_NONFINITE
    inf = good.copy()
    inf[0, 2] = np.inf
    assert otree.build_tree([inf], k, 5)[0] is None
    assert otree.build_tree([np.full((1, vd), -np.inf)], k, 5)[0] is None
    # a later level failing fails the sequence
    assert otree.build_tree([good, np.vstack([good, good, bad])], k, 5)[0] is None
    # -inf entries are allowed; a child of probability 0 is never emitted
    z = np.full((1, vd), -np.inf)
    z[0, 6] = 1.0
    z[0, 1] = 0.0
    res, err, tb = otree.build_tree([z], k, 5)
    assert err == 0 and res["n_nodes"] == 3 and res["tokens"][1:] == [6, 1]
    assert len(tb.pool) == 3 and tb.pool[2]["value"] == -np.inf


def test_d2t_maps_tokens_only():
    rng = np.random.default_rng(9)
    vd, k = 40, 4
    levels = [rng.normal(size=(1, vd))] + [rng.normal(size=(k, vd)) for _ in range(3)]
    d2t = rng.integers(0, 1000, size=vd)
    a, _, _ = otree.build_tree(levels, k, 12)
    b, _, _ = otree.build_tree(levels, k, 12, d2t=d2t)
    assert a["parents"] == b["parents"] and a["value"] == b["value"]
    ids = a["tokens"][1:]
    assert b["tokens"][1:] == [i + int(d2t[i]) for i in ids]


def test_brute_force_is_exhaustive_on_a_full_tree():
    """top_k = Vd: nothing is pruned by expansion at levels 1-2, so the pool is
    every path of length <= 2 and the top N is a plain sort of the full tree."""
    vd = 4
    f = _draft_fn(77, vd, 1.0)
    tb, res = _drive(f, vd, 2, 10)
    allp = [p for L in (1, 2) for p in itertools.product(range(vd), repeat=L)]
    val = {}
    for p in allp:
        v = 1.0
        for t in range(len(p)):
            v *= _probs(f(p[:t]))[p[t]]
        val[p] = v
    best = set(sorted(allp, key=lambda q: -val[q])[:10])
    paths = [()]
    for j in range(1, res["n_nodes"]):
        paths.append(paths[res["parents"][j]] + (res["tokens"][j],))
    assert set(paths[1:]) == best


def test_value_ties_go_to_lower_pool_index():
    """Reading T4 by hand: equal logits under equal parents give equal values
    (the same float64 sums), and the lower pool index wins each tie."""
    root = np.array([[0.0, 0.0, -1.0, -1.0]])
    row = np.array([0.0, 0.0, 0.0, -5.0])
    tb = otree.TreeBuilder(2)
    assert tb.expand(root) == [0, 1]
    assert tb.pool[0]["value"] == tb.pool[1]["value"]
    assert tb.expand(np.stack([row, row])) == [2, 3]
    assert len({tb.pool[p]["value"] for p in (2, 3, 4, 5)}) == 1
    res = tb.finalize(3, root_token=1)
    assert res["pool_ids"] == [0, 1, 2]
    assert res["parents"] == [-1, 0, 0, 1] and res["tokens"] == [1, 0, 1, 0]
    res = tb.finalize(1, root_token=1)
    assert res["pool_ids"] == [0]
