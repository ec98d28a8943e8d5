"""Pins for the oracle's KV commit (CPU only).

Fixed by the rollback bookkeeping of page "推测解码与 EAGLE-3" (section
"KV cache 回滚" and build step 4) and its batched-rollback exercise, worked by
hand in tests/golden/batched_rollback.json.
"""
import json
import os

import numpy as np
import pytest

import oracle
from eagle_tree_verification_amd.workloads import tree_shape

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
HI = float(np.nextafter(1.0, 0.0))


@pytest.mark.parametrize("seed", range(8))
def test_commit_invariants(seed):
    rng = np.random.default_rng(seed)
    depth = int(rng.integers(1, 4))
    parents = tree_shape(int(rng.integers(depth, 10 * depth)), depth, rng)
    n = len(parents)
    leaf = int(rng.integers(0, n))
    path = oracle.path_to_root(parents, leaf)
    a = len(path) - 1
    hkv, d, L = 3, 8, int(rng.integers(0, 30))
    cap = L + n + 4
    k = rng.normal(size=(hkv, cap, d))
    v = rng.normal(size=(hkv, cap, d))
    k2, v2, new_len = oracle.kv_commit(k, v, L, path, a)
    assert new_len == L + a + 1
    np.testing.assert_array_equal(k2[:, :L], k[:, :L])
    np.testing.assert_array_equal(v2[:, :L], v[:, :L])
    for i, node in enumerate(path):
        np.testing.assert_array_equal(k2[:, L + i], k[:, L + node])
        np.testing.assert_array_equal(v2[:, L + i], v[:, L + node])
    np.testing.assert_array_equal(k2[:, L + a + 1:], k[:, L + a + 1:])


def test_chain_commit_moves_nothing():
    rng = np.random.default_rng(1)
    k = rng.normal(size=(2, 20, 4))
    v = rng.normal(size=(2, 20, 4))
    for a in range(6):
        k2, v2, new_len = oracle.kv_commit(k, v, 9, list(range(a + 1)), a)
        np.testing.assert_array_equal(k2, k)
        np.testing.assert_array_equal(v2, v)
        assert new_len == 9 + a + 1


def test_failed_sequence_is_left_alone():
    k = np.arange(24.0).reshape(1, 6, 4)
    k2, v2, new_len = oracle.kv_commit(k, k, 2, [], -1)
    np.testing.assert_array_equal(k2, k)
    assert new_len == 2


def test_batched_rollback_exercise():
    with open(os.path.join(GOLDEN, "batched_rollback.json")) as f:
        g = json.load(f)
    V = 16
    for seq in g["sequences"]:
        parents = np.asarray(seq["parents"], np.int32)
        n = len(parents)
        # verifier == draft except that the draft over-weights the token of
        # the node that must be rejected; u = 0 accepts, u just below 1 rejects
        q = np.full(V, 1.0 / V)
        logits = np.log(np.tile(q, (n, 1)))
        p = np.tile(q, (n, 1))
        tokens = np.arange(n) % V
        u = np.zeros(n)
        for node in seq["rejected_nodes"]:
            prow = np.full(V, 0.5 / (V - 1))
            prow[tokens[node]] = 0.5
            p[parents[node]] = prow
            u[node] = HI
        r = oracle.accept_tree(tokens, parents, n, p, logits, 1.0, u, np.zeros(n), n)
        assert r.accept_len == seq["accept_len"]
        assert r.path == seq["path"]
        hkv, d, L = 2, 4, seq["prefix_len"]
        k = np.random.default_rng(0).normal(size=(hkv, L + n + 2, d))
        k2, _, new_len = oracle.kv_commit(k, k, L, r.path, r.accept_len)
        assert new_len == seq["new_len"]
        moved = sum(int(not np.array_equal(k2[:, L + i], k[:, L + i])) for i in range(n))
        assert moved == seq["rows_moved"]


@pytest.mark.parametrize("seed", range(6))
def test_commit_from_buffer_matches_in_place(seed):
    """The scratch-buffer form and the in-place form of the rollback section
    commit the same rows when the scratch rows equal the cache's tree rows;
    rows the scratch form never touches stay as they were."""
    rng = np.random.default_rng(100 + seed)
    depth = int(rng.integers(1, 4))
    parents = tree_shape(int(rng.integers(depth, 10 * depth)), depth, rng)
    n = len(parents)
    path = oracle.path_to_root(parents, int(rng.integers(0, n)))
    a = len(path) - 1
    hkv, d, L = 2, 4, int(rng.integers(0, 20))
    cap = L + n + 3
    k = rng.normal(size=(hkv, cap, d))
    v = rng.normal(size=(hkv, cap, d))
    k_tree, v_tree = k[:, L:L + n].copy(), v[:, L:L + n].copy()
    ki, vi, li = oracle.kv_commit(k, v, L, path, a)
    # the scratch form starts from a cache whose tree rows hold stale data
    stale_k, stale_v = k.copy(), v.copy()
    stale_k[:, L:] = -7.0
    stale_v[:, L:] = -7.0
    kb, vb, lb = oracle.kv_commit_from_buffer(stale_k, stale_v, k_tree, v_tree, L, path, a)
    assert lb == li == L + a + 1
    np.testing.assert_array_equal(kb[:, :L + a + 1], ki[:, :L + a + 1])
    np.testing.assert_array_equal(vb[:, :L + a + 1], vi[:, :L + a + 1])
    assert np.all(kb[:, L + a + 1:] == -7.0) and np.all(vb[:, L + a + 1:] == -7.0)


def test_commit_from_buffer_chain_and_failure():
    # a chain accepts its first a drafts in order; a failed walk changes nothing
    hkv, d, L, n = 1, 2, 5, 4
    k = np.zeros((hkv, L + n, d))
    v = np.zeros((hkv, L + n, d))
    kt = np.arange(n * d, dtype=float).reshape(1, n, d)
    vt = -kt
    k2, v2, ln = oracle.kv_commit_from_buffer(k, v, kt, vt, L, [0, 1, 2], 2)
    assert ln == L + 3
    np.testing.assert_array_equal(k2[0, L:L + 3], kt[0, :3])
    np.testing.assert_array_equal(v2[0, L:L + 3], vt[0, :3])
    assert np.all(k2[0, L + 3:] == 0)
    k3, v3, l3 = oracle.kv_commit_from_buffer(k, v, kt, vt, L, [], -1)
    assert l3 == L and np.all(k3 == k) and np.all(v3 == v)
