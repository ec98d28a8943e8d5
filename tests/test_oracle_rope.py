"""Pins for the oracle's rotary position embedding of tree nodes (CPU only).

The rotation is pinned by routes other than its own formula: complex
multiplication, the relative-position property, composition, norm
preservation, a quarter turn worked by hand and the fixed permutation between
the two pair layouts.  Tree positions (prefix_len + depth, page "EAGLE-1/2/3
拆解", the init_tree passage: the candidates of a level share one position)
are pinned by explicit causal attention: every node's output equals the last
row of causal attention over "prefix, then its root path" with each element
rotated at its index in that sequence.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import rope as orope
from eagle_tree_verification_amd.workloads import tree_shape


def _freq(d, base=10000.0):
    return base ** (-np.arange(d // 2) * 2.0 / d)


@pytest.mark.parametrize("style", orope.STYLES)
def test_complex_multiplication_form(style):
    rng = np.random.default_rng(1)
    d = 16
    x = rng.normal(size=(5, d))
    pos = rng.integers(0, 5000, size=5)
    f = _freq(d)
    got = orope.rope_rotate(x, pos, f, style)
    if style == "half":
        z = x[:, : d // 2] + 1j * x[:, d // 2:]
    else:
        z = x[:, 0::2] + 1j * x[:, 1::2]
    w = z * np.exp(1j * pos[:, None] * f)
    if style == "half":
        want = np.concatenate([w.real, w.imag], axis=1)
    else:
        want = np.stack([w.real, w.imag], axis=-1).reshape(5, d)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("style", orope.STYLES)
def test_relative_position_norm_and_composition(style):
    rng = np.random.default_rng(2)
    d = 32
    f = _freq(d, 500000.0)
    q, k = rng.normal(size=d), rng.normal(size=d)
    for m, n, t in [(0, 0, 7), (3, 11, 100), (4096, 17, 3001), (9, 9000, -9)]:
        a = orope.rope_rotate(q, m, f, style) @ orope.rope_rotate(k, n, f, style)
        b = orope.rope_rotate(q, m + t, f, style) @ orope.rope_rotate(k, n + t, f, style)
        assert a == pytest.approx(b, rel=1e-9, abs=1e-9)
    x = rng.normal(size=(4, d))
    np.testing.assert_allclose(np.linalg.norm(orope.rope_rotate(x, 12345, f, style), axis=1),
                               np.linalg.norm(x, axis=1), rtol=1e-12)
    np.testing.assert_allclose(orope.rope_rotate(x, 0, f, style), x, rtol=0, atol=0)
    two = orope.rope_rotate(orope.rope_rotate(x, 30, f, style), 45, f, style)
    np.testing.assert_allclose(two, orope.rope_rotate(x, 75, f, style), rtol=0, atol=1e-12)


def test_quarter_turn_by_hand():
    # d = 4, frequencies (pi/2, pi): at position 1 plane 0 turns a quarter,
    # plane 1 a half.  "half" planes are (0, 2) and (1, 3).
    f = np.array([np.pi / 2, np.pi])
    x = np.array([1.0, 2.0, 3.0, 4.0])
    # plane (0,2): (1, 3) -> (-3, 1); plane (1,3): (2, 4) -> (-2, -4)
    np.testing.assert_allclose(orope.rope_rotate(x, 1, f, "half"), [-3.0, -2.0, 1.0, -4.0],
                               atol=1e-15)
    # "interleaved" planes (0,1) and (2,3): (1,2) -> (-2,1); (3,4) -> (-3,-4)
    np.testing.assert_allclose(orope.rope_rotate(x, 1, f, "interleaved"), [-2.0, 1.0, -3.0, -4.0],
                               atol=1e-15)


def test_layouts_differ_by_a_fixed_permutation():
    rng = np.random.default_rng(3)
    d = 8
    f = _freq(d)
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])  # interleaved -> half
    x = rng.normal(size=(3, d))
    a = orope.rope_rotate(x, 77, f, "interleaved")
    b = orope.rope_rotate(x[:, perm], 77, f, "half")
    np.testing.assert_allclose(a[:, perm], b, atol=1e-14)


def _sdpa_last_row(qv, keys, vals, hq, hkv):
    S, d = keys.shape[1], keys.shape[2]
    g = hq // hkv
    k = torch.from_numpy(np.repeat(keys, g, axis=0))[None]
    v = torch.from_numpy(np.repeat(vals, g, axis=0))[None]
    q = torch.zeros((1, hq, S, d), dtype=torch.float64)
    q[0, :, -1] = torch.from_numpy(qv)
    return F.scaled_dot_product_attention(q, k, v, is_causal=True)[0, :, -1].numpy()


@pytest.mark.parametrize("style", orope.STYLES)
@pytest.mark.parametrize("seed", range(3))
def test_tree_positions_match_explicit_causal_attention(style, seed):
    rng = np.random.default_rng(10 + seed)
    hq, hkv, d = 4, 2, 16
    L = int(rng.integers(0, 12))
    depth = int(rng.integers(1, 4))
    parents = tree_shape(int(rng.integers(depth, 9)), depth, rng)
    n = len(parents)
    f = _freq(d)
    # raw (unrotated) vectors: prefix keys at positions 0..L-1, tree q/k/v
    kp_raw = rng.normal(size=(hkv, L, d))
    vp = rng.normal(size=(hkv, L, d))
    q_raw = rng.normal(size=(n, hq, d))
    kn_raw = rng.normal(size=(n, hkv, d))
    vn = rng.normal(size=(n, hkv, d))
    # the cache holds the prefix rotated at its positions, as committed earlier
    kc = np.zeros((hkv, L + n + 2, d))
    vc = np.zeros((hkv, L + n + 2, d))
    kc[:, :L] = orope.rope_rotate(kp_raw, np.arange(L)[None, :], f, style)
    vc[:, :L] = vp
    kc, vc = orope.tree_kv_write(kc, vc, kn_raw, vn, L, parents, n, f, style)
    pos = orope.node_positions(parents, n, L)
    q = orope.rope_rotate(q_raw, pos[:, None], f, style)
    out = oracle.tree_attention(q, kc, vc, L, parents)
    for j in range(n):
        path = oracle.path_to_root(parents, j)
        seq_pos = np.arange(L + len(path))
        keys = np.concatenate([kp_raw, np.transpose(kn_raw[path], (1, 0, 2))], axis=1)
        vals = np.concatenate([vp, np.transpose(vn[path], (1, 0, 2))], axis=1)
        keys = orope.rope_rotate(keys, seq_pos[None, :], f, style)
        qv = orope.rope_rotate(q_raw[j], seq_pos[-1], f, style)
        np.testing.assert_allclose(out[j], _sdpa_last_row(qv, keys, vals, hq, hkv), atol=1e-12)


def test_positions_and_unrotated_write():
    parents = np.array([-1, 0, 0, 1, 3, 2])
    assert list(orope.node_positions(parents, 6, 40)) == [40, 41, 41, 42, 43, 42]
    rng = np.random.default_rng(5)
    kc, vc = np.zeros((2, 9, 4)), np.ones((2, 9, 4))
    kn, vn = rng.normal(size=(6, 2, 4)), rng.normal(size=(6, 2, 4))
    k2, v2 = orope.tree_kv_write(kc, vc, kn, vn, 3, parents, 6)
    np.testing.assert_array_equal(k2[:, 3:9], np.transpose(kn, (1, 0, 2)))
    np.testing.assert_array_equal(v2[:, 3:9], np.transpose(vn, (1, 0, 2)))
    np.testing.assert_array_equal(v2[:, :3], 1.0)
