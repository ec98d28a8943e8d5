"""Rotary position embedding of tree nodes -- TEST INFRASTRUCTURE ONLY.

Parity: pinned (tests/test_oracle_rope.py) by the complex-number form of the
rotation (an independent formula route), the relative-position property
<R(m) q, R(n) k> = <R(m+t) q, R(n+t) k>, composition R(m) R(n) = R(m+n), norm
preservation, a rotation by a quarter turn worked by hand, the relation
between the two pair layouts (a fixed permutation), and, for attention, a
chain tree equal to causal attention over the rotated sequence.

Positions of tree nodes.  Page "EAGLE-1/2/3 拆解", the init_tree passage: the
draft's position ids for the top_k candidates of one level start as zeros,
i.e. every candidate of a level sits at the same offset from the accepted
sequence.  Reading (listed in the design notes as RP1): tree node j is at
position prefix_len + depth(j); the root (the pending token, depth 0) is at
prefix_len, the first position after the committed prefix.

The rotation itself is the published rotary embedding (Su et al., RoFormer,
2021): the head dimension is split into d/2 planes, and plane i is rotated by
the angle pos * inv_freq[i].  Readings (RP2): the caller supplies inv_freq
(any frequency schedule, e.g. base**(-2i/d) or a rescaled one); "half" pairs
dimension i with i + d/2 (the layout of the LLaMA-family targets the configs
name), "interleaved" pairs 2i with 2i + 1.  Angles, cosines and sines are
float64 here.
"""
import numpy as np

STYLES = ("half", "interleaved")


def _planes(d, style):
    """Index arrays (first, second) of the d/2 rotation planes."""
    i = np.arange(d // 2)
    if style == "half":
        return i, i + d // 2
    if style == "interleaved":
        return 2 * i, 2 * i + 1
    raise ValueError(style)


def rope_rotate(x, pos, inv_freq, style="half"):
    """Rotate vectors x[..., d] at positions pos (broadcast over x[..., 0])."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    f = np.asarray(inv_freq, dtype=np.float64)
    assert f.shape == (d // 2,)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * f
    c, s = np.cos(ang), np.sin(ang)
    a, b = _planes(d, style)
    out = x.copy()
    out[..., a] = x[..., a] * c - x[..., b] * s
    out[..., b] = x[..., b] * c + x[..., a] * s
    return out


def node_positions(parents, n, prefix_len):
    """prefix_len + depth(j) for nodes 0..n-1 (reading RP1)."""
    depth = np.zeros(n, dtype=np.int64)
    for j in range(1, n):
        depth[j] = depth[int(parents[j])] + 1
    return int(prefix_len) + depth


def tree_kv_write(k_cache, v_cache, k_new, v_new, prefix_len, parents, n, inv_freq=None,
                  style="half"):
    """The verify pass's write of the tree's K/V into the cache: cache row
    prefix_len + j receives K of node j rotated at its position (unrotated if
    inv_freq is None) and V of node j.

    k_cache, v_cache: [Hkv][rows][d]; k_new, v_new: [n_max][Hkv][d].
    Returns float64 copies of the caches.
    """
    k2 = np.array(k_cache, dtype=np.float64)
    v2 = np.array(v_cache, dtype=np.float64)
    L = int(prefix_len)
    pos = node_positions(parents, n, L)
    kn = np.asarray(k_new, dtype=np.float64)[:n]          # [n][Hkv][d]
    if inv_freq is not None:
        kn = rope_rotate(kn, pos[:, None], inv_freq, style)
    k2[:, L:L + n] = np.transpose(kn, (1, 0, 2))
    v2[:, L:L + n] = np.transpose(np.asarray(v_new, dtype=np.float64)[:n], (1, 0, 2))
    return k2, v2
