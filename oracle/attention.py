"""Tree-masked attention, plain definition (float64).

Parity: pinned (tests/test_oracle_attention.py) against PyTorch's
scaled-dot-product attention with a causal mask on the explicit sequence
"prefix, then the node's root-to-node path", a chain closed form, a
constant-key closed form, invariance to non-ancestors and node relabelling.

What is computed.  During verification every draft-tree node attends to the
whole committed prefix and to its own ancestors, itself included, and to no
other tree node: the verifier runs attention with a non-causal mask that
follows the tree topology (page "推测解码与 EAGLE-3", section "KV cache 回滚";
page "EAGLE-1/2/3 拆解", section on EAGLE-2's two stages, where the initial
tree mask is the identity so a node sees itself and siblings do not see each
other; page "EAGLE-3 完全拆解", section on the training-time tree mask, where
each simulated token sees only its legal ancestors).  So the output of node j
is exactly the last row of ordinary causal attention over the sequence
"prefix tokens, then path(j)".

Readings where the pages are silent: scale = 1/sqrt(d) unless given; query
head h reads KV head h // (Hq / Hkv) (grouped-query attention); Q and K are
already position-encoded; output is float64 here, float32 on the device.
"""
import numpy as np


def path_to_root(parents, j):
    """Node ids from the root (node 0) down to node j, both included."""
    path = []
    while j >= 0:
        path.append(int(j))
        j = int(parents[j])
    return path[::-1]


def ancestors(parents, n):
    """List of root-to-node paths for nodes 0..n-1."""
    return [path_to_root(parents, j) for j in range(n)]


def tree_attention(q, k, v, prefix_len, parents, scale=None, nodes=None, heads=None):
    """Attention of every tree node over prefix + its ancestor path.

    q: [n][Hq][d]; k, v: [Hkv][rows][d] with rows >= prefix_len + n, prefix
    K/V in rows [0, prefix_len) and tree node i in row prefix_len + i.
    Returns out [n][Hq][d] float64; entries not in `nodes` x `heads` are NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, hq, d = q.shape
    hkv = k.shape[0]
    group = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    L = int(prefix_len)
    nodes = range(n) if nodes is None else nodes
    heads = range(hq) if heads is None else heads
    out = np.full((n, hq, d), np.nan)
    for j in nodes:
        keys = np.concatenate([np.arange(L), L + np.asarray(path_to_root(parents, j))])
        for h in heads:
            g = h // group
            s = (k[g, keys] @ q[j, h]) * scale
            w = np.exp(s - s.max())
            w /= w.sum()
            out[j, h] = w @ v[g, keys]
    return out
