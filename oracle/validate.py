"""Input validation rules of the oracle (parity: pinned by tests/test_oracle_accept.py).

A draft tree is given as parent indices with the pending root at node 0.  A
node is accepted only if every node on its path from the root is accepted
(page "EAGLE-1/2/3 拆解", section "一个可核对的经验性质", the prefix property
of tree acceptance), so the tree must be rooted and acyclic; requiring
parents[j] < j (topological ids) makes both checks local.
"""
import numpy as np

# Device error bits (same meaning as the C header's SPEC_DEVERR_* flags; the
# values are part of the interface, not shared code).
ERR_TREE = 1        # n_nodes outside [1, n_max], bad parents, or depth > max_depth
ERR_TOKEN = 2       # a draft token outside [0, V)
ERR_NONFINITE = 4   # NaN/Inf in a logits or draft-probability entry the walk read
ERR_CAPACITY = 8    # prefix_len < 0 or prefix_len + n_nodes > L_cap


def validate_tree(parents, n_nodes, n_max, max_depth):
    """Return (ok, depths) for one sequence's tree."""
    n = int(n_nodes)
    if n < 1 or n > n_max:
        return False, None
    par = [int(x) for x in parents[:n]]
    if par[0] != -1:
        return False, None
    depth = [0] * n
    for j in range(1, n):
        if not (0 <= par[j] < j):
            return False, None
        depth[j] = depth[par[j]] + 1
        if depth[j] > max_depth:
            return False, None
    return True, np.asarray(depth, dtype=np.int64)
