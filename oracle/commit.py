"""KV commit of the accepted path (plain copies).

Parity: pinned (tests/test_oracle_commit.py) by the bookkeeping invariants of
page "推测解码与 EAGLE-3", section "KV cache 回滚" and build step 4, the
page's batched-rollback exercise worked out by hand under tests/golden/, and
(for the scratch-buffer form) its agreement with the in-place form on the same
tree rows.

The verify pass has written the K/V of every tree node into cache rows
prefix_len + i.  Rollback is either a physical cache with a logical length
that is cut back on rejection, or a scratch area committed on acceptance
(section "KV cache 回滚").  For a tree, the accepted path's rows are in
general scattered, so they are gathered to the rows right after the prefix:
row prefix_len + i receives the pre-commit row prefix_len + path[i], for the
root (i = 0) and the a accepted drafts.

Reading of the logical length (build step 4 sets it to prefix_length + j + 1
on rejection at position j): j is the number of accepted drafts and the +1 is
the root, the previous step's emitted token whose KV this pass produced.  The
terminal (corrected or bonus) token has no KV yet; it becomes the next root.
"""
import numpy as np


def kv_commit(k, v, prefix_len, path, accept_len):
    """k, v: [Hkv][L_cap][d] of one sequence.  Returns (k', v', new_len)."""
    k = np.asarray(k)
    v = np.asarray(v)
    if accept_len < 0:
        return k.copy(), v.copy(), int(prefix_len)
    L = int(prefix_len)
    k2 = k.copy()
    v2 = v.copy()
    for i in range(int(accept_len) + 1):
        k2[:, L + i] = k[:, L + int(path[i])]
        v2[:, L + i] = v[:, L + int(path[i])]
    return k2, v2, L + int(accept_len) + 1


def kv_commit_from_buffer(k, v, k_tree, v_tree, prefix_len, path, accept_len):
    """The other rollback form of section "KV cache 回滚": the verify pass wrote
    the tree's K/V to a scratch buffer, and acceptance commits the root and the
    accepted drafts into the cache.

    k, v: [Hkv][L_cap][d] cache of one sequence; k_tree, v_tree: [Hkv][n][d]
    scratch rows of its tree.  Cache row prefix_len + i receives scratch row
    path[i] for i = 0..a (the root included: the cache never held it).
    Returns (k', v', new_len); a sequence with accept_len < 0 is unchanged.
    """
    k = np.asarray(k)
    v = np.asarray(v)
    if accept_len < 0:
        return k.copy(), v.copy(), int(prefix_len)
    L = int(prefix_len)
    k2 = k.copy()
    v2 = v.copy()
    for i in range(int(accept_len) + 1):
        k2[:, L + i] = np.asarray(k_tree)[:, int(path[i])]
        v2[:, L + i] = np.asarray(v_tree)[:, int(path[i])]
    return k2, v2, L + int(accept_len) + 1
