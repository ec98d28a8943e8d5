"""EAGLE-2 draft-tree construction: expansion by path value, then rerank.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may use it).

Parity: pinned (tests/test_oracle_tree.py) by a tree worked out by hand
(tests/golden/tree_build_small.json), by a brute-force restatement over the
complete draft tree of tiny vocabularies (values recomputed as products of
probabilities, every level's expansion and the final top N checked from their
definitions), by top_k = 1 reducing to greedy decoding of the draft, and by
structural invariants (ancestor closure, topological ids, depths).

What the method computes (page "EAGLE-1/2/3 拆解"):
  * section "一个可核对的经验性质": a draft node is accepted only if every
    node on its root path is, so its value is the product of the draft's
    confidences along that path;
  * section "两阶段，而不是'按置信度决定深度'": Expansion -- level by level,
    the draft runs only on the k most valuable nodes of the level before (one
    forward for all of them, thanks to tree attention); Reranking -- every
    node of the grown tree is ranked by value and the N best go to
    verification, because an unexpanded shallow node can be worth more than
    an expanded deep one;
  * the paragraph after init_tree: the papers' settings (60/50/48 drafts,
    depth 6, 10 nodes expanded per level) and the code defaults
    (total_tokens 63, depth 5, top_k 8);
  * section "代码里能直接读到的三处改动": an EAGLE-3 draft head ranks its own
    vocabulary and draft id i stands for target token i + d2t[i].
Page "EAGLE-3 完全拆解", section "EAGLE-3 和 EAGLE-2 动态树如何拼在一起": the
same path value decides what is expanded and what is verified; EAGLE-3 keeps
the dynamic tree and grows it to depth 8.

Readings where the pages leave a step open (each listed in the design notes):
  T1  a confidence is the draft's softmax probability of the token (no
      temperature); values are kept as sums of log-probabilities, which orders
      nodes exactly as the product does;
  T2  the children of an expanded node are its top_k most probable draft ids,
      equal logits going to the lower id;
  T3  level 1 is the root's one draft row; all of its top_k children are
      expanded.  At level l >= 2 the draft rows belong to the expanded nodes
      of level l-1, most valuable first; their top_k * top_k children join the
      pool and the top_k most valuable of them are expanded next;
  T4  pool order is (level, draft row, child rank); equal values go to the
      lower pool index.  A child's value never exceeds its parent's and a
      parent precedes its children, so the top N always hold every ancestor
      of every member;
  T5  the N chosen drafts follow the root (node 0) in pool order, so parents
      precede children; a node of value -inf (probability 0) is never chosen.
"""
import numpy as np

from .validate import ERR_NONFINITE


def draft_log_probs(z):
    """log softmax of one draft row, in float64 (reading T1).

    Returns None when the row has a NaN or +inf entry, or no finite entry:
    such a row defines no distribution.
    """
    z = np.asarray(z, dtype=np.float64)
    if np.isnan(z).any() or np.isposinf(z).any() or not np.isfinite(z).any():
        return None
    m = z.max()
    return z - (m + np.log(np.sum(np.exp(z - m))))


def top_children(z, k):
    """The k most probable draft ids of row z, best first; ties to the lower
    id (reading T2).  Sorting by logit equals sorting by probability."""
    z = np.asarray(z, dtype=np.float64)
    # lexsort: last key is primary -> by -z, then by id
    order = np.lexsort((np.arange(len(z)), -z))
    return [int(i) for i in order[:k]]


class TreeBuilder:
    """One sequence's tree, grown one level per draft forward (reading T3).

    Pool entries are dicts with the draft id, target token, pool parent (-1 =
    the root), depth and value (sum of log-probabilities).
    """

    def __init__(self, top_k, d2t=None):
        self.k = int(top_k)
        self.d2t = None if d2t is None else np.asarray(d2t, dtype=np.int64)
        self.pool = []
        self.expanded = []      # expanded[l-1]: pool ids expanded at level l, best first
        self.failed = False

    def expand(self, rows):
        """Add one level from the draft rows of the last expanded nodes.

        rows: [1][Vd] at level 1 (the root's row), [top_k][Vd] afterwards; row
        r belongs to the r-th expanded node of the previous level.  Returns
        the pool ids chosen for expansion at this level (empty on failure).
        """
        if self.failed:
            self.expanded.append([])
            return []
        rows = np.atleast_2d(np.asarray(rows, dtype=np.float64))
        level = len(self.expanded) + 1
        if level == 1:
            feeders = [(-1, 0.0)]
        else:
            feeders = [(pid, self.pool[pid]["value"]) for pid in self.expanded[-1]]
        assert rows.shape[0] == len(feeders), "one draft row per expanded node"
        new_ids = []
        for r, (parent, pval) in enumerate(feeders):
            lp = draft_log_probs(rows[r])
            if lp is None:
                self.failed = True
                self.expanded.append([])
                return []
            for i in top_children(rows[r], self.k):
                tok = i if self.d2t is None else i + int(self.d2t[i])
                self.pool.append({"draft_id": i, "token": tok, "parent": parent,
                                  "depth": level, "value": pval + lp[i]})
                new_ids.append(len(self.pool) - 1)
        chosen = sorted(new_ids, key=lambda p: (-self.pool[p]["value"], p))[:self.k]
        self.expanded.append(chosen)
        return chosen

    def finalize(self, total_tokens, root_token, prefix_len=0):
        """Rerank (readings T4, T5): the total_tokens most valuable pool nodes
        in pool order after the root.  Returns a dict of per-node lists, or
        None if a draft row was invalid (ERR_NONFINITE)."""
        if self.failed:
            return None
        live = [p for p in range(len(self.pool)) if self.pool[p]["value"] > -np.inf]
        chosen = sorted(live, key=lambda p: (-self.pool[p]["value"], p))[:int(total_tokens)]
        chosen.sort()
        node_of = {p: j + 1 for j, p in enumerate(chosen)}
        # draft row of an expanded node: row 0 is the root's, then level l's
        # k rows follow level l-1's; the last level's choices have no rows.
        row_of = {}
        for lv, ids in enumerate(self.expanded[:-1]):
            for r, pid in enumerate(ids):
                row_of[pid] = 1 + lv * self.k + r
        tokens = [int(root_token)]
        parents = [-1]
        depth = [0]
        value = [0.0]
        draft_row = [0]
        for p in chosen:
            e = self.pool[p]
            assert e["parent"] == -1 or e["parent"] in node_of, "ancestor closure"
            tokens.append(e["token"])
            parents.append(0 if e["parent"] == -1 else node_of[e["parent"]])
            depth.append(e["depth"])
            value.append(e["value"])
            draft_row.append(row_of.get(p, -1))
        n = len(tokens)
        mask = [0] * n
        mask[0] = 1
        for j in range(1, n):
            mask[j] = mask[parents[j]] | (1 << j)
        return {"n_nodes": n, "tokens": tokens, "parents": parents, "depth": depth,
                "positions": [int(prefix_len) + d for d in depth], "value": value,
                "draft_row": draft_row, "anc_mask": mask, "pool_ids": chosen}


def build_tree(level_rows, top_k, total_tokens, root_token=0, prefix_len=0, d2t=None):
    """Whole construction for one sequence from its per-level draft rows.

    level_rows[0] is the root's row, level_rows[l] (l >= 1) the top_k rows of
    level l's expanded nodes.  Returns (result or None, error bits, builder).
    """
    tb = TreeBuilder(top_k, d2t)
    for rows in level_rows:
        tb.expand(rows)
    res = tb.finalize(total_tokens, root_token, prefix_len)
    return res, (ERR_NONFINITE if res is None else 0), tb
