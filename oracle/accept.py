"""Leviathan acceptance walked down a draft tree (float64).

Parity: pinned (tests/test_oracle_accept.py) by exact enumeration of the
first- and second-token marginals on tiny trees (they must equal the
verifier's distributions), a 50,000-step chi-square test of the first emitted
token, the closed form for the expected number of emitted tokens of an i.i.d.
chain, a brute-force greedy check at T = 0, the inverse-CDF definition on
hand-worked cases, and the special cases the pages fix.  The sampling
filters are pinned by hand-worked tables, the nucleus size of a geometric
distribution (closed form), ties, and enumeration with filtered q.

Rule (page "推测解码与 EAGLE-3", section "不变量：Leviathan 拒绝采样" and
build steps 1-3): a draft token d drawn from the draft distribution p is
accepted with probability min(1, q(d)/p(d)), q being the verifier's
distribution; on rejection one token is drawn from the residual
(q - p)_+ / ||(q - p)_+||_1 and the step stops; when every draft is accepted
a bonus token is drawn from the verifier's distribution after the last one.
The comparison is strict and a draft token with p(d) <= 0 is accepted (step
1); a residual of zero mass falls back to the distribution being corrected
(step 2).  The same rule appears with the letters swapped on page
"EAGLE-1/2/3 拆解", section "无损性的来源与它的证明位置".

Trees.  A node counts only if all nodes on its root path are accepted (page
"EAGLE-1/2/3 拆解", section "一个可核对的经验性质"), so the walk starts at the
root and descends.  The pages give the rule for one child per node only.
Reading used for several children (all drawn independently from the same
draft distribution p_v of their parent): test the children in ascending node
id; after each rejection replace the distribution being tested by its
residual against p_v; sample the terminal token from the distribution left
after the last rejection.  With one child this is exactly the pages' rule,
and it keeps the output distribution equal to q (checked by enumeration).

Temperature.  q = softmax(logits / T); T = 0 means greedy decoding: a draft is
accepted iff it equals the verifier's argmax (lowest id on ties) and the
terminal token is that argmax (page "EAGLE-1/2/3 拆解", opening section,
Temperature = 0 is greedy decoding, and the eagenerate flow section: the
longest passing prefix plus one corrected token lands each cycle).

Sampling filters.  top_k / top_p restrict every q of the walk (filter_keep);
the rule itself is unchanged, so the output follows the filtered q.

Near ties.  Decisions whose |u - min(1, ratio)| < TIE_BAND, samples whose
threshold u * W lies within SAMPLE_BAND * W of an edge of the chosen bucket,
top-p boundaries within FILTER_BAND of p, and residuals whose mass is a
positive fraction below DEGENERATE_BAND of the distribution they came from
are flagged; a flagged sequence-step is excluded from bit-exact comparison
with another implementation and logged.  The bands are readings, not the
pages': each is at least ten times the rounding an implementation that sums
the same float64 quantities in another order (or, for the top-p masses, in
fixed point of 2^-47 per entry, at most V * 2^-47 < 1e-9 for V up to 128k)
can make.
"""
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .validate import ERR_NONFINITE, ERR_TOKEN, ERR_TREE, validate_tree

TIE_BAND = 1e-6
SAMPLE_BAND = 1e-9
FILTER_BAND = 1e-8
DEGENERATE_BAND = 1e-12


def _full_distribution(lr, T):
    x = lr / float(T)
    e = np.exp(x - x.max())
    return e / e.sum()


def filter_keep(logit_row, T, top_k=0, top_p=0.0):
    """Tokens kept by the verifier's sampling filters, and the top-p margin.

    Page "EAGLE-1/2/3 拆解", section "一次 eagenerate 调用的完整流转", lists
    top_p and top_k (both 0, i.e. off, by default) beside temperature as the
    sampling arguments of the generation call.  Readings (listed in the design
    notes): both filters act on the verifier's q only (p is the draft's
    distribution as given) and are computed on the tempered distribution over
    the whole vocabulary; a token is kept when it passes both.  Top-k keeps
    every token whose logit is at least the k-th largest (ties at the k-th
    value all kept); 0 < top_k < V turns it on.  Top-p keeps a token when the
    mass of the tokens with strictly larger logits is below top_p (so ties are
    kept or dropped together, and the argmax always stays); 0 < top_p < 1
    turns it on.

    Returns (keep, margin): margin is the smallest |mass above - top_p| over
    the tokens the top-k filter keeps, leaving out the largest logit's tokens
    (nothing is above them, an exactly zero mass); inf with top-p off.  A
    margin under TIE_BAND marks a decision rounding could flip.
    """
    lr = np.asarray(logit_row, dtype=np.float64)
    V = len(lr)
    keep = np.ones(V, dtype=bool)
    if 0 < top_k < V:
        kth = np.sort(lr)[::-1][top_k - 1]
        keep &= lr >= kth
    margin = np.inf
    if 0.0 < top_p < 1.0:
        q = _full_distribution(lr, T)
        # distinct logits in descending order; mass of each tie group
        _, grp = np.unique(-lr, return_inverse=True)
        gmass = np.bincount(grp, weights=q)
        above = np.concatenate([[0.0], np.cumsum(gmass)[:-1]])[grp]
        # the tokens of the largest logit have nothing above them: that mass
        # is an empty sum, exactly 0 < top_p in any precision, so it decides
        # nothing rounding could flip
        cand = above[keep]
        cand = cand[cand > 0.0]
        margin = float(np.min(np.abs(cand - top_p))) if cand.size else np.inf
        keep &= above < top_p
    return keep, margin


def target_distribution(logit_row, T, top_k=0, top_p=0.0):
    """q = softmax(logits / T) in float64, restricted to the tokens
    filter_keep keeps and renormalised."""
    lr = np.asarray(logit_row, dtype=np.float64)
    e = _full_distribution(lr, T)
    if (0 < top_k < len(lr)) or (0.0 < top_p < 1.0):
        keep, _ = filter_keep(lr, T, top_k, top_p)
        e = np.where(keep, e, 0.0)
    return e / e.sum()


def keep_probability(target_x, draft_x):
    """Probability with which a draft token x survives its test.

    Page "推测解码与 EAGLE-3", build step 1 (section "第 1 步：拒绝规则"): the
    token is kept with probability min(1, target(x) / draft(x)).  A token the
    draft distribution gives no mass is kept outright; that case is returned
    as +inf so that every u in [0, 1) passes the strict comparison u < value.
    """
    if draft_x > 0.0:
        return min(1.0, target_x / draft_x)
    return np.inf


def remove_draft_mass(dist, draft):
    """The distribution a rejection leaves behind, and the mass it had.

    Page "推测解码与 EAGLE-3", build step 2 (section "第 2 步：残差分布"): after
    a rejection the next token comes from the part of the distribution the
    draft under-covers, (dist - draft)_+, renormalised.  When that part is
    empty (draft >= dist everywhere) the page keeps the distribution that was
    being corrected.  Returns (next distribution, mass of (dist - draft)_+);
    the mass is the ratio of successive residual masses that a closed-form
    implementation computes, and a tiny positive value marks a residual that
    rounding decides.
    """
    excess = np.clip(np.asarray(dist, np.float64) - np.asarray(draft, np.float64), 0.0, None)
    mass = float(excess.sum())
    if mass > 0.0:
        return excess / mass, mass
    return np.array(dist, dtype=np.float64, copy=True), mass


def sample_inverse_cdf(dist, u):
    """Token drawn from `dist` with uniform u in [0, 1).

    Reading (the pages do not fix the sampling procedure): inverse CDF in
    ascending token id -- the smallest i whose running sum exceeds u times the
    total; if rounding leaves none, the last i with positive mass.  Returns
    (i, margin) with margin the distance of u * total to the nearer edge of
    bucket i, relative to the total.
    """
    cdf = np.cumsum(dist)
    total = cdf[-1]
    t = float(u) * total
    i = int(np.searchsorted(cdf, t, side="right"))
    if i >= len(dist):
        i = int(np.nonzero(np.asarray(dist) > 0)[0][-1])
    lo = cdf[i - 1] if i > 0 else 0.0
    margin = min(abs(t - lo), abs(cdf[i] - t)) / total
    return i, float(margin)


@dataclass
class AcceptResult:
    accept_len: int                      # accepted drafts a (-1 on error)
    path: List[int]                      # node ids root..deepest accepted (a + 1)
    out_tokens: List[int]                # a accepted drafts, then the terminal token
    final_dist: Optional[np.ndarray]     # distribution the terminal token came from
    decisions: list = field(default_factory=list)  # (node, child, kind, u, value, margin, accepted)
    near_tie: bool = False
    error: int = 0


def draft_p_to_target(p_draft, d2t, V):
    """A draft distribution over the draft head's own vocabulary, moved onto
    the target vocabulary.

    Page "EAGLE-1/2/3 拆解", section "代码里能直接读到的三处改动": an EAGLE-3
    draft head ranks its own (smaller) vocabulary and draft id i stands for
    target token i + d2t[i].  So p(i + d2t[i]) = p_draft(i), and p is 0 on
    target tokens no draft id maps to (a child with such a token has draft
    probability 0, which the rule accepts).  p_draft: [..., Vd].  Returns None
    when the map is not one-to-one into [0, V) (reported as ERR_TOKEN).
    """
    d2t = np.asarray(d2t, dtype=np.int64)
    tgt = np.arange(len(d2t)) + d2t
    if (tgt < 0).any() or (tgt >= V).any() or len(np.unique(tgt)) != len(tgt):
        return None
    p_draft = np.asarray(p_draft, dtype=np.float64)
    out = np.zeros(p_draft.shape[:-1] + (V,))
    out[..., tgt] = p_draft
    return out


def _fail(err):
    return AcceptResult(-1, [], [], None, [], False, err)


def _children_lists(parents, n):
    kids = [[] for _ in range(n)]
    for j in range(1, n):
        kids[int(parents[j])].append(j)
    return kids


def visit_node(v, target, draft_row, kids, toks, u_accept, records):
    """The child tests at one visited node (T > 0).

    target: the verifier's distribution at v (already filtered).  The
    children are tested in ascending id (reading for several children, module
    docstring); each rejection replaces the distribution under test by what
    remove_draft_mass leaves of it against v's draft row.  The draft row is
    checked for non-finite entries only once a rejection uses all of it (a
    walk reads nothing else of it).  Appends a record per test and per
    residual to `records` and returns (accepted child or None, the
    distribution under test when the node's tests ended, error bits).
    """
    dist = target
    checked = False
    for c in kids:
        x = toks[c]
        px = float(draft_row[x])
        if not np.isfinite(px):
            return None, dist, ERR_NONFINITE
        u = float(u_accept[c])
        kp = keep_probability(dist[x], px)
        passed = u < kp
        records.append((v, c, "accept-test", u, kp, abs(u - kp) if np.isfinite(kp) else np.inf,
                        passed))
        if passed:
            return c, dist, 0
        if not checked:
            if not np.all(np.isfinite(np.asarray(draft_row, dtype=np.float64))):
                return None, dist, ERR_NONFINITE
            checked = True
        dist, mass = remove_draft_mass(dist, draft_row)
        records.append((v, c, "residual", None, mass, mass, None))
    return None, dist, 0


def accept_tree(tokens, parents, n_nodes, draft_p, logits, T, u_accept, u_sample,
                max_depth, n_max=None, top_k=0, top_p=0.0):
    """One sequence's acceptance walk.

    tokens/parents/u_accept/u_sample: [n_max]; draft_p/logits: [n_max][V].
    Node 0 is the pending root; row v of draft_p is the distribution the
    children of v were drawn from, row v of logits the verifier's logits
    after v.  top_k / top_p: the sampling filters of filter_keep, applied to
    every q of the walk at T > 0 (greedy decoding is unaffected: the argmax
    always passes both).

    Near ties (flag `near_tie`): a test with |u - keep probability| <
    TIE_BAND, a sample whose threshold lies within SAMPLE_BAND of an edge of
    the chosen bucket, a top-p boundary within FILTER_BAND, and a residual whose
    mass is positive but below DEGENERATE_BAND of the distribution it came
    from (rounding then decides what is left).
    """
    n = int(n_nodes)
    if n_max is None:
        n_max = len(parents)
    ok, _ = validate_tree(parents, n, n_max, max_depth)
    if not ok:
        return _fail(ERR_TREE)
    V = np.asarray(logits[0]).shape[-1]
    toks = [int(t) for t in tokens[:n]]
    if any(t < 0 or t >= V for t in toks[1:]):
        return _fail(ERR_TOKEN)
    kids = _children_lists(parents, n)

    path, emitted, records = [0], [], []
    v = 0
    while True:
        lrow = np.asarray(logits[v], dtype=np.float64)
        if not np.all(np.isfinite(lrow)):
            return _fail(ERR_NONFINITE)
        if T == 0:
            # greedy: the first child carrying the verifier's argmax survives
            best = int(np.argmax(lrow))
            nxt = next((c for c in kids[v] if toks[c] == best), None)
            records.append((v, -1 if nxt is None else nxt, "argmax", None, best, None,
                            nxt is not None))
            emitted.append(best)
            if nxt is None:
                final = np.zeros(V)
                final[best] = 1.0
                break
            path.append(nxt)
            v = nxt
            continue

        target = target_distribution(lrow, T, top_k, top_p)
        if 0.0 < top_p < 1.0:
            _, fm = filter_keep(lrow, T, top_k, top_p)
            records.append((v, -1, "filter", None, top_p, fm, None))
        nxt, dist, err = visit_node(v, target, draft_p[v], kids[v], toks, u_accept, records)
        if err:
            return _fail(err)
        if nxt is not None:
            path.append(nxt)
            emitted.append(toks[nxt])
            v = nxt
            continue
        us = float(u_sample[v])
        tok, margin = sample_inverse_cdf(dist, us)
        records.append((v, -1, "sample", us, tok, margin, None))
        emitted.append(tok)
        final = dist
        break
    near = any(_is_near_tie(r) for r in records)
    return AcceptResult(len(path) - 1, path, emitted, final, records, near, 0)


def _is_near_tie(record):
    kind, margin = record[2], record[5]
    if kind == "accept-test":
        return margin < TIE_BAND
    if kind == "filter":
        return margin < FILTER_BAND
    if kind == "sample":
        return margin < SAMPLE_BAND
    if kind == "residual":
        return 0.0 < margin < DEGENERATE_BAND
    return False


def terminal_distribution(node, tokens, parents, n_nodes, draft_p, logits, T, top_k=0, top_p=0.0):
    """The distribution a walk that stops at `node` draws its last token
    from: the verifier's distribution there with every child of the node
    rejected in ascending id (T > 0), or the point mass at the argmax (T = 0).
    Used to check a walk taken by another implementation."""
    lrow = np.asarray(logits[node], dtype=np.float64)
    if T == 0:
        out = np.zeros(len(lrow))
        out[int(np.argmax(lrow))] = 1.0
        return out
    dist = target_distribution(lrow, T, top_k, top_p)
    draft = np.asarray(draft_p[node], dtype=np.float64)
    for c in _children_lists(parents, int(n_nodes))[node]:
        dist, _ = remove_draft_mass(dist, draft)
    return dist
