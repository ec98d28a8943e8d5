"""CPU oracle for EAGLE-2/3 tree verification -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 NumPy reference of the three steps of the verify path:
tree-masked attention (`attention`), the Leviathan acceptance walk down the
draft tree (`accept`) and the KV commit (`commit`), plus the step before it,
EAGLE-2's construction of the draft tree from draft probabilities (`tree`),
the rotary position embedding of tree nodes with the write of their K/V
into the cache (`rope`), and the logical view of a cache held in blocks
through a block table (`paged`).  Every function cites the
passage of the pages it follows.  Pages cited throughout:

  * "推测解码与 EAGLE-3" -- a lesson on speculative decoding and EAGLE-3
    (the rejection rule, the residual distribution, KV rollback, the
    Leviathan check and the expected-accepted closed form);
  * "EAGLE-1/2/3 拆解" -- a guide to the EAGLE repository and papers
    (losslessness, the prefix property of tree acceptance, the tree mask);
  * "EAGLE-3 完全拆解" -- an article on EAGLE-3's training-time test
    (tree-shaped masks, tree budgets).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  It shares no code with the HIP library or its Python
binding, and imports neither.  Parity status of every function is listed in
its module docstring ("pinned" = fixed by CPU tests against something other
than itself).
"""
from .attention import tree_attention, ancestors, path_to_root  # noqa: F401
from .accept import (AcceptResult, accept_tree, keep_probability, remove_draft_mass,  # noqa: F401
                     target_distribution, sample_inverse_cdf, draft_p_to_target, filter_keep,
                     terminal_distribution, TIE_BAND, SAMPLE_BAND, FILTER_BAND,
                     DEGENERATE_BAND)
from .commit import kv_commit, kv_commit_from_buffer  # noqa: F401
from .tree import TreeBuilder, build_tree  # noqa: F401
from .rope import rope_rotate, node_positions, tree_kv_write  # noqa: F401
from . import paged  # noqa: F401
from .validate import validate_tree, ERR_TREE, ERR_TOKEN, ERR_NONFINITE, ERR_CAPACITY  # noqa: F401
