"""EAGLE-2/3 tree verification on AMD MI355X (gfx950).

The verify step of speculative decoding with draft trees, as hand-written HIP
kernels behind a C ABI (include/spec_verify.h):

  * spec_verify_tree_attn -- tree-masked attention of every draft node over
    the committed prefix KV plus its own ancestors;
  * spec_accept_tree      -- the Leviathan acceptance rule walked down the tree
    (greedy at T = 0, residual resampling and bonus token at T > 0);
  * spec_kv_commit        -- gathers the accepted path's KV rows behind the
    prefix and advances the logical length.

`api` is the thin Python binding (argument marshalling only; it loads the
shared library and fails loudly when it is missing).  `workloads` draws the
seeded synthetic inputs used by tests and the benchmark.
"""
__all__ = ["api", "workloads"]
