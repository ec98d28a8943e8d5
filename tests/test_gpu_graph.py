"""The verify step captured into a HIP graph and replayed.

The library's calls launch kernels only (no memset, no allocation, no host
synchronisation), so a caller can capture a whole step.  Each case captures
attention, the acceptance walk and the commit once, then replays the graph
three times, each time on new uniforms (and so new walks): before every
replay the caches and lengths are restored and the new uniforms copied in by
eager copies, the eagerly issued step on the same inputs gives the
reference, and an eager call of the walk runs on the same stream; after
every replay every output (attention rows, walk outputs, committed caches
and lengths, tie records) must equal the eager step's bit for bit.  A replay
repeats the host's launch ids, so this also shows that no exchange word a
previous launch left in the workspace is taken for a current one.  The
eager steps are checked against the oracle.
"""
import numpy as np
import pytest
import torch

from eagle_tree_verification_amd.workloads import make_workload, small_cases, to_device
from gpu_helpers import SENTINEL, compare_accept, compare_attention, say

pytestmark = pytest.mark.gpu


def _step(api, w, dev, bufs, *, noalloc=False, filters=None):
    api.verify_tree_attn(dev["q"], dev["k_cache"], dev["v_cache"], dev["prefix_len"],
                         dev["n_nodes"], dev["parents"], out=bufs["out"],
                         workspace=bufs["ws_attn"], dev_error=bufs["err"])
    kw = {}
    if filters is not None:
        kw = dict(top_k=filters[0], top_p=filters[1], workspace=bufs["ws_acc_ex"])
    elif not noalloc:
        kw = dict(workspace=bufs["ws_acc"])
    res = api.accept_tree(dev["tokens"], dev["parents"], dev["n_nodes"], dev["draft_p"],
                          dev["logits"], w.T, dev["u_accept"], dev["u_sample"], w.max_depth,
                          final_dist=True, tie_cap=64, dev_error=bufs["err"],
                          outputs=bufs["outs"], noalloc=noalloc, **kw)
    api.kv_commit(dev["k_cache"], dev["v_cache"], dev["prefix_len"], res["path"],
                  res["accept_len"], w.max_depth, dev_error=bufs["err"])
    return res


def _snapshot(bufs, res, dev):
    snap = {"out": bufs["out"].clone(), "err": bufs["err"].clone(),
            "k": dev["k_cache"].clone(), "v": dev["v_cache"].clone(),
            "len": dev["prefix_len"].clone()}
    for k in ("accept_len", "path", "out_tokens", "n_out", "final_dist", "tie_log", "tie_count"):
        snap[k] = res[k].clone()
    return snap


@pytest.mark.parametrize("case", ["plain", "noalloc", "filters", "tiny-trees"])
def test_step_graph_replays_match_eager(hip_lib, case):
    """tiny-trees: root-only and two- or three-node trees, whose walks make one
    to three exchanges, with new logits as well as new uniforms each replay
    (a launch whose tags repeated the previous one's could then take that
    launch's words for its own first exchanges)."""
    api = hip_lib
    kw = dict(small_cases()["c4-mini"])
    if case == "tiny-trees":
        kw["drafts"] = [0, 1, 0, 2, 0]
    w = make_workload(poison=True, **kw)
    dev = to_device(w)
    say(f"[gpu] graph of the verify step ({case}): B={w.B} V={w.V} n_max={w.n_max}")
    kv_dt = api.SPEC_BF16 if w.kv_dtype == "bf16" else api.SPEC_F32
    bufs = {
        "out": torch.full((w.B, w.n_max, w.Hq, w.d), SENTINEL, dtype=torch.float32, device="cuda"),
        "ws_attn": torch.empty(max(1, api.verify_tree_attn_workspace_size(
            w.B, w.n_max, w.Hq, w.Hkv, w.d, w.L_cap, kv_dt)), dtype=torch.uint8, device="cuda"),
        "ws_acc": torch.empty(api.accept_tree_workspace_size(w.B, w.n_max, w.V),
                              dtype=torch.uint8, device="cuda"),
        "ws_acc_ex": torch.empty(api.accept_tree_ex_workspace_size(w.B, w.n_max, w.V, 0, True),
                                 dtype=torch.uint8, device="cuda"),
        "err": torch.zeros(1, dtype=torch.int32, device="cuda"),
        "outs": {"accept_len": torch.empty(w.B, dtype=torch.int32, device="cuda"),
                 "path": torch.empty((w.B, w.max_depth + 1), dtype=torch.int32, device="cuda"),
                 "out_tokens": torch.empty((w.B, w.max_depth + 1), dtype=torch.int32,
                                           device="cuda"),
                 "n_out": torch.empty(w.B, dtype=torch.int32, device="cuda")},
    }
    filters = None
    if case == "filters":
        filters = (torch.tensor([0, 5, 50, 1, 0][: w.B], dtype=torch.int32, device="cuda"),
                   torch.tensor([0.9, 0.0, 0.8, 0.0, 0.5][: w.B], dtype=torch.float32,
                                device="cuda"))
    noalloc = case == "noalloc"
    k0, v0, len0 = dev["k_cache"].clone(), dev["v_cache"].clone(), dev["prefix_len"].clone()

    def restore():
        dev["k_cache"].copy_(k0)
        dev["v_cache"].copy_(v0)
        dev["prefix_len"].copy_(len0)
        bufs["err"].zero_()

    rng = np.random.default_rng(1234)
    u_sets = [(dev["u_accept"].clone(), dev["u_sample"].clone(), dev["logits"].clone())]
    for _ in range(3):
        lg = w.logits
        if case == "tiny-trees":  # the same values at other token ids
            lg = np.ascontiguousarray(lg[:, :, rng.permutation(w.V)])
        u_sets.append((torch.from_numpy(rng.random(w.u_accept.shape, dtype=np.float32)).cuda(),
                       torch.from_numpy(rng.random(w.u_sample.shape, dtype=np.float32)).cuda(),
                       torch.from_numpy(lg).cuda()))

    def use(k):
        dev["u_accept"].copy_(u_sets[k][0])
        dev["u_sample"].copy_(u_sets[k][1])
        dev["logits"].copy_(u_sets[k][2])

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        eager = []
        for k in range(4):
            restore()
            use(k)
            res = _step(api, w, dev, bufs, noalloc=noalloc, filters=filters)
            torch.cuda.synchronize()
            eager.append(_snapshot(bufs, res, dev))
            assert int(eager[k]["err"].item()) == 0
        restore()
        use(0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            gres = _step(api, w, dev, bufs, noalloc=noalloc, filters=filters)
        torch.cuda.synchronize()
        changed = 0
        for r in range(1, 4):
            restore()
            use(r)
            # the program's own eager work between replays: a walk on the same stream
            api.accept_tree(dev["tokens"], dev["parents"], dev["n_nodes"], dev["draft_p"],
                            dev["logits"], w.T, dev["u_accept"], dev["u_sample"], w.max_depth,
                            dev_error=bufs["err"])
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = _snapshot(bufs, gres, dev)
            ref = eager[r]
            for key, val in ref.items():
                if key == "tie_log":  # records append in any order: compared as sets below
                    continue
                # bytes, so that the NaN the poisoned cache rows hold compare equal
                assert torch.equal(got[key].contiguous().view(torch.uint8),
                                   val.contiguous().view(torch.uint8)), (
                    f"replay {r}: {key} differs from the eager step on the same inputs")
            tie_key = lambda t: (int(t["b"]), int(t["node"]), int(t["kind"]))
            assert (sorted(map(tie_key, api.decode_ties(got["tie_log"], got["tie_count"])))
                    == sorted(map(tie_key, api.decode_ties(ref["tie_log"], ref["tie_count"]))))
            changed += not torch.equal(ref["out_tokens"], eager[r - 1]["out_tokens"])
            say(f"[gpu]   replay {r}: every output equals the eager step's")
        assert changed >= 2, "the new uniforms should change the walks"

    # the eager step on the workload's own uniforms against the oracle
    host = {key: eager[0][key].cpu().numpy() for key in ("accept_len", "path", "out_tokens",
                                                         "n_out", "final_dist")}
    host["ties"] = api.decode_ties(eager[0]["tie_log"], eager[0]["tie_count"])
    if filters is None:
        compare_accept(w, host)
    compare_attention(w, eager[0]["out"].cpu().numpy())
