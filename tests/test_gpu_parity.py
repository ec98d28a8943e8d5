"""GPU parity of the three C-ABI calls against the oracle on reduced configs.

Each case keeps its config's head layout, head dim, dtype and tree budget but
shrinks the prefix and vocabulary so the oracle finishes in seconds; all still
span several 64-key tiles with a ragged tail.  Inputs are poisoned with NaN
everywhere the path must not read.  Bars: attention within 1e-5 (f32) /
2e-2 (bf16) absolute; accepted lengths, paths, emitted tokens and committed KV
bit-exact except a near tie the oracle confirms (at most one sequence per
case, itself checked for a valid walk); residual distributions within 1e-5
absolute.
"""
import numpy as np
import pytest
import torch

from eagle_tree_verification_amd.workloads import make_workload, small_cases, to_device
import oracle
from gpu_helpers import (SENTINEL, compare_accept, compare_attention, compare_commit, kv_host,
                         oracle_accept, run_gpu_step, say)

pytestmark = pytest.mark.gpu

CASES = small_cases()


@pytest.mark.parametrize("name", list(CASES))
def test_step_parity(hip_lib, name):
    w = make_workload(poison=True, **CASES[name])
    say(f"[gpu] step parity {name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} d={w.d} "
        f"L={w.prefix_len.tolist()} n={w.n_nodes.tolist()} V={w.V} T={w.T}")
    dev = to_device(w)
    host = run_gpu_step(w, dev)
    assert host["dev_error"] == 0
    worst = compare_attention(w, host["attn"])
    excluded = compare_accept(w, host)
    say(f"[gpu]   attention max|diff|={worst:.3g}; near-tie sequences excluded: {excluded}")
    compare_commit(w, host, kv_host(dev["k_cache"], w.kv_dtype), kv_host(dev["v_cache"], w.kv_dtype),
                   dev["prefix_len"].cpu().numpy())


@pytest.mark.parametrize("T", [0.0, 0.7, 1.0, 2.5])
def test_ragged_trees_and_temperatures(hip_lib, T):
    # ragged n_nodes (including a single-root tree), empty and tiny prefixes
    w = make_workload(4, batch=6, prefix=(0, 150), vocab=2053, drafts=[60, 1, 0, 17, 33, 8],
                      T=T, poison=True, seed=77, prefix_lens=[0, 1, 63, 64, 150, 97])
    say(f"[gpu] ragged T={T} L={w.prefix_len.tolist()} n={w.n_nodes.tolist()}")
    dev = to_device(w)
    host = run_gpu_step(w, dev)
    assert host["dev_error"] == 0
    compare_attention(w, host["attn"])
    compare_accept(w, host)
    compare_commit(w, host, kv_host(dev["k_cache"], w.kv_dtype), kv_host(dev["v_cache"], w.kv_dtype),
                   dev["prefix_len"].cpu().numpy())


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_maximum_trees(hip_lib, T):
    """The largest trees the ABI takes (64 nodes): a 63-deep chain, a root
    with 63 children, a random depth-8 tree and a binary tree, over prefixes
    from 0 to 8000 keys (so the attention splits its prefix), at the serving
    head layout."""
    from eagle_tree_verification_amd.workloads import tree_shape
    rng = np.random.default_rng(64)
    chain = np.arange(-1, 63, dtype=np.int32)
    star = np.array([-1] + [0] * 63, dtype=np.int32)
    rand = tree_shape(63, 8, rng).astype(np.int32)
    binary = np.array([-1] + [(j - 1) // 2 for j in range(1, 64)], dtype=np.int32)
    pars = [chain, star, rand, binary]
    w = make_workload(4, batch=4, prefix=(0, 8000), vocab=4099, T=T, poison=True, seed=641,
                      parents=pars, prefix_lens=[8000, 0, 4097, 1])
    say(f"[gpu] maximum trees T={T}: n={w.n_nodes.tolist()} depth={w.max_depth} "
        f"L={w.prefix_len.tolist()}")
    assert w.n_max == 64 and int(w.n_nodes.max()) == 64
    dev = to_device(w)
    host = run_gpu_step(w, dev)
    assert host["dev_error"] == 0
    compare_attention(w, host["attn"], nodes_per_seq=12, rng=np.random.default_rng(1))
    compare_accept(w, host)
    compare_commit(w, host, kv_host(dev["k_cache"], w.kv_dtype), kv_host(dev["v_cache"], w.kv_dtype),
                   dev["prefix_len"].cpu().numpy())


@pytest.mark.parametrize("hq,hkv,d,dt", [(4, 4, 16, "f32"), (8, 2, 64, "bf16"), (6, 3, 32, "f32"),
                                         (16, 16, 128, "f32"), (12, 4, 128, "bf16"),
                                         (4, 1, 128, "bf16"), (8, 1, 128, "bf16")])
def test_attention_layouts(hip_lib, hq, hkv, d, dt):
    w = make_workload(4, batch=3, prefix=(70, 200), vocab=64, hq=hq, hkv=hkv, head_dim=d,
                      kv_dtype=dt, poison=True, seed=hq * 100 + d)
    say(f"[gpu] attention layout hq={hq} hkv={hkv} d={d} {dt}")
    dev = to_device(w)
    host = run_gpu_step(w, dev, commit=False)
    compare_attention(w, host["attn"])


@pytest.mark.parametrize("splits", [1, 2, 3, 7])
def test_forced_prefix_splits(hip_lib, monkeypatch, splits):
    """SPEC_ATTN_SPLITS forces the number of prefix splits (merged by
    log-sum-exp); every count, odd ones included, must give the oracle's
    attention, on one KV head per sequence (the tensor-parallel share's
    layout) with ragged prefixes and a tree-only sequence."""
    api = hip_lib
    w = make_workload(4, batch=5, prefix=(0, 1500), vocab=64, hq=4, hkv=1, poison=True, seed=600 + splits,
                      prefix_lens=[0, 1, 200, 777, 1500])
    say(f"[gpu] forced splits {splits}: n={w.n_nodes.tolist()} L={w.prefix_len.tolist()}")
    monkeypatch.setenv("SPEC_ATTN_SPLITS", str(splits))
    dev = to_device(w)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.full((w.B, w.n_max, w.Hq, w.d), SENTINEL, dtype=torch.float32, device="cuda")
    api.verify_tree_attn(dev["q"], dev["k_cache"], dev["v_cache"], dev["prefix_len"],
                         dev["n_nodes"], dev["parents"], out=out, dev_error=err)
    torch.cuda.synchronize()
    monkeypatch.delenv("SPEC_ATTN_SPLITS")
    assert int(err.item()) == 0
    compare_attention(w, out.cpu().numpy())


@pytest.mark.parametrize("rope", [False, True])
def test_pipelined_order_is_bit_identical(hip_lib, monkeypatch, rope):
    """The two-sub-tile attention kernel runs in a pipelined order by default
    (a sub-tile's PV product interleaved with the next sub-tile's softmax);
    SPEC_ATTN_PIPE=0 selects the plain order.  The operations on O keep their
    order, so every output bit must agree: stages of one and of two
    sub-tiles, a tree-only pass (empty prefix), single-node trees, and
    prefixes long enough to be split over several workgroups."""
    api = hip_lib
    w = make_workload(4, batch=8, prefix=(0, 8000), vocab=64, drafts=[63, 0, 40, 63, 5, 63, 33, 63],
                      poison=True, seed=515, prefix_lens=[0, 1, 64, 127, 128, 129, 4097, 8000])
    say(f"[gpu] pipelined vs plain order rope={rope}: n={w.n_nodes.tolist()} "
        f"L={w.prefix_len.tolist()}")
    assert w.n_max * (w.Hq // w.Hkv) > 128          # the two-sub-tile kernel
    dev = to_device(w)
    f = (torch.from_numpy((500000.0 ** (-np.arange(w.d // 2) * 2.0 / w.d)).astype(np.float32)).cuda()
         if rope else None)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    outs = []
    for pipe in ("1", "0"):
        monkeypatch.setenv("SPEC_ATTN_PIPE", pipe)
        out = torch.full((w.B, w.n_max, w.Hq, w.d), SENTINEL, dtype=torch.float32, device="cuda")
        api.verify_tree_attn(dev["q"], dev["k_cache"], dev["v_cache"], dev["prefix_len"],
                             dev["n_nodes"], dev["parents"], out=out, dev_error=err, inv_freq=f)
        torch.cuda.synchronize()
        outs.append(out)
    monkeypatch.delenv("SPEC_ATTN_PIPE")
    assert int(err.item()) == 0
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
    if not rope:
        compare_attention(w, outs[0].cpu().numpy(), nodes_per_seq=8, rng=np.random.default_rng(5))


@pytest.mark.parametrize("T", [0.0, 1.0])
@pytest.mark.parametrize("vocab", [500, 32000])
def test_first_child_rows_read_ahead(hip_lib, vocab, T):
    """With short slices a node's statistics pass (T > 0) also covers its
    first child's row.  A NaN there fails the sequence only if the walk enters
    that child, as when every row is read at its own visit: NaN in an entered
    node's row (even sequences) and in a first child the walk passes over (odd
    ones).  T = 0 checks the same for the greedy walk, which reads each row at
    its own visit."""
    w = make_workload(4, batch=8, prefix=(20, 40), vocab=vocab, poison=False, seed=11, T=T)
    say(f"[gpu] first-child rows read ahead: V={w.V} T={T}")
    entered, passed = [], []
    for b in range(w.B):
        r = oracle_accept(w, b)
        path = [int(x) for x in r.path[: r.accept_len + 1]]
        n = int(w.n_nodes[b])
        if b % 2 == 0 and len(path) > 1:
            w.logits[b, path[1], 7] = np.nan
            entered.append(b)
            continue
        for d, v in enumerate(path):
            kids = [c for c in range(v + 1, n) if w.parents[b, c] == v]
            if kids and (d + 1 == len(path) or path[d + 1] != kids[0]):
                w.logits[b, kids[0], 7] = np.nan
                passed.append(b)
                break
    assert len(entered) >= 2 and len(passed) >= 2, (entered, passed)
    dev = to_device(w)
    host = run_gpu_step(w, dev, commit=False)
    from eagle_tree_verification_amd import api
    assert host["dev_error"] == api.DEVERR_NONFINITE
    assert all(host["accept_len"][b] == -1 for b in entered)
    assert all(host["accept_len"][b] >= 0 for b in passed)
    compare_accept(w, host)


def test_device_errors_are_reported(hip_lib):
    w = make_workload(4, batch=4, prefix=(20, 40), vocab=500, poison=False, seed=5)
    w.parents[0, 5] = 7          # parent after child: bad tree
    w.tokens[1, 3] = w.V         # token out of range
    w.logits[2, 0, 10] = np.nan  # the root row is always read
    w.prefix_len[3] = w.L_cap - 2  # tree does not fit
    say("[gpu] device error bits")
    dev = to_device(w)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.full((w.B, w.n_max, w.Hq, w.d), -7.0, device="cuda")
    from eagle_tree_verification_amd import api
    api.verify_tree_attn(dev["q"], dev["k_cache"], dev["v_cache"], dev["prefix_len"],
                         dev["n_nodes"], dev["parents"], out=out, dev_error=err)
    torch.cuda.synchronize()
    assert int(err.item()) == api.DEVERR_TREE | api.DEVERR_CAPACITY
    assert torch.all(out[0] == -7.0) and torch.all(out[3] == -7.0)
    err.zero_()
    acc = api.accept_tree(dev["tokens"], dev["parents"], dev["n_nodes"], dev["draft_p"],
                          dev["logits"], 1.0, dev["u_accept"], dev["u_sample"], w.max_depth,
                          dev_error=err)
    torch.cuda.synchronize()
    assert int(err.item()) == api.DEVERR_TREE | api.DEVERR_TOKEN | api.DEVERR_NONFINITE
    al = acc["accept_len"].cpu().numpy()
    assert list(al[:3]) == [-1, -1, -1] and al[3] >= 0
    assert np.all(acc["path"][:3].cpu().numpy() == -1)
    # the commit skips failed sequences; the fourth one overflows the cache
    before = dev["prefix_len"].clone()
    err.zero_()
    api.kv_commit(dev["k_cache"], dev["v_cache"], dev["prefix_len"], acc["path"], acc["accept_len"],
                  w.max_depth, dev_error=err)
    torch.cuda.synchronize()
    after = dev["prefix_len"].cpu().numpy()
    assert np.all(after[:3] == before[:3].cpu().numpy())


def test_host_errors_are_returned(hip_lib):
    from eagle_tree_verification_amd import api
    w = make_workload(1, T=1.0)
    dev = to_device(w)
    with pytest.raises(api.SpecError) as e:
        api.accept_tree(dev["tokens"], dev["parents"], dev["n_nodes"], dev["draft_p"], dev["logits"],
                        -1.0, dev["u_accept"], dev["u_sample"], w.max_depth)
    assert e.value.status == -4
    with pytest.raises(api.SpecError) as e:
        api.verify_tree_attn(dev["q"], dev["k_cache"], dev["v_cache"], dev["prefix_len"],
                             dev["n_nodes"], dev["parents"], scale=0.0)
    assert e.value.status == -4


def test_commit_in_place_hazard(hip_lib):
    # path [0, 2, 5]: row 2 is read for slot 1 and overwritten by slot 2
    from eagle_tree_verification_amd import api
    B, Hkv, L_cap, d, L = 2, 3, 64, 128, 9
    rng = np.random.default_rng(0)
    k = torch.from_numpy(rng.standard_normal((B, Hkv, L_cap, d), dtype=np.float32)).cuda()
    v = torch.from_numpy(rng.standard_normal((B, Hkv, L_cap, d), dtype=np.float32)).cuda()
    k0, v0 = k.clone(), v.clone()
    plen = torch.tensor([L, L], dtype=torch.int32, device="cuda")
    path = torch.tensor([[0, 2, 5, -1], [0, 1, 2, 3]], dtype=torch.int32, device="cuda")
    alen = torch.tensor([2, 3], dtype=torch.int32, device="cuda")
    say("[gpu] commit hazard")
    api.kv_commit(k, v, plen, path, alen, 3)
    torch.cuda.synchronize()
    for src, dst in ((0, 0), (2, 1), (5, 2)):
        assert torch.equal(k[0, :, L + dst], k0[0, :, L + src])
        assert torch.equal(v[0, :, L + dst], v0[0, :, L + src])
    assert torch.equal(k[1], k0[1]) and torch.equal(v[1], v0[1])
    assert plen.cpu().tolist() == [L + 3, L + 4]


def test_accept_wait_bound_reports_sync(hip_lib, monkeypatch):
    """A host-set negative wait bound makes every vocabulary exchange give up:
    the call must end normally with SPEC_DEVERR_SYNC set and the failed
    sequences marked.  The remedy the header gives, the same call repeated
    with the cooperative launch, and then an ordinary call, both with the
    default bound on the same workspace, must be exact again."""
    import torch
    from eagle_tree_verification_amd import api
    w = make_workload(4, batch=8, prefix=(64, 64), vocab=128256, drafts=12, depth=4, seed=5)
    dev = to_device(w)
    ws = torch.empty(api.accept_tree_workspace_size(w.B, w.n_max, w.V), dtype=torch.uint8,
                     device="cuda")
    say(f"[gpu] wait bound: B={w.B} V={w.V}, forced give-up then default")

    def call(launch="ordinary"):
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        r = api.accept_tree(dev["tokens"], dev["parents"], dev["n_nodes"], dev["draft_p"],
                            dev["logits"], w.T, dev["u_accept"], dev["u_sample"], w.max_depth,
                            workspace=ws, dev_error=err, launch=launch)
        torch.cuda.synchronize()
        return r, int(err.item())

    monkeypatch.setenv("SPEC_ACCEPT_SPIN_LIMIT", "-1")
    r0, e0 = call()
    assert e0 & api.DEVERR_SYNC, e0
    assert (r0["accept_len"].cpu().numpy() == -1).all()
    monkeypatch.delenv("SPEC_ACCEPT_SPIN_LIMIT")
    for launch in ("cooperative", "ordinary"):
        r, e1 = call(launch)
        assert e1 == 0, launch
        host = {k: v.cpu().numpy() for k, v in r.items() if isinstance(v, torch.Tensor)}
        host["ties"] = np.zeros(0, dtype=api.TIE_DTYPE)
        host["final_dist"] = None
        compare_accept(w, host)


def _layer_setup(nl, seed):
    """A ragged batch, its oracle walk, and nl per-layer caches and scratch
    buffers (random storage patterns: the commit copies bytes)."""
    import torch
    w = make_workload(4, batch=6, prefix=(0, 150), vocab=2053, drafts=[60, 1, 0, 17, 33, 8],
                      T=1.0, seed=seed, prefix_lens=[0, 1, 63, 64, 150, 97])
    D = w.max_depth
    path = np.full((w.B, D + 1), -1, dtype=np.int32)
    acc = np.full(w.B, -1, dtype=np.int32)
    for b in range(w.B):
        r = oracle_accept(w, b)
        acc[b] = r.accept_len
        path[b, : r.accept_len + 1] = r.path
    rng = np.random.default_rng(seed)
    shape_c = w.k_cache.shape
    shape_t = (w.B, w.Hkv, w.n_max, w.d)
    kc = [rng.integers(0, 1 << 16, size=shape_c, dtype=np.uint16) for _ in range(nl)]
    vc = [rng.integers(0, 1 << 16, size=shape_c, dtype=np.uint16) for _ in range(nl)]
    kt = [rng.integers(0, 1 << 16, size=shape_t, dtype=np.uint16) for _ in range(nl)]
    vt = [rng.integers(0, 1 << 16, size=shape_t, dtype=np.uint16) for _ in range(nl)]
    dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return w, path, acc, kc, vc, kt, vt, dev


@pytest.mark.parametrize("scratch", [False, True], ids=["in-place", "scratch"])
def test_commit_layers_parity(hip_lib, scratch):
    import torch
    from eagle_tree_verification_amd import api
    nl = 5
    w, path, acc, kc, vc, kt, vt, dev = _layer_setup(nl, 31)
    say(f"[gpu] commit_layers {'scratch' if scratch else 'in-place'}: layers={nl} "
        f"accept_len={acc.tolist()}")
    kd, vd = [dev(a) for a in kc], [dev(a) for a in vc]
    td = ([dev(a) for a in kt], [dev(a) for a in vt]) if scratch else (None, None)
    plen = torch.from_numpy(w.prefix_len.copy()).cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    api.kv_commit_layers(kd, vd, plen, torch.from_numpy(path).cuda(), torch.from_numpy(acc).cuda(),
                         w.max_depth, k_tree=td[0], v_tree=td[1], dev_error=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    np.testing.assert_array_equal(plen.cpu().numpy(), w.prefix_len + acc + 1)
    for l in range(nl):
        kg = kd[l].view(torch.int16).cpu().numpy().view(np.uint16)
        vg = vd[l].view(torch.int16).cpu().numpy().view(np.uint16)
        for b in range(w.B):
            a, L = int(acc[b]), int(w.prefix_len[b])
            if scratch:
                k2, v2, _ = oracle.kv_commit_from_buffer(kc[l][b], vc[l][b], kt[l][b], vt[l][b], L,
                                                         path[b, : a + 1], a)
            else:
                k2, v2, _ = oracle.kv_commit(kc[l][b], vc[l][b], L, path[b, : a + 1], a)
            np.testing.assert_array_equal(kg[b], k2)
            np.testing.assert_array_equal(vg[b], v2)


@pytest.mark.parametrize("which", ["cache", "scratch"])
def test_commit_layers_misaligned_layer(hip_lib, which):
    """One layer buffer 2 bytes off 16-byte alignment (a cache in the in-place
    form, a scratch buffer in the other): the kernels refuse the whole call,
    so no layer of any sequence changes, no length advances, and
    SPEC_DEVERR_ALIGN is set.  The misaligned pointer is only compared, never
    dereferenced; its buffer is an in-bounds view of a larger allocation."""
    import torch
    from eagle_tree_verification_amd import api
    nl = 3
    w, path, acc, kc, vc, kt, vt, dev = _layer_setup(nl, 53)
    say(f"[gpu] commit_layers: misaligned {which} buffer of layer 1")

    def shifted(a):  # the same contents at an address 2 bytes past 16-byte alignment
        t = dev(a)
        backing = torch.empty(t.numel() + 8, dtype=t.dtype, device="cuda")
        view = backing[1:1 + t.numel()].view(t.shape)
        view.copy_(t)
        assert view.data_ptr() % 16 == 2
        return view

    kd, vd = [dev(a) for a in kc], [dev(a) for a in vc]
    td = None
    if which == "cache":
        kd[1] = shifted(kc[1])
    else:
        td = ([dev(a) for a in kt], [dev(a) for a in vt])
        td[1][1] = shifted(vt[1])
    plen = torch.from_numpy(w.prefix_len.copy()).cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    api.kv_commit_layers(kd, vd, plen, torch.from_numpy(path).cuda(), torch.from_numpy(acc).cuda(),
                         w.max_depth, k_tree=None if td is None else td[0],
                         v_tree=None if td is None else td[1], dev_error=err)
    torch.cuda.synchronize()
    assert int(err.item()) == api.DEVERR_ALIGN
    np.testing.assert_array_equal(plen.cpu().numpy(), w.prefix_len)
    for l in range(nl):
        np.testing.assert_array_equal(kd[l].view(torch.int16).cpu().numpy().view(np.uint16), kc[l])
        np.testing.assert_array_equal(vd[l].view(torch.int16).cpu().numpy().view(np.uint16), vc[l])


def test_commit_layers_bad_path_and_forms_agree(hip_lib):
    import torch
    from eagle_tree_verification_amd import api
    nl = 3
    w, path, acc, kc, vc, kt, vt, dev = _layer_setup(nl, 47)
    b_bad = int(np.argmax(acc))
    assert acc[b_bad] >= 1
    bad = path.copy()
    bad[b_bad, 1] = bad[b_bad, 0]  # not increasing
    say(f"[gpu] commit_layers: corrupted path of sequence {b_bad}; scratch form on cache rows")
    # scratch rows taken from the caches' own tree rows: both forms must agree
    for l in range(nl):
        for b in range(w.B):
            L, n = int(w.prefix_len[b]), int(w.n_nodes[b])
            kt[l][b, :, :n] = kc[l][b, :, L:L + n]
            vt[l][b, :, :n] = vc[l][b, :, L:L + n]
    outs = []
    for use_scratch in (False, True):
        kd, vd = [dev(a) for a in kc], [dev(a) for a in vc]
        td = ([dev(a) for a in kt], [dev(a) for a in vt]) if use_scratch else (None, None)
        plen = torch.from_numpy(w.prefix_len.copy()).cuda()
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        api.kv_commit_layers(kd, vd, plen, torch.from_numpy(bad).cuda(),
                             torch.from_numpy(acc).cuda(), w.max_depth, k_tree=td[0],
                             v_tree=td[1], dev_error=err)
        torch.cuda.synchronize()
        assert int(err.item()) & api.DEVERR_TREE
        lens = plen.cpu().numpy()
        assert lens[b_bad] == w.prefix_len[b_bad]
        ok = np.arange(w.B) != b_bad
        np.testing.assert_array_equal(lens[ok], (w.prefix_len + acc + 1)[ok])
        got = [(k.view(torch.int16).cpu().numpy(), v.view(torch.int16).cpu().numpy())
               for k, v in zip(kd, vd)]
        for l in range(nl):  # the failed sequence is untouched in every layer
            np.testing.assert_array_equal(got[l][0][b_bad].view(np.uint16), kc[l][b_bad])
            np.testing.assert_array_equal(got[l][1][b_bad].view(np.uint16), vc[l][b_bad])
        outs.append((got, lens))
    for l in range(nl):
        for b in range(w.B):
            rows = int(w.prefix_len[b]) + int(acc[b]) + 1
            np.testing.assert_array_equal(outs[0][0][l][0][b][:, :rows], outs[1][0][l][0][b][:, :rows])
            np.testing.assert_array_equal(outs[0][0][l][1][b][:, :rows], outs[1][0][l][1][b][:, :rows])
