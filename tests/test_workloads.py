"""Checks of the seeded input generator (CPU only)."""
import numpy as np
import pytest

from eagle_tree_verification_amd import workloads as W


def _levels(parents):
    return W.node_depths(np.asarray(parents))


@pytest.mark.parametrize("drafts,depth", [(60, 6), (60, 8), (50, 8), (48, 8), (5, 5), (9, 1)])
def test_tree_shape_rules(drafts, depth):
    rng = np.random.default_rng(drafts * 31 + depth)
    for _ in range(5):
        p = W.tree_shape(drafts, depth, rng)
        assert len(p) == drafts + 1 and p[0] == -1
        assert all(0 <= p[j] < j for j in range(1, len(p)))
        dep = _levels(p)
        assert dep.max() == depth
        # every level has a node; at most 10 children per node; at most 10 expanded per level
        for lv in range(1, depth + 1):
            kids = p[dep == lv]
            assert len(kids) >= 1
            assert len(np.unique(kids)) <= 10
            assert np.bincount(kids).max() <= 10
        # ids grow with depth
        assert np.all(np.diff(dep) >= 0)


def test_workload_is_deterministic_and_well_formed():
    a = W.make_workload(4, batch=3, prefix=(10, 90), vocab=777)
    b = W.make_workload(4, batch=3, prefix=(10, 90), vocab=777)
    for f in ("q", "k_cache", "v_cache", "prefix_len", "parents", "tokens", "logits",
              "draft_p", "u_accept", "u_sample"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert a.q.dtype == np.uint16 and a.k_cache.shape == (3, 8, a.L_cap, 128)
    assert a.L_cap >= a.prefix_len.max() + a.n_max and a.L_cap % 64 == 0
    assert np.all((a.tokens[:, 1:] >= 0) & (a.tokens[:, 1:] < a.V))
    assert np.all((a.u_accept >= 0) & (a.u_accept < 1))
    np.testing.assert_allclose(a.draft_p.sum(-1), 1.0, atol=1e-5)
    assert a.max_depth == 8


def test_poison_marks_unread_rows():
    w = W.make_workload(4, batch=2, prefix=(5, 40), vocab=300, drafts=[10, 20], poison=True)
    for b in range(2):
        rows = w.prefix_len[b] + w.n_nodes[b]
        k = W.bf16_bits_to_f32(w.k_cache[b])
        assert np.isnan(k[:, rows:]).all() and np.isfinite(k[:, :rows]).all()
        assert np.isnan(w.logits[b, w.n_nodes[b]:]).all()
        assert np.isnan(W.bf16_bits_to_f32(w.q[b, w.n_nodes[b]:])).all()


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.5, 3.0e38, 1e-40], np.float32)
    back = W.bf16_bits_to_f32(W.f32_to_bf16_bits(x))
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0)
    assert back[1] == 1.0
    assert back[2] == np.float32(1.0078125)
    assert back[0] == 1.0 and back[3] == -2.5
    assert np.isfinite(back[4])


def test_noise_calibration_hits_target_overlap():
    rng = np.random.default_rng(0)
    V = 20000
    sig = W.calibrate_noise([0.6, 0.8, 0.9], V, 3.0, np.random.default_rng(1))
    assert np.all(np.diff(sig) < 0)
    for target, s in zip([0.6, 0.8, 0.9], sig):
        l = rng.normal(0, 3.0, size=(32, V))
        q = W._softmax_rows64(l)
        p = W._softmax_rows64(l + s * rng.standard_normal(size=(32, V)))
        assert abs(W._overlap(p, q) - target) < 0.02
