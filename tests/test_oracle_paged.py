"""Pins for the oracle's paged-cache view (CPU only): a block table worked by
hand, the identity table, round trips through random tables, and writes
confined to the rows written."""
import numpy as np

from oracle import paged


def test_table_by_hand():
    # 3 blocks of 2 rows, 1 head, d = 1; pool value = 10 * block + row
    pool = np.array([[[[0.0], [1.0]]], [[[10.0], [11.0]]], [[[20.0], [21.0]]]])
    assert pool.shape == (3, 1, 2, 1)
    # logical blocks 0, 1, 2 -> physical 2, 0, 1: logical rows read
    # 20 21 | 0 1 | 10 11
    got = paged.logical_rows(pool, [2, 0, 1], 2, 6)
    np.testing.assert_array_equal(got[0, :, 0], [20, 21, 0, 1, 10, 11])
    # a ragged view stops inside a block
    np.testing.assert_array_equal(paged.logical_rows(pool, [1, 2], 2, 3)[0, :, 0], [10, 11, 20])
    # writing logical rows 1..3 of table [2, 0]: pool (2, row 1), (0, rows 0-1)
    cache = np.full((1, 4, 1), -1.0)
    cache[0, :, 0] = [100, 101, 102, 103]
    new = paged.write_rows(pool, [2, 0], 2, cache, 1, 4)
    np.testing.assert_array_equal(new[:, 0, :, 0], [[102, 103], [10, 11], [20, 101]])
    assert paged.blocks_valid([2, 0], 2, 4, 3)
    assert not paged.blocks_valid([2, 3], 2, 4, 3)        # block 3 does not exist
    assert not paged.blocks_valid([2], 2, 3, 3)           # table too short
    assert paged.blocks_valid([2, -1], 2, 2, 3)           # rows 0-1 need block 0 only


def test_identity_table_is_a_reshape():
    rng = np.random.default_rng(0)
    nb, h, bs, d = 5, 3, 4, 2
    pool = rng.normal(size=(nb, h, bs, d))
    got = paged.logical_rows(pool, np.arange(nb), bs, nb * bs)
    want = np.transpose(pool, (1, 0, 2, 3)).reshape(h, nb * bs, d)
    np.testing.assert_array_equal(got, want)


def test_round_trip_and_confined_writes():
    rng = np.random.default_rng(1)
    nb, h, bs, d = 12, 2, 8, 3
    pool = rng.normal(size=(nb, h, bs, d))
    table = rng.permutation(nb)[:5]
    rows = 37
    view = paged.logical_rows(pool, table, bs, rows)
    # writing the view back changes nothing
    np.testing.assert_array_equal(paged.write_rows(pool, table, bs, view, 0, rows), pool)
    # a write of rows [9, 20) changes exactly those rows
    cache = view.copy()
    cache[:, 9:20] += 1.0
    new = paged.write_rows(pool, table, bs, cache, 9, 20)
    changed = np.argwhere((new != pool).any(axis=(1, 3)))
    want = sorted((int(table[r // bs]), r % bs) for r in range(9, 20))
    assert sorted(map(tuple, changed.tolist())) == want
    np.testing.assert_array_equal(paged.logical_rows(new, table, bs, rows)[:, 9:20],
                                  view[:, 9:20] + 1.0)
