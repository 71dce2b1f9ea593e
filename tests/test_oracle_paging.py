"""Pins for oracle.paging (CPU): the logical view of a paged pool."""
import numpy as np

from oracle import paging as OP


def test_physical_rows_hand_computed():
    # page of 2 positions; sequence 0 maps blocks (2, unmapped, 0), sequence 1 maps (1, 3, unmapped)
    table = np.array([[2, -1, 0], [1, 3, -1]], dtype=np.int32)
    want = {0: [4, 5, -1, -1, 0, 1, -1], 1: [2, 3, 6, 7, -1, -1, -1]}
    for b, rows in want.items():
        got = [OP.physical_row(table, 2, b, p) for p in range(7)]
        assert got == rows, (b, got)
    assert OP.physical_row(table, 2, 0, -1) == -1


def test_identity_map_is_the_dense_layout():
    B, nb, page = 3, 4, 5
    pool = np.arange(B * nb * page * 2).reshape(B * nb * page, 2)
    table = np.arange(B * nb, dtype=np.int32).reshape(B, nb)
    view, mapped = OP.logical_view(pool, table, page, nb * page)
    assert mapped.all()
    assert np.array_equal(view, pool.reshape(B, nb * page, 2))


def test_permuted_pool_round_trip_and_holes():
    rng = np.random.default_rng(5)
    B, nb, page = 2, 6, 4
    T = nb * page - 3
    dense = rng.integers(0, 256, size=(B, nb * page, 3), dtype=np.uint8)
    perm = rng.permutation(B * nb + 2)[:B * nb].astype(np.int32).reshape(B, nb)
    pool = np.full(((B * nb + 2) * page, 3), 99, dtype=np.uint8)
    for b in range(B):
        for j in range(nb):
            pool[perm[b, j] * page:(perm[b, j] + 1) * page] = dense[b, j * page:(j + 1) * page]
    view, mapped = OP.logical_view(pool, perm, page, T)
    assert mapped.all() and np.array_equal(view, dense[:, :T])
    holed = perm.copy()
    holed[1, 2] = -1
    view, mapped = OP.logical_view(pool, holed, page, T)
    assert not mapped[1, 8:12].any() and mapped.sum() == B * T - page
    assert (view[1, 8:12] == 0).all() and np.array_equal(view[0], dense[0, :T])
