"""Pins of the oracle's index bookkeeping: blocked prepack of A, grouped tile
order and the shared-memory budget (CPU only).  The worked examples the pages
print are stored under tests/golden/ with their citation."""
import json
import os

import numpy as np
import pytest

from oracle import layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_lds_budget_worked_example():
    g = load("lds_budget.json")
    assert layout.lds_bytes(g["BM"], g["BN"], g["BK"], g["elem_bytes"], g["stages"]) == g["bytes"]


def test_grouped_order_9x9_worked_example():
    g = load("grouped_order_9x9.json")
    m, n, t, kb = g["num_pid_m"], g["num_pid_n"], g["tiles"], g["k_blocks"]
    rm = [layout.row_major_pid(p, m, n) for p in range(t)]
    gr = [layout.grouped_pid(p, m, n, g["group_m"]) for p in range(t)]
    assert layout.blocks_loaded(rm, kb) == g["row_major_blocks"]
    assert layout.blocks_loaded(gr, kb) == g["grouped_blocks"]
    # the grouped order's first 9 tiles form the 3x3 corner of the grid
    assert sorted(gr) == [(i, j) for i in range(3) for j in range(3)]


@pytest.mark.parametrize("group_m", [1, 2, 3, 4, 8, 16])
def test_grouped_order_is_a_bijection(group_m):
    for m in range(1, 40, 3):
        for n in (1, 2, 5, 9, 17, 33):
            seen = {layout.grouped_pid(p, m, n, group_m) for p in range(m * n)}
            assert seen == {(i, j) for i in range(m) for j in range(n)}


def test_group_m_one_is_column_major_and_large_group_is_column_major_within():
    # GROUP_M = 1 walks a row of tiles at a time (row-major)
    assert [layout.grouped_pid(p, 3, 4, 1) for p in range(12)] == [layout.row_major_pid(p, 3, 4) for p in range(12)]
    # GROUP_M >= num_pid_m walks the whole grid column by column
    assert [layout.grouped_pid(p, 3, 4, 8) for p in range(12)] == [(p % 3, p // 3) for p in range(12)]


def test_prepack_small_worked_case():
    # M=2, K=4, BK=2: the blocked rows are [a00 a01], [a10 a11], [a02 a03], [a12 a13]
    A = np.array([[0, 1, 2, 3], [10, 11, 12, 13]], dtype=np.uint16)
    Ap = layout.prepack_a(A, 2)
    assert Ap.reshape(-1, 2).tolist() == [[0, 1], [10, 11], [2, 3], [12, 13]]


@pytest.mark.parametrize("M,K,BK", [(1, 1, 8), (5, 7, 8), (33, 129, 32), (64, 256, 64), (3, 100, 64)])
def test_prepack_roundtrip_padding_and_index(M, K, BK):
    rng = np.random.default_rng(M + K)
    A = rng.integers(1, 65535, size=(M, K)).astype(np.uint16)
    Ap = layout.prepack_a(A, BK)
    assert Ap.shape == layout.prepacked_shape(M, K, BK)
    assert np.array_equal(layout.unpack_a(Ap, K), A)
    flat = Ap.ravel()
    for m in range(0, M, max(1, M // 4)):
        for k in range(0, K, max(1, K // 5)):
            assert flat[layout.prepacked_index(m, k, M, BK)] == A[m, k]
    # the zero padding of the last K block never holds data
    pad = Ap.shape[0] * BK - K
    if pad:
        assert np.all(Ap[-1, :, BK - pad:] == 0)
