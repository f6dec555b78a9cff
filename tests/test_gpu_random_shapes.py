"""Seeded random shapes through the automatic row choice, against the oracle.

The other parity tests force each table row on chosen shapes; here the
library picks the row itself (swept shapes from the cached best, the rest
from the time model), so the selection and every row it can return are
exercised together on shapes nobody picked by hand.  M, N and K are drawn
log-uniformly (M up to 2^17, N up to 2^14, K up to about 5800), within
bounds that keep each case to a few seconds of oracle time, and about half
the cases are integer-valued (bit-exact gate), the rest random floats
(1e-2 gate plus Higham's bound).  Every output element is compared.
"""
import numpy as np
import pytest

import tiled_matrix_multiplication_gemm_amd as mg
from tiled_matrix_multiplication_gemm_amd import inputs
from tests.test_gpu_parity import check_full

SEED = 3
COUNT = 48


def draw_cases(seed=SEED, count=COUNT):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        M = int(np.exp2(rng.uniform(4, 17)))
        N = int(np.exp2(rng.uniform(4, 14)))
        K = int(np.exp2(rng.uniform(5, 12.5)))
        # at least a few hundred million products (so the larger rows get
        # chosen), at most 6e9, and operands of at most 2e7 elements each
        if M * N * K > 6e9 or M * N * K < 2e8 or M * N > 3e7 or M * K > 2e7 or K * N > 2e7:
            continue
        dtype = int(rng.integers(0, 2))
        integer = bool(rng.integers(0, 2))
        epi = bool(rng.integers(0, 2))
        cases.append((M, N, K, dtype, integer, epi, int(rng.integers(0, 2**31))))
    return cases


CASES = draw_cases()


def test_draws_spread_over_the_rows():
    """The drawn shapes land on several rows, all of them rows with the
    direct-to-LDS kernel (with the current table: 0, 1, 2, 3, 4, 8 and 9,
    every row the choice returns for a dense problem but 256x256 w2x2)."""
    rows = {mg.mg_select_config(M, N, K, dt) for M, N, K, dt, *_ in CASES}
    assert len(rows) >= 5 and rows <= {0, 1, 2, 3, 4, 6, 8, 9}, sorted(rows)


@pytest.fixture(scope="module")
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mg.lib()
    mg.mg_set_config(-1)
    yield


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=lambda c: "%dx%dx%d_%s_%s%s" % (
    c[0], c[1], c[2], "bf16" if c[3] else "f16", "int" if c[4] else "float", "_epi" if c[5] else ""))
def test_random_shape_auto_row(orc, _gpu, case):
    M, N, K, dtype, integer, epi, seed = case
    if integer:
        c = inputs.integer_dense(M, N, K, dtype, seed, epilogue=epi, name="random")
    else:
        c = inputs.random_dense(M, N, K, dtype, seed, epilogue=epi, name="random")
    check_full(orc, c)
    assert mg.mg_last_kernel() == "gemm_dlds_kernel", (M, N, K, mg.mg_last_kernel())
