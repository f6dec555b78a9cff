"""Pins of the oracle's fp32 path (decode, single RNE rounding, GEMM) against
references other than itself: numpy's float32 conversions, exact rational
arithmetic, and closed forms.  CPU only."""
from fractions import Fraction

import numpy as np
import pytest

import oracle


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


def _finite_patterns(rng, n):
    b = rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    return b[(b & 0x7F800000) != 0x7F800000]


def test_decode32_matches_numpy_and_special_values():
    rng = np.random.default_rng(1)
    b = rng.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    got = oracle.decode32(b)
    with np.errstate(invalid="ignore"):  # signalling NaN patterns among the draws
        ref = b.view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    special = np.array([0x00000000, 0x80000000, 0x00000001, 0x007FFFFF, 0x00800000, 0x7F7FFFFF, 0x7F800000,
                        0xFF800000, 0x3F800000], dtype=np.uint32)
    want = [0.0, -0.0, 2.0 ** -149, (2 ** 23 - 1) * 2.0 ** -149, 2.0 ** -126, (2 - 2.0 ** -23) * 2.0 ** 127,
            np.inf, -np.inf, 1.0]
    assert list(oracle.decode32(special)) == want
    assert np.signbit(oracle.decode32(special)[1])


def test_encode32_round_trip_and_numpy_cast():
    rng = np.random.default_rng(2)
    b = _finite_patterns(rng, 500_000)
    assert np.array_equal(oracle.encode32(oracle.decode32(b)), b)
    x = rng.standard_normal(500_000) * np.exp2(rng.integers(-160, 130, size=500_000))
    with np.errstate(over="ignore"):
        ref = x.astype(np.float32).view(np.uint32)
    assert np.array_equal(oracle.encode32(x), ref)


def test_encode32_ties_to_even_at_every_kind_of_midpoint():
    rng = np.random.default_rng(3)
    b = _finite_patterns(rng, 200_000) & np.uint32(0x7FFFFFFF)  # positive
    b = b[b < 0x7F7FFFFF]                                       # has a finite successor
    lo, hi = oracle.decode32(b), oracle.decode32(b + 1)
    mid = (lo + hi) / 2                                         # exact in fp64
    even = np.where(b % 2 == 0, b, b + 1)
    assert np.array_equal(oracle.encode32(mid), even)
    assert np.array_equal(oracle.encode32(np.nextafter(mid, 0)), b)
    assert np.array_equal(oracle.encode32(np.nextafter(mid, np.inf)), b + 1)
    # the midpoint above the largest finite value rounds to the even pattern: +inf
    top = (2 - 2.0 ** -23) * 2.0 ** 127
    assert oracle.encode32(np.array([top + 2.0 ** 103]))[0] == 0x7F800000
    assert oracle.encode32(np.array([np.nextafter(top + 2.0 ** 103, 0)]))[0] == 0x7F7FFFFF
    # half the smallest subnormal ties to +0, a hair more rounds up
    assert oracle.encode32(np.array([2.0 ** -150]))[0] == 0
    assert oracle.encode32(np.array([np.nextafter(2.0 ** -150, 1)]))[0] == 1


def test_encode32_is_the_nearest_value_by_exact_arithmetic():
    rng = np.random.default_rng(4)
    xs = rng.standard_normal(2000) * np.exp2(rng.integers(-140, 120, size=2000))
    got = oracle.encode32(xs)
    for x, g in zip(xs, got):
        fx = Fraction(float(x))
        cand = [int(g) - 1, int(g), int(g) + 1]
        best = None
        for c in cand:
            if c < 0 or (c & 0x7F800000) == 0x7F800000 or (c ^ int(g)) & 0x80000000:
                continue
            v = Fraction(float(oracle.decode32(np.array([c], dtype=np.uint32))[0]))
            d = abs(v - fx)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        assert best[1] == int(g), (x, g, best)


def _f32_bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def test_gemm_f32_exact_on_integers_and_identity():
    rng = np.random.default_rng(5)
    A = rng.integers(-50, 51, size=(7, 13)).astype(np.float64)
    B = rng.integers(-50, 51, size=(13, 5)).astype(np.float64)
    ref, q = oracle.gemm_f32(_f32_bits(A), _f32_bits(B))
    exact = [[sum(Fraction(int(A[i, k])) * Fraction(int(B[k, j])) for k in range(13)) for j in range(5)]
             for i in range(7)]
    assert all(ref[i, j] == exact[i][j] for i in range(7) for j in range(5))
    assert np.array_equal(q, _f32_bits(ref))
    X = rng.standard_normal((6, 6)).astype(np.float32)
    r, q = oracle.gemm_f32(X.view(np.uint32), _f32_bits(np.eye(6)))
    assert np.array_equal(q, X.view(np.uint32))
    P = np.eye(6)[[3, 0, 5, 1, 4, 2]]
    r, q = oracle.gemm_f32(_f32_bits(P), X.view(np.uint32))
    assert np.array_equal(q.view(np.float32), X[[3, 0, 5, 1, 4, 2]])


def test_gemm_f32_random_against_fp64_matmul_and_samples():
    rng = np.random.default_rng(6)
    A = rng.standard_normal((33, 70)).astype(np.float32)
    B = rng.standard_normal((70, 17)).astype(np.float32)
    ref, q = oracle.gemm_f32(A.view(np.uint32), B.view(np.uint32))
    want = A.astype(np.float64) @ B.astype(np.float64)
    bound = 1e-13 * (np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64)))
    assert np.all(np.abs(ref - want) <= bound)
    rows = rng.integers(0, 33, size=50)
    cols = rng.integers(0, 17, size=50)
    rs, qs = oracle.gemm_f32_sampled(A.view(np.uint32), B.view(np.uint32), rows, cols)
    assert np.array_equal(rs, ref[rows, cols]) and np.array_equal(qs, q[rows, cols])
