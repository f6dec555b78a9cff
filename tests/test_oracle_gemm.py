"""Pins of the oracle's dense and grouped GEMM (CPU only).

Each check is fixed by something other than the oracle itself: brute force in
exact rational arithmetic, a textbook product, numpy's float64 matmul (another
summation order), identity and permutation matrices, the all-ones closed form
(every entry equals K), linearity, the transpose identity, and for the
epilogue and the grouped variant their reductions to simpler cases.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

from tiled_matrix_multiplication_gemm_amd import inputs

F16, BF16 = 0, 1


def bits(x, dtype):
    return inputs.to_bits(np.asarray(x, dtype=np.float64), dtype)


def exact_value(b, dtype):
    b = np.asarray(b, dtype=np.uint16)
    if dtype == F16:
        return b.view(np.float16).astype(np.float64)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_textbook_2x2(orc):
    A = bits([[1, 2], [3, 4]], F16)
    B = bits([[5, 6], [7, 8]], F16)
    ref, ref_q = orc.gemm(A, B, F16)
    assert ref.tolist() == [[19.0, 22.0], [43.0, 50.0]]
    assert exact_value(ref_q, F16).tolist() == [[19.0, 22.0], [43.0, 50.0]]


def test_all_2x2_matrices_over_minus1_0_1(orc):
    """Every pair of 2x2 matrices over {-1,0,1} (3^8 pairs) against the expanded formula."""
    vals = (-1.0, 0.0, 1.0)
    for a00, a01, a10, a11 in itertools.product(vals, repeat=4):
        A = bits([[a00, a01], [a10, a11]], F16)
        for b00, b01, b10, b11 in itertools.product(vals, repeat=4):
            B = bits([[b00, b01], [b10, b11]], F16)
            ref, _ = orc.gemm(A, B, F16, nthreads=1)
            want = [[a00 * b00 + a01 * b10, a00 * b01 + a01 * b11],
                    [a10 * b00 + a11 * b10, a10 * b01 + a11 * b11]]
            assert ref.tolist() == want


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (2, 3, 5), (5, 8, 3), (8, 5, 8), (3, 1, 7), (1, 8, 2)])
def test_brute_force_exact_rationals(orc, dtype, M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K + 1000 * dtype)
    A = bits(rng.uniform(-2, 2, size=(M, K)), dtype)
    B = bits(rng.uniform(-2, 2, size=(K, N)), dtype)
    bias = bits(rng.uniform(-1, 1, size=N), dtype)
    ref, ref_q = orc.gemm(A, B, dtype, bias=bias, relu=True, nthreads=1)
    a, b, c = exact_value(A, dtype), exact_value(B, dtype), exact_value(bias, dtype)
    for i in range(M):
        for j in range(N):
            s = sum(Fraction(float(a[i, k])) * Fraction(float(b[k, j])) for k in range(K)) + Fraction(float(c[j]))
            s = max(s, Fraction(0))
            scale = sum(abs(Fraction(float(a[i, k])) * Fraction(float(b[k, j]))) for k in range(K)) + abs(
                Fraction(float(c[j])))
            assert abs(Fraction(float(ref[i, j])) - s) <= scale * Fraction(1, 2 ** 50)
            # the rounded value is nearer to the exact result than either neighbouring pattern
            qb = int(ref_q[i, j])
            dq = abs(Fraction(float(exact_value(qb, dtype))) - s)
            for nb in (qb - 1, qb + 1):
                if 0 <= nb < 0x10000:
                    v = float(exact_value(nb, dtype))
                    if np.isfinite(v):
                        assert abs(Fraction(v) - s) >= dq


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_integer_brute_force_is_exact(orc, dtype):
    rng = np.random.default_rng(3 + dtype)
    for M, N, K in [(4, 6, 9), (7, 3, 33), (1, 5, 64)]:
        ai = rng.integers(-4, 5, size=(M, K))
        bi = rng.integers(-4, 5, size=(K, N))
        ref, ref_q = orc.gemm(bits(ai, dtype), bits(bi, dtype), dtype, nthreads=1)
        want = [[sum(int(ai[i, k]) * int(bi[k, j]) for k in range(K)) for j in range(N)] for i in range(M)]
        assert ref.astype(np.int64).tolist() == want
        assert np.array_equal(ref, np.array(want, dtype=np.float64))


def test_agrees_with_numpy_matmul(orc):
    rng = np.random.default_rng(5)
    for dtype in (F16, BF16):
        A = bits(rng.standard_normal((65, 300)), dtype)
        B = bits(rng.standard_normal((300, 70)), dtype)
        ref, _ = orc.gemm(A, B, dtype)
        want = exact_value(A, dtype) @ exact_value(B, dtype)
        scale = np.abs(exact_value(A, dtype)) @ np.abs(exact_value(B, dtype))
        assert np.all(np.abs(ref - want) <= 1e-12 * scale)


def test_identity_and_permutation(orc):
    rng = np.random.default_rng(9)
    for dtype in (F16, BF16):
        Bv = rng.standard_normal((16, 24))
        B = bits(Bv, dtype)
        _, q = orc.gemm(bits(np.eye(16), dtype), B, dtype)
        assert np.array_equal(q, B)
        P = np.eye(16)[rng.permutation(16)]
        _, q = orc.gemm(bits(P, dtype), B, dtype)
        assert np.array_equal(q, B[np.argmax(P, axis=1)])
        A = bits(rng.standard_normal((10, 24)), dtype)
        _, q = orc.gemm(A, bits(np.eye(24), dtype), dtype)
        assert np.array_equal(q, A)


@pytest.mark.parametrize("M,N,K,dtype", [(3, 5, 256, F16), (4, 4, 1024, F16), (2, 3, 2048, F16),
                                         (3, 2, 8192, BF16), (2, 2, 1, BF16)])
def test_all_ones_closed_form(orc, M, N, K, dtype):
    ref, q = orc.gemm(bits(np.ones((M, K)), dtype), bits(np.ones((K, N)), dtype), dtype)
    assert np.all(ref == K)
    assert np.all(exact_value(q, dtype) == K)


def test_linearity_in_both_operands_and_transpose(orc):
    rng = np.random.default_rng(13)
    M, N, K = 9, 11, 40
    A1, A2 = rng.integers(-4, 5, (M, K)), rng.integers(-4, 5, (M, K))
    B1, B2 = rng.integers(-4, 5, (K, N)), rng.integers(-4, 5, (K, N))
    al, be = 3, -2
    g = lambda A, B: orc.gemm(bits(A, F16), bits(B, F16), F16)[0]
    assert np.array_equal(g(al * A1 + be * A2, B1), al * g(A1, B1) + be * g(A2, B1))
    assert np.array_equal(g(A1, al * B1 + be * B2), al * g(A1, B1) + be * g(A1, B2))
    assert np.array_equal(g(A1, B1).T, g(B1.T, A1.T))


def test_epilogue_bias_relu(orc):
    rng = np.random.default_rng(17)
    N = 12
    bias_v = rng.integers(-4, 5, N).astype(np.float64)
    bias = bits(bias_v, F16)
    # A = 0: the output is ReLU(bias) broadcast over rows
    ref, q = orc.gemm(bits(np.zeros((5, 7)), F16), bits(rng.standard_normal((7, N)), F16), F16,
                      bias=bias, relu=True)
    assert np.array_equal(ref, np.broadcast_to(np.maximum(bias_v, 0), (5, N)))
    # ReLU of a non-positive value is +0.0 (bit pattern 0)
    assert np.all(q[:, bias_v <= 0] == 0)
    # all-ones: max(K + bias, 0)
    K = 3
    ref, _ = orc.gemm(bits(np.ones((4, K)), F16), bits(np.ones((K, N)), F16), F16, bias=bits(bias_v - 1, F16),
                      relu=True)
    assert np.array_equal(ref[0], np.maximum(K + bias_v - 1, 0))
    # bias without ReLU keeps negative values
    ref, _ = orc.gemm(bits(np.ones((2, K)), F16), bits(-np.ones((K, N)), F16), F16, bias=bias, relu=False)
    assert np.array_equal(ref[1], -K + bias_v)


def test_k_zero_is_the_empty_sum(orc):
    A = np.zeros((3, 0), dtype=np.uint16)
    B = np.zeros((0, 4), dtype=np.uint16)
    ref, q = orc.gemm(A, B, F16)
    assert np.all(ref == 0) and np.all(q == 0)
    bias_v = np.array([1.0, -2.0, 0.5, 3.0])
    ref, _ = orc.gemm(A, B, F16, bias=bits(bias_v, F16), relu=True)
    assert np.array_equal(ref[2], np.maximum(bias_v, 0))


def test_sampled_equals_full(orc):
    c = inputs.random_dense(70, 90, 130, BF16, seed=21, epilogue=True)
    ref, q = orc.gemm(c.A, c.B, BF16, bias=c.bias, relu=True)
    rows = np.array([0, 69, 13, 40, 69, 5])
    cols = np.array([0, 89, 77, 1, 0, 45])
    r2, q2 = orc.gemm_sampled(c.A, c.B, BF16, rows, cols, bias=c.bias, relu=True)
    assert np.array_equal(r2, ref[rows, cols])
    assert np.array_equal(q2, q[rows, cols])


def test_grouped_is_concatenation_of_dense(orc):
    counts = np.array([0, 5, 1, 0, 17, 3])
    c = inputs.random_grouped(E=6, T=int(counts.sum()), K=24, N=20, dtype=F16, seed=4, counts=counts)
    ref, q = orc.grouped_gemm(c.X, c.W, c.offsets, F16)
    off = c.offsets
    for e in range(c.E):
        r0, r1 = off[e], off[e + 1]
        if r1 > r0:
            dr, dq = orc.gemm(c.X[r0:r1], c.W[e], F16)
            assert np.array_equal(ref[r0:r1], dr)
            assert np.array_equal(q[r0:r1], dq)
    assert counts.sum() == c.T and off[-1] == c.T
    rows = np.array([0, 5, 6, 22, 25])
    cols = np.array([0, 19, 3, 7, 11])
    r2, q2 = orc.grouped_sampled(c.X, c.W, c.offsets, F16, rows, cols)
    assert np.array_equal(r2, ref[rows, cols]) and np.array_equal(q2, q[rows, cols])


def test_grouped_single_expert_is_plain_gemm(orc):
    c = inputs.random_grouped(E=1, T=33, K=16, N=9, dtype=BF16, seed=8)
    ref, q = orc.grouped_gemm(c.X, c.W, c.offsets, BF16)
    dr, dq = orc.gemm(c.X, c.W[0], BF16)
    assert np.array_equal(ref, dr) and np.array_equal(q, dq)


def test_grouped_rejects_bad_offsets(orc):
    c = inputs.random_grouped(E=2, T=4, K=8, N=8, dtype=F16, seed=1, counts=[2, 2])
    with pytest.raises(ValueError):
        orc.grouped_gemm(c.X, c.W, np.array([0, 3, 2], dtype=np.int32), F16)
