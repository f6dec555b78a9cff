"""Pins of the Higham summation bound used as a float diagnostic gate
(oracle/compare.py): simulated fp32 accumulations in several orders stay
inside it, and plausible kernel mistakes -- a dropped or doubled k-block, a
truncating output conversion -- leave it."""
import numpy as np
import pytest

from oracle import compare
from tiled_matrix_multiplication_gemm_amd import inputs

F16, BF16 = compare.F16, compare.BF16


def test_gamma_definition():
    u = 2.0 ** -24
    assert compare.gamma(1) == u / (1 - u)
    assert compare.gamma(2048) > 2048 * u
    with pytest.raises(AssertionError):
        compare.gamma(2 ** 24)


def _case(M, N, K, seed):
    rng = np.random.default_rng(seed)
    a = inputs.to_bits(rng.standard_normal((M, K)) / np.sqrt(K), F16)
    b = inputs.to_bits(rng.standard_normal((K, N)) / np.sqrt(K), F16)
    A, B = compare.to_f64(a, F16), compare.to_f64(b, F16)
    return A, B, A @ B, np.abs(A) @ np.abs(B)


def _fp32_sum(A, B, order):
    """fp32 accumulation of exact products (each fits fp32) in a given order."""
    M, K = A.shape
    N = B.shape[1]
    acc = np.zeros((M, N), dtype=np.float32)
    for k in order:
        acc = (acc + (A[:, k:k + 1] * B[k:k + 1, :]).astype(np.float32)).astype(np.float32)
    return acc


def _round(acc32, dtype, mode="rne"):
    x = acc32.astype(np.float64)
    if mode == "rne":
        return inputs.to_bits(x, dtype)
    # round toward zero: the RNE neighbour of smaller magnitude
    q = inputs.to_bits(x, dtype)
    back = compare.to_f64(q, dtype)
    over = np.abs(back) > np.abs(x)
    q = q.copy()
    q[over] -= 1  # one step toward zero in magnitude (same sign)
    return q


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("order", ["ascending", "descending", "blocked16"])
def test_fp32_accumulation_in_any_order_is_inside(dtype, order):
    M, N, K = 24, 40, 2048
    A, B, ref, absdot = _case(M, N, K, 11)
    if order == "ascending":
        ks = range(K)
    elif order == "descending":
        ks = range(K - 1, -1, -1)
    else:  # 16-wide blocks, last block first, ascending inside a block
        ks = [k for blk in range(K // 16 - 1, -1, -1) for k in range(16 * blk, 16 * blk + 16)]
    got = _round(_fp32_sum(A, B, ks), dtype)
    bound = compare.higham_bound(absdot, ref, K, dtype)
    assert compare.higham_ratio(got, ref, bound, dtype) <= 1.0


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_bias_add_is_inside(dtype):
    M, N, K = 16, 32, 1024
    A, B, ref, absdot = _case(M, N, K, 12)
    bias = compare.to_f64(inputs.to_bits(np.random.default_rng(3).standard_normal(N) * 0.1, dtype), dtype)
    acc = _fp32_sum(A, B, range(K))
    v = np.maximum((acc + bias.astype(np.float32)).astype(np.float32), 0.0)
    got = _round(v, dtype)
    refb = np.maximum(ref + bias, 0.0)
    bound = compare.higham_bound(absdot, refb, K, dtype, abs_bias=np.abs(bias))
    assert compare.higham_ratio(got, refb, bound, dtype) <= 1.0


def test_dropped_or_doubled_k_block_is_outside():
    M, N, K = 24, 40, 2048
    A, B, ref, absdot = _case(M, N, K, 13)
    bound = compare.higham_bound(absdot, ref, K, F16)
    dropped = _round(_fp32_sum(A, B, range(16, K)), F16)
    doubled = _round(_fp32_sum(A, B, list(range(K)) + list(range(16))), F16)
    assert compare.higham_ratio(dropped, ref, bound, F16) > 1.0
    assert compare.higham_ratio(doubled, ref, bound, F16) > 1.0


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_truncating_output_conversion_is_outside(dtype):
    M, N, K = 64, 64, 512
    A, B, ref, absdot = _case(M, N, K, 14)
    got = _round(_fp32_sum(A, B, range(K)), dtype, mode="rtz")
    bound = compare.higham_bound(absdot, ref, K, dtype)
    assert compare.higham_ratio(got, ref, bound, dtype) > 1.0


def test_non_finite_is_outside():
    got = np.array([0x7C00], dtype=np.uint16)  # fp16 +inf
    assert compare.higham_ratio(got, np.array([1.0]), np.array([1.0]), F16) == float("inf")


def test_abs_bits_clears_only_the_sign():
    b = np.array([0x8000, 0xBC00, 0x3C00, 0xFBFF], dtype=np.uint16)
    assert np.array_equal(compare.abs_bits(b), np.array([0x0000, 0x3C00, 0x3C00, 0x7BFF], dtype=np.uint16))
