"""The direct-to-LDS kernel off the tile grid and on the blocked A layout,
and fp16 subnormal inputs, against the oracle over every output element.

* K and N tails: K not a multiple of the K slice (K % 8 == 0 and != 0) and
  N % 8 != 0 at full size, on the table's row, in row-major and transposed
  layouts; the kernel family that ran is checked to be the pipelined
  direct-to-LDS one.
* Prepacked A ([ceil(K/BK), M, BK], the yfxerp page's layout planner,
  section 3.2) on the same kernel, on the 1024x1024x2048 and 8192^3 shapes
  and a K tail.
* fp16 and bf16 subnormal inputs (A = k 2^-24 or k 2^-133, k in -4..4):
  exact in fp32, so the
  bit-exact gate shows whether the matrix cores keep subnormals rather
  than flushing them (a flush would zero every product).
"""
import numpy as np
import pytest

import tiled_matrix_multiplication_gemm_amd as mg
from oracle import compare, layout
from tiled_matrix_multiplication_gemm_amd import inputs
from tests.gpu_util import (BF16, F16, Guarded, announce, assert_bitexact, assert_tolerance, to_dev, to_host)
from tests.test_gpu_parity import assert_higham, run_transposed

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mg.lib()
    yield
    mg.mg_set_config(-1)


def padded_dev(bits, dt):
    """bits [R, C] on the device with the row stride rounded up to 8."""
    R, C = bits.shape
    ld = (C + 7) // 8 * 8
    full = np.zeros((R, ld), dtype=np.uint16)
    full[:, :C] = bits
    return to_dev(full, dt)[:, :C]


def run(case, bias=False):
    import torch

    dt = case.dtype
    A, B = padded_dev(case.A, dt), padded_dev(case.B, dt)
    out = Guarded(case.M, case.N, dt, ld=(case.N + 7) // 8 * 8)
    if bias:
        mg.mg_gemm_bias_relu(A, B, to_dev(case.bias, dt), out=out.mat)
    else:
        mg.mg_gemm(A, B, out=out.mat)
    torch.cuda.synchronize()
    assert out.guards_intact(), "write outside the output"
    return out.result()


# (M, N, K, dtype): K % 8 != 0, K % 8 == 0 with a slice tail, N % 8 != 0
RAGGED_LARGE = [(4096, 4096, 4100, F16), (2048, 8190, 2048, BF16), (3000, 2050, 4104, BF16),
                (1024, 1021, 2047, F16)]


@pytest.mark.parametrize("M,N,K,dt", RAGGED_LARGE)
def test_ragged_large_on_the_fast_kernel(orc, M, N, K, dt):
    for integer in (True, False):
        epi = integer
        seed = 8800 + M % 97 + N % 89 + K % 83 + integer
        if integer:
            c = inputs.integer_dense(M, N, K, dt, seed, epilogue=epi, name="ragged_fast")
        else:
            c = inputs.random_dense(M, N, K, dt, seed, epilogue=epi, name="ragged_fast")
        announce("ragged fast M=%d N=%d K=%d dt=%d int=%s" % (M, N, K, dt, integer))
        got = run(c, bias=epi)
        assert mg.mg_last_kernel() == "gemm_dlds_kernel"
        ref, ref_q = orc.gemm(c.A, c.B, dt, bias=c.bias, relu=c.relu)
        if integer:
            assert_bitexact(got, ref_q, dt, c.name)
        else:
            assert_tolerance(got, ref, dt, c.name)
            absdot, _ = orc.gemm(compare.abs_bits(c.A), compare.abs_bits(c.B), dt)
            assert_higham(got, ref, absdot, c)


@pytest.mark.parametrize("ta,tb", [(1, 0), (0, 1), (1, 1)])
def test_ragged_large_transposed(orc, ta, tb):
    M, N, K = 2050, 1030, 2052
    c = inputs.integer_dense(M, N, K, BF16, 8900 + 2 * ta + tb, name="ragged_transposed")
    announce("ragged transposed ta=%d tb=%d" % (ta, tb))
    got, guards = run_transposed(c, ta, tb)
    assert guards
    assert mg.mg_last_kernel() == "gemm_dlds_kernel"
    _, ref_q = orc.gemm(c.A, c.B, BF16)
    assert_bitexact(got, ref_q, BF16, c.name)


def run_packed(case):
    import torch

    dt = case.dtype
    M, K = case.M, case.K
    BK = mg.mg_config_bk(M, case.N, K, dt)
    Ap = mg.mg_prepack_a(padded_dev(case.A, dt), BK)
    out = Guarded(M, case.N, dt, ld=(case.N + 7) // 8 * 8)
    mg.mg_gemm_prepacked(Ap, BK, padded_dev(case.B, dt), M, K, out=out.mat)
    torch.cuda.synchronize()
    assert out.guards_intact(), "write outside the output"
    assert mg.mg_last_kernel() == "gemm_dlds_kernel"
    return Ap, BK, out.result()


@pytest.mark.parametrize("M,N,K,dt", [(1024, 1024, 2048, F16), (8192, 8192, 8192, BF16), (700, 390, 1000, F16),
                                      (2048, 2048, 4100, BF16)])
def test_prepacked_a_on_the_fast_kernel(orc, M, N, K, dt):
    c = inputs.integer_dense(M, N, K, dt, 9100 + K % 101, name="packed_fast")
    announce("prepacked fast M=%d N=%d K=%d dt=%d" % (M, N, K, dt))
    Ap, BK, got = run_packed(c)
    if M * K <= 1 << 22:
        assert np.array_equal(to_host(Ap).reshape(Ap.shape), layout.prepack_a(c.A, BK))
    del Ap
    _, ref_q = orc.gemm(c.A, c.B, dt)
    assert_bitexact(got, ref_q, dt, c.name)
    if M * N <= 1 << 22:
        f = inputs.random_dense(M, N, K, dt, 9200 + K % 101, name="packed_fast_float")
        _, _, gotf = run_packed(f)
        ref, _ = orc.gemm(f.A, f.B, dt)
        assert_tolerance(gotf, ref, dt, f.name)


@pytest.mark.parametrize("M,N,K", [(1024, 1024, 2048), (256, 256, 64), (300, 200, 129)])
def test_fp16_subnormal_inputs_bitexact(orc, M, N, K):
    c = inputs.subnormal_dense(M, N, K, 9300 + K)
    assert np.all((c.A & 0x7C00) == 0)  # zero or subnormal
    announce("fp16 subnormal inputs M=%d N=%d K=%d" % (M, N, K))
    got = run(c)
    _, ref_q = orc.gemm(c.A, c.B, F16)
    assert np.count_nonzero(ref_q & 0x7FFF) > 0.9 * ref_q.size
    assert_bitexact(got, ref_q, F16, "fp16 subnormal")


@pytest.mark.parametrize("M,N,K", [(1024, 1024, 2048), (256, 256, 64), (300, 200, 129)])
def test_bf16_subnormal_inputs_bitexact(orc, M, N, K):
    """The same with bf16 subnormals (k 2^-133): the fp32 accumulators then
    hold values near and below fp32's smallest normal, 2^-126, so a flush of
    fp32 denormals would show as well as a flush of the inputs."""
    c = inputs.subnormal_dense(M, N, K, 9400 + K, dtype=BF16)
    assert np.all((c.A & 0x7F80) == 0)  # zero or subnormal
    announce("bf16 subnormal inputs M=%d N=%d K=%d" % (M, N, K))
    got = run(c)
    _, ref_q = orc.gemm(c.A, c.B, BF16)
    assert np.count_nonzero(ref_q & 0x7FFF) > 0.9 * ref_q.size
    assert_bitexact(got, ref_q, BF16, "bf16 subnormal")
