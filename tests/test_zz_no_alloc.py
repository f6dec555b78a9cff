"""mg_gemm_splitk_noalloc (split-K with the partials in the library's own
scratch array) against mg_gemm_splitk with a caller workspace, called
through the C ABI: two calls in a row, the second on a smaller problem, each
bit-identical to the workspace form (the same kernels in the same split
order) and, on integer inputs, bit-exact against the oracle.  Also the size
limit and the validation that runs before any HIP call."""
import ctypes

import numpy as np
import pytest

import tiled_matrix_multiplication_gemm_amd as mg
from oracle import compare
from tiled_matrix_multiplication_gemm_amd import inputs
from tests.gpu_util import BF16, F16, Guarded, announce, assert_bitexact, assert_tolerance, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mg.lib()


def _call_noalloc(A, B, out, splits):
    L = mg.lib()
    M, K = A.shape
    N = B.shape[1]
    return L.mg_gemm_splitk_noalloc(A.data_ptr(), B.data_ptr(), out.data_ptr(), splits, M, N, K, A.stride(0),
                                    A.stride(1), B.stride(0), B.stride(1), out.stride(0), out.stride(1),
                                    mg._dtype_code(A), mg._dtype_code(out), mg._stream(A))


def _call_workspace(A, B, out, splits):
    import torch

    L = mg.lib()
    M, K = A.shape
    N = B.shape[1]
    need = L.mg_splitk_workspace_bytes(M, N, splits)
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    st = L.mg_gemm_splitk(A.data_ptr(), B.data_ptr(), out.data_ptr(), ws.data_ptr(), need, splits, M, N, K,
                          A.stride(0), A.stride(1), B.stride(0), B.stride(1), out.stride(0), out.stride(1),
                          mg._dtype_code(A), mg._dtype_code(out), mg._stream(A))
    return st, ws


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_noalloc_matches_workspace_form_twice(orc, dtype):
    import torch

    # the second problem is smaller: its call reuses the front of the scratch
    # array, which still holds the first call's partials
    problems = [(512, 768, 8192, 8, True), (128, 256, 4096, 4, True), (520, 264, 2048, 2, False)]
    for i, (M, N, K, splits, integer) in enumerate(problems):
        announce("noalloc split-K #%d M=%d N=%d K=%d splits=%d dt=%d int=%s" % (i, M, N, K, splits, dtype, integer))
        if integer:
            c = inputs.integer_dense(M, N, K, dtype, 7100 + i, name="noalloc")
        else:
            c = inputs.random_dense(M, N, K, dtype, 7100 + i, name="noalloc")
        A, B = to_dev(c.A, dtype), to_dev(c.B, dtype)
        o1, o2 = Guarded(M, N, dtype), Guarded(M, N, dtype)
        assert _call_noalloc(A, B, o1.mat, splits) == 0
        st, ws = _call_workspace(A, B, o2.mat, splits)
        assert st == 0
        torch.cuda.synchronize()
        del ws
        assert o1.guards_intact() and o2.guards_intact()
        got = o1.result()
        assert np.array_equal(got, o2.result()), "no-alloc and workspace forms differ"
        ref, ref_q = orc.gemm(c.A, c.B, dtype)
        if integer:
            assert_bitexact(got, ref_q, dtype, "noalloc")
        else:
            assert_tolerance(got, ref, dtype, "noalloc")


def test_noalloc_limits_and_validation():
    import torch

    announce("noalloc limits")
    L = mg.lib()
    cap = L.mg_splitk_noalloc_max_bytes()
    assert cap == 32 << 20
    M, N, K = 1024, 1024, 4096
    A = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    B = torch.zeros((K, N), dtype=torch.float16, device="cuda")
    out = torch.zeros((M, N), dtype=torch.float16, device="cuda")
    assert 8 * M * N * 4 <= cap < 16 * M * N * 4
    assert _call_noalloc(A, B, out, 16) == 1  # partials beyond the scratch array: INVALID_ARG
    assert _call_noalloc(A, B, out, 0) == 1
    assert _call_noalloc(A, B, out, 8) == 0
    torch.cuda.synchronize()
    assert int((out != 0).sum()) == 0
    with pytest.raises(RuntimeError, match="INVALID_ARG"):
        mg.mg_gemm_splitk_noalloc(A, B, splits=16, out=out)
