"""The Python binding refuses, before any launch, arguments that the C ABI
cannot see are wrong: an output of the wrong shape, dtype or device, a
non-unit inner stride on an output, operands of mixed dtypes or devices."""
import pytest

import tiled_matrix_multiplication_gemm_amd as mg
from tests.gpu_util import announce

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mg.lib()


def _t(*shape, dtype=None, device="cuda"):
    import torch

    return torch.zeros(shape, dtype=dtype or torch.float16, device=device)


def test_gemm_family_rejects_bad_outputs():
    import torch

    announce("binding: bad outputs")
    a, b = _t(64, 32), _t(32, 48)
    bias = _t(48)
    for fn in (lambda o: mg.mg_gemm(a, b, out=o), lambda o: mg.mg_gemm_bias_relu(a, b, bias, out=o),
               lambda o: mg.mg_gemm_splitk(a, b, splits=2, out=o)):
        with pytest.raises(RuntimeError, match="INVALID_ARG"):
            fn(_t(63, 48))  # fewer rows than M: the kernel would write past its end
        with pytest.raises(RuntimeError, match="INVALID_ARG"):
            fn(_t(64, 40))
        with pytest.raises(RuntimeError, match="UNSUPPORTED_DTYPE"):
            fn(_t(64, 48, dtype=torch.bfloat16))
        with pytest.raises(RuntimeError, match="GPU tensors only"):
            fn(_t(64, 48, device="cpu"))
        with pytest.raises(RuntimeError, match="UNSUPPORTED_LAYOUT"):
            fn(_t(48, 64).t())
    out = _t(64, 48)
    mg.mg_gemm(a, b, out=out)  # the right output is taken
    torch.cuda.synchronize()


def test_mixed_operand_dtypes_are_refused():
    import torch

    announce("binding: mixed dtypes")
    a, bb = _t(64, 32), _t(32, 48, dtype=torch.bfloat16)
    with pytest.raises(RuntimeError, match="UNSUPPORTED_DTYPE"):
        mg.mg_gemm(a, bb)
    with pytest.raises(RuntimeError, match="UNSUPPORTED_DTYPE"):
        mg.mg_gemm_splitk(a, bb, splits=2)
    with pytest.raises(RuntimeError, match="UNSUPPORTED_DTYPE"):
        mg.mg_gemm_batched(_t(2, 64, 32), _t(2, 32, 48, dtype=torch.bfloat16))
    with pytest.raises(RuntimeError, match="UNSUPPORTED_DTYPE"):
        mg.mg_gemm_bias_relu(a, _t(32, 48), _t(48, dtype=torch.bfloat16))
    with pytest.raises(RuntimeError, match="GPU tensors only"):
        mg.mg_gemm(a, _t(32, 48, device="cpu"))


def test_batched_grouped_attention_reject_bad_outputs():
    import torch

    announce("binding: batched, grouped, attention outputs")
    with pytest.raises(RuntimeError, match="INVALID_ARG"):
        mg.mg_gemm_batched(_t(3, 64, 32), _t(3, 32, 48), out=_t(2, 64, 48))
    x, w = _t(100, 64), _t(4, 64, 48)
    off = torch.tensor([0, 10, 50, 50, 100], dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError, match="INVALID_ARG"):
        mg.mg_grouped_gemm(x, w, off, out=_t(99, 48))
    with pytest.raises(RuntimeError, match="UNSUPPORTED_DTYPE"):
        mg.mg_grouped_gemm(x, w, off, out=_t(100, 48, dtype=torch.bfloat16))
    q, k = _t(2, 64, 32), _t(2, 80, 32)
    with pytest.raises(RuntimeError, match="INVALID_ARG"):
        mg.mg_attention_scores(q, k, out=_t(2, 64, 64))
    with pytest.raises(RuntimeError, match="UNSUPPORTED_DTYPE"):
        mg.mg_attention_scores(q, k, out=_t(2, 64, 80, dtype=torch.float32))
    with pytest.raises(RuntimeError, match="UNSUPPORTED_LAYOUT"):
        mg.mg_attention_scores(q, k, out=_t(2, 80, 64).transpose(1, 2))
