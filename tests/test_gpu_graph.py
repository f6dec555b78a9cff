"""The entry points under HIP graph capture (torch.cuda.graph on the caller's
stream): every replay must give the eager result bit for bit.  Covered:
the plain, bias+ReLU, grouped, batched (with a broadcast operand) and fp32
GEMMs, the attention scores, both forms of the convolution (implicit GEMM,
and im2col into a caller's workspace followed by the GEMM) and the
allocation-free split-K.

The library makes no allocation and no memset on the stream, so a captured
call is just its kernels.  The allocation-free split-K exists for callers
that capture (its partials live in the library's static scratch array); it
is first called once outside capture, which takes the array's device
address, as a caller that captures would.  Each graph is replayed several
times with the outputs cleared and other GPU work run between replays, and
every replay is checked.
"""
import numpy as np
import pytest

import tiled_matrix_multiplication_gemm_amd as mg
from tiled_matrix_multiplication_gemm_amd import inputs
from tests.gpu_util import BF16, F16, announce, to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mg.lib()
    yield


def replay_and_check(calls, outs):
    """Capture `calls` into one graph on a side stream, then replay it
    REPLAYS times; before each replay the outputs are cleared (a fill
    kernel, not a memset node) and unrelated work runs, and after it every
    output must equal its eager value."""
    import torch

    for c in calls:
        c()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in calls:  # warm-up on the capture stream
            c()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    noise = torch.randn(1 << 20, device="cuda")
    for r in range(REPLAYS):
        for o in outs:
            o.zero_()
        noise.mul_(1.0001).add_(0.5)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outs, want)):
            assert torch.equal(o, w), "replay %d, output %d differs from the eager result" % (r, i)


def test_gemm_bias_relu_and_grouped_in_one_graph():
    import torch

    announce("graph: gemm 1024x1024x2048 f16, bias+relu, grouped E=8")
    c1 = inputs.random_dense(1024, 1024, 2048, F16, 8101)
    c2 = inputs.random_dense(520, 264, 200, BF16, 8102, epilogue=True)
    g = inputs.random_grouped(E=8, T=1100, K=256, N=264, dtype=F16, seed=8103)
    A1, B1 = to_dev(c1.A, F16), to_dev(c1.B, F16)
    A2, B2, b2 = to_dev(c2.A, BF16), to_dev(c2.B, BF16), to_dev(c2.bias, BF16)
    X, W = to_dev(g.X, F16), to_dev(g.W, F16)
    off = torch.from_numpy(g.offsets.astype(np.int32)).cuda()
    C1 = torch.empty((1024, 1024), dtype=torch.float16, device="cuda")
    C2 = torch.empty((520, 264), dtype=torch.bfloat16, device="cuda")
    Y = torch.empty((g.T, g.N), dtype=torch.float16, device="cuda")
    replay_and_check([lambda: mg.mg_gemm(A1, B1, out=C1),
                      lambda: mg.mg_gemm_bias_relu(A2, B2, b2, out=C2),
                      lambda: mg.mg_grouped_gemm(X, W, off, out=Y)], [C1, C2, Y])


@pytest.mark.parametrize("M,N,K,splits", [(1024, 1024, 2048, 4), (256, 256, 65536, 16)])
def test_splitk_noalloc_in_a_graph(M, N, K, splits):
    import torch

    announce("graph: split-K without allocation %dx%dx%d, %d splits" % (M, N, K, splits))
    c = inputs.random_dense(M, N, K, BF16, 8200 + splits)
    A, B = to_dev(c.A, BF16), to_dev(c.B, BF16)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    assert mg.mg_splitk_workspace_bytes(M, N, splits) <= mg.mg_splitk_noalloc_max_bytes()
    mg.mg_gemm_splitk_noalloc(A, B, splits=splits, out=C)  # outside capture: takes the scratch address
    torch.cuda.synchronize()
    eager_ws = torch.empty((mg.mg_splitk_workspace_bytes(M, N, splits),), dtype=torch.uint8, device="cuda")
    ref = mg.mg_gemm_splitk(A, B, splits=splits, workspace=eager_ws)
    torch.cuda.synchronize()
    replay_and_check([lambda: mg.mg_gemm_splitk_noalloc(A, B, splits=splits, out=C)], [C])
    assert torch.equal(C, ref), "the graph's result differs from the workspace form"


def test_batched_attention_conv_and_fp32_in_one_graph():
    import torch

    announce("graph: batched (broadcast B), attention scores, conv implicit + im2col, fp32 gemm")
    g = torch.Generator(device="cuda").manual_seed(8300)
    def rnd(*shape, dtype=torch.float16, scale=0.1):
        return (torch.randn(*shape, device="cuda", generator=g) * scale).to(dtype)
    a3 = rnd(6, 300, 136, dtype=torch.bfloat16)
    b3 = rnd(1, 136, 264, dtype=torch.bfloat16).expand(6, 136, 264)  # one B for every entry (stride 0)
    c3 = torch.empty((6, 300, 264), dtype=torch.bfloat16, device="cuda")
    q = rnd(8, 384, 64)
    k = rnd(8, 320, 64)
    s = torch.empty((8, 384, 320), dtype=torch.float16, device="cuda")
    x1, w1 = rnd(2, 17, 15, 64), rnd(3, 3, 64, 64)      # C % 32 == 0: implicit GEMM, no workspace
    y1 = torch.empty((2, 17, 15, 64), dtype=torch.float16, device="cuda")
    x2, w2 = rnd(2, 13, 11, 40), rnd(3, 3, 40, 48)      # C = 40: im2col into the workspace, then the GEMM
    y2 = torch.empty((2, 13, 11, 48), dtype=torch.float16, device="cuda")
    shape2 = mg.conv2d_shape(x2.shape, (3, 3), 48, 1, 1, 1)
    need = mg.mg_conv2d_workspace_bytes(shape2, mg.MG_F16)
    assert need > 0, "the C = 40 case should take the im2col path"
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    assert mg.mg_conv2d_workspace_bytes(mg.conv2d_shape(x1.shape, (3, 3), 64, 1, 1, 1), mg.MG_F16) == 0
    af, bf = rnd(200, 96, dtype=torch.float32, scale=1.0), rnd(96, 132, dtype=torch.float32, scale=1.0)
    cf = torch.empty((200, 132), dtype=torch.float32, device="cuda")
    replay_and_check([lambda: mg.mg_gemm_batched(a3, b3, out=c3),
                      lambda: mg.mg_attention_scores(q, k, out=s),
                      lambda: mg.mg_conv2d(x1, w1, 1, 1, 1, out=y1),
                      lambda: mg.mg_conv2d(x2, w2, 1, 1, 1, workspace=ws, out=y2),
                      lambda: mg.mg_gemm(af, bf, out=cf)], [c3, s, y1, y2, cf])
