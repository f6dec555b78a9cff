"""Pins of the oracle's GEMM consumers: 2-D convolution, im2col and attention
scores (CPU only).

The convolution is pinned by hand-derived worked examples, by torch's own
float64 CPU convolution (another implementation and summation order; exact on
integer inputs), by its reductions (a 1x1 convolution is the GEMM oracle; a
centred identity kernel copies the input), and by the all-ones closed form
(each output counts its in-image taps times C).  im2col is pinned by worked
examples and by "GEMM of im2col = convolution".  Attention scores are pinned
by brute force, by the symmetry of X X^T and by S(Q,K) = S(K,Q)^T.
"""
import itertools

import numpy as np
import pytest

from oracle import layout
from tiled_matrix_multiplication_gemm_amd import inputs

F16, BF16, F32 = 0, 1, 2


def bits(x, dtype):
    x = np.asarray(x, dtype=np.float64)
    if dtype == F32:
        return x.astype(np.float32).view(np.uint32)
    return inputs.to_bits(x, dtype)


def values(b, dtype):
    b = np.asarray(b)
    if dtype == F32:
        return b.view(np.float32).astype(np.float64)
    if dtype == F16:
        return b.view(np.float16).astype(np.float64)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def torch_conv(xd, wd, stride, pad, dil):
    """torch's float64 CPU convolution on NHWC / [KH,KW,C,OC] data, NHWC out."""
    import torch

    x = torch.from_numpy(xd).permute(0, 3, 1, 2)
    w = torch.from_numpy(wd).permute(3, 2, 0, 1)
    y = torch.nn.functional.conv2d(x, w, stride=stride, padding=pad, dilation=dil)
    return y.permute(0, 2, 3, 1).contiguous().numpy()


def image(vals, dtype=F16):
    """A one-image, one-channel NHWC batch from a 2-D list."""
    return bits(np.asarray(vals, dtype=np.float64)[None, :, :, None], dtype)


def test_conv_worked_examples(orc):
    x = image([[1, 2, 3], [4, 5, 6], [7, 8, 9]])
    w = bits(np.array([[1, 0], [0, -1]], dtype=np.float64)[:, :, None, None], F16)
    # valid positions: x[i,j] - x[i+1,j+1] = -4 everywhere
    ref, ref_q = orc.conv2d(x, w, F16)
    assert ref[0, :, :, 0].tolist() == [[-4.0, -4.0], [-4.0, -4.0]]
    assert values(ref_q, F16)[0, :, :, 0].tolist() == [[-4.0, -4.0], [-4.0, -4.0]]
    # padding 1, stride 2: windows start at (-1,-1), (-1,1), (1,-1), (1,1)
    ref, _ = orc.conv2d(x, w, F16, stride=(2, 2), pad=(1, 1))
    assert ref[0, :, :, 0].tolist() == [[-1.0, -3.0], [-7.0, -4.0]]
    # dilation 2 on a 3x3 image: the only window takes the four corners
    ref, _ = orc.conv2d(x, w, F16, dil=(2, 2))
    assert ref[0, :, :, 0].tolist() == [[1.0 - 9.0]]


CONV_PARAMS = [
    # (Nb, H, W, C, OC, KH, KW, stride, pad, dil)
    (1, 5, 5, 1, 1, 3, 3, (1, 1), (0, 0), (1, 1)),
    (2, 7, 6, 3, 4, 3, 3, (1, 1), (1, 1), (1, 1)),
    (1, 9, 8, 2, 3, 2, 3, (2, 1), (1, 2), (1, 1)),
    (2, 11, 10, 4, 2, 3, 2, (2, 2), (3, 0), (2, 1)),
    (1, 8, 12, 3, 5, 1, 5, (1, 3), (0, 2), (1, 2)),
    (1, 13, 13, 2, 2, 7, 7, (2, 2), (3, 3), (1, 1)),
]


@pytest.mark.parametrize("p", CONV_PARAMS)
@pytest.mark.parametrize("dtype", [F16, BF16, F32])
def test_conv_matches_torch_float64(orc, p, dtype):
    Nb, H, W, C, OC, KH, KW, stride, pad, dil = p
    rng = np.random.default_rng(hash((p, dtype)) & 0xFFFF)
    # integer inputs: every sum is exact, so any correct order gives the same value
    xi = bits(rng.integers(-4, 5, (Nb, H, W, C)), dtype)
    wi = bits(rng.integers(-4, 5, (KH, KW, C, OC)), dtype)
    ref, _ = orc.conv2d(xi, wi, dtype, stride, pad, dil)
    want = torch_conv(values(xi, dtype), values(wi, dtype), stride, pad, dil)
    assert ref.shape == want.shape
    assert np.array_equal(ref, want)
    # float inputs: another summation order, agreement far inside fp64 error
    xf = bits(rng.standard_normal((Nb, H, W, C)), dtype)
    wf = bits(rng.standard_normal((KH, KW, C, OC)), dtype)
    xd, wd = values(xf, dtype), values(wf, dtype)
    ref, ref_q = orc.conv2d(xf, wf, dtype, stride, pad, dil)
    want = torch_conv(xd, wd, stride, pad, dil)
    scale = torch_conv(np.abs(xd), np.abs(wd), stride, pad, dil)
    assert np.all(np.abs(ref - want) <= 1e-12 * scale + 1e-300)
    assert np.array_equal(ref_q, orc._encode_any(ref, dtype))


@pytest.mark.parametrize("dtype", [F16, F32])
def test_conv_1x1_is_the_gemm(orc, dtype):
    rng = np.random.default_rng(5)
    x = bits(rng.standard_normal((2, 5, 7, 6)), dtype)
    w = bits(rng.standard_normal((1, 1, 6, 9)), dtype)
    ref, ref_q = orc.conv2d(x, w, dtype)
    A, B = x.reshape(-1, 6), w.reshape(6, 9)
    g, gq = orc.gemm_f32(A, B) if dtype == F32 else orc.gemm(A, B, dtype)
    assert np.array_equal(ref.reshape(-1, 9), g)
    assert np.array_equal(ref_q.reshape(-1, 9), gq)


def test_conv_centred_identity_kernel_copies_the_input(orc):
    rng = np.random.default_rng(6)
    C = 5
    x = bits(rng.standard_normal((2, 6, 4, C)), F16)
    w = np.zeros((3, 3, C, C))
    w[1, 1] = np.eye(C)
    ref, ref_q = orc.conv2d(x, bits(w, F16), F16, pad=(1, 1))
    assert np.array_equal(ref, values(x, F16))
    assert np.array_equal(ref_q, x)


@pytest.mark.parametrize("p", CONV_PARAMS)
def test_conv_all_ones_counts_taps(orc, p):
    Nb, H, W, C, OC, KH, KW, stride, pad, dil = p
    x = bits(np.ones((Nb, H, W, C)), F16)
    w = bits(np.ones((KH, KW, C, OC)), F16)
    ref, _ = orc.conv2d(x, w, F16, stride, pad, dil)
    OH, OW = ref.shape[1:3]
    for oh, ow in itertools.product(range(OH), range(OW)):
        rows = sum(0 <= oh * stride[0] - pad[0] + kh * dil[0] < H for kh in range(KH))
        cols = sum(0 <= ow * stride[1] - pad[1] + kw * dil[1] < W for kw in range(KW))
        assert np.all(ref[:, oh, ow, :] == rows * cols * C)


def test_conv_output_size_matches_torch(orc):
    import torch

    for (H, KH, s, p, d) in itertools.product([1, 5, 8, 17], [1, 2, 3, 7], [1, 2, 3], [0, 1, 3], [1, 2]):
        if H + 2 * p - d * (KH - 1) - 1 < 0:
            continue
        oh, ow = orc.conv_out_hw(H, H + 1, KH, KH, (s, s), (p, p), (d, d))
        y = torch.nn.functional.conv2d(torch.zeros(1, 1, H, H + 1), torch.zeros(1, 1, KH, KH), stride=s, padding=p,
                                       dilation=d)
        assert (oh, ow) == tuple(y.shape[2:])


def test_conv_bias_relu(orc):
    rng = np.random.default_rng(7)
    x = bits(np.zeros((1, 4, 4, 3)), F16)
    w = bits(rng.standard_normal((3, 3, 3, 6)), F16)
    bias = bits([-2.0, -0.5, 0.0, 0.25, 1.5, 3.0], F16)
    ref, ref_q = orc.conv2d(x, w, F16, pad=(1, 1), bias=bias, relu=True)
    want = np.maximum(values(bias, F16), 0.0)
    assert np.array_equal(ref, np.broadcast_to(want, ref.shape))
    assert np.all(ref_q[..., :3] == 0)  # ReLU of a non-positive value is the +0.0 pattern


def test_conv_sampled_equals_full(orc):
    rng = np.random.default_rng(8)
    x = bits(rng.standard_normal((2, 9, 7, 4)), BF16)
    w = bits(rng.standard_normal((3, 2, 4, 5)), BF16)
    bias = bits(rng.standard_normal(5), BF16)
    ref, ref_q = orc.conv2d(x, w, BF16, (2, 1), (1, 1), (1, 2), bias=bias, relu=True)
    M = ref.shape[0] * ref.shape[1] * ref.shape[2]
    rows = rng.integers(0, M, 50)
    cols = rng.integers(0, 5, 50)
    s, sq = orc.conv2d(x, w, BF16, (2, 1), (1, 1), (1, 2), bias=bias, relu=True, rows=rows, cols=cols)
    assert np.array_equal(s, ref.reshape(M, 5)[rows, cols])
    assert np.array_equal(sq, ref_q.reshape(M, 5)[rows, cols])


def test_im2col_worked_examples():
    x = np.arange(1, 10, dtype=np.uint16).reshape(1, 3, 3, 1)
    assert layout.im2col(x, 2, 2).tolist() == [[1, 2, 4, 5], [2, 3, 5, 6], [4, 5, 7, 8], [5, 6, 8, 9]]
    # padding 1, stride 2: windows at (-1,-1), (-1,1), (1,-1), (1,1); outside = 0
    assert layout.im2col(x, 2, 2, (2, 2), (1, 1)).tolist() == [[0, 0, 0, 1], [0, 0, 2, 3], [0, 4, 0, 7],
                                                                 [5, 6, 8, 9]]
    # two channels interleave per tap: column k = (kh KW + kw) C + c
    x2 = np.stack([x[..., 0], 10 * x[..., 0]], axis=-1)
    assert layout.im2col(x2, 1, 2)[0].tolist() == [1, 10, 2, 20]


@pytest.mark.parametrize("p", CONV_PARAMS)
def test_gemm_of_im2col_is_the_convolution(orc, p):
    Nb, H, W, C, OC, KH, KW, stride, pad, dil = p
    rng = np.random.default_rng(11)
    x = bits(rng.standard_normal((Nb, H, W, C)), F16)
    w = bits(rng.standard_normal((KH, KW, C, OC)), F16)
    cols = layout.im2col(x, KH, KW, stride, pad, dil)
    g, gq = orc.gemm(np.ascontiguousarray(cols), np.ascontiguousarray(w.reshape(KH * KW * C, OC)), F16)
    ref, ref_q = orc.conv2d(x, w, F16, stride, pad, dil)
    # same products in the same k order: identical sums
    assert np.array_equal(g, ref.reshape(g.shape))
    assert np.array_equal(gq, ref_q.reshape(g.shape))


def test_attention_scores_brute_force(orc):
    rng = np.random.default_rng(12)
    Q = bits(rng.integers(-4, 5, (3, 4, 5)), F16)
    K = bits(rng.integers(-4, 5, (3, 6, 5)), F16)
    ref, ref_q = orc.attention_scores(Q, K, F16)
    q, k = values(Q, F16), values(K, F16)
    for h, i, j in itertools.product(range(3), range(4), range(6)):
        assert ref[h, i, j] == sum(q[h, i, t] * k[h, j, t] for t in range(5))
    assert np.array_equal(values(ref_q, F16), ref)


def test_attention_scores_symmetry_and_transpose(orc):
    rng = np.random.default_rng(13)
    X = bits(rng.standard_normal((2, 7, 16)), BF16)
    Y = bits(rng.standard_normal((2, 5, 16)), BF16)
    s, _ = orc.attention_scores(X, X, BF16)
    assert np.array_equal(s, s.transpose(0, 2, 1))
    a, _ = orc.attention_scores(X, Y, BF16)
    b, _ = orc.attention_scores(Y, X, BF16)
    assert np.array_equal(a, b.transpose(0, 2, 1))


def test_attention_scores_sampled_equals_full(orc):
    rng = np.random.default_rng(14)
    Q = bits(rng.standard_normal((4, 9, 8)), F16)
    K = bits(rng.standard_normal((4, 11, 8)), F16)
    ref, ref_q = orc.attention_scores(Q, K, F16)
    h, i, j = rng.integers(0, 4, 40), rng.integers(0, 9, 40), rng.integers(0, 11, 40)
    s, sq = orc.attention_scores_sampled(Q, K, F16, h, i, j)
    assert np.array_equal(s, ref[h, i, j])
    assert np.array_equal(sq, ref_q[h, i, j])
