"""Seeded random shapes through the automatic row choice, against the oracle.

The other parity tests force each table row on chosen shapes; here the
library picks the row itself (swept shapes from the cached best, the rest
from the time model), so the selection and every row it can return are
exercised together on shapes nobody picked by hand.  M, N and K are drawn
log-uniformly (M up to 2^17, N up to 2^14, K up to about 5800), within
bounds that keep each case to a few seconds of oracle time, and about half
the cases are integer-valued (bit-exact gate), the rest random floats
(1e-2 gate plus Higham's bound).  Every output element is compared.

Grouped launches get the same treatment: 1 to about 160 experts, up to
about 23000 tokens split by a Dirichlet-multinomial draw (concentration
0.2, 1 or 20: from a few experts holding almost every token, with many
empty ones, to near-equal counts), N and K log-uniform.  Split-K takes the
library's own split count and workspace, batched products share A or B
across entries (batch stride 0) in some of the cases, convolutions reach
each of the three ways the library runs one, dense products also take
transposed operands, and attention scores span head counts, lengths and
head dimensions.
"""
import numpy as np
import pytest

import tiled_matrix_multiplication_gemm_amd as mg
from tiled_matrix_multiplication_gemm_amd import inputs
from tests.gpu_util import Guarded, announce, assert_bitexact, assert_tolerance, to_dev
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


GROUPED_SEED = 7
GROUPED_COUNT = 24


def draw_grouped_cases(seed=GROUPED_SEED, count=GROUPED_COUNT):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        E = int(np.exp2(rng.uniform(0, 7.3)))
        T = int(np.exp2(rng.uniform(0, 14.5)))
        N = int(np.exp2(rng.uniform(3, 12.5)))
        K = int(np.exp2(rng.uniform(3, 11.5)))
        if T * N * K > 4e9 or E * K * N > 3e7 or T * K > 2e7 or T * N > 3e7:
            continue
        alpha = float(rng.choice([0.2, 1.0, 20.0]))
        counts = rng.multinomial(T, rng.dirichlet([alpha] * E))
        dtype = int(rng.integers(0, 2))
        integer = bool(rng.integers(0, 2))
        cases.append((E, T, N, K, tuple(int(c) for c in counts), dtype, integer, int(rng.integers(0, 2**31))))
    return cases


GROUPED_CASES = draw_grouped_cases()


def test_grouped_draws_spread_over_rows_and_counts():
    """Several rows; count vectors with empty experts and with experts of more
    than one 256-row tile; and launches of 64 or more experts."""
    rows = {mg.mg_select_config(T, N, K, dt, E) for E, T, N, K, _, dt, *_ in GROUPED_CASES}
    assert len(rows) >= 4 and rows <= {0, 1, 2, 3, 4, 6, 8, 9}, sorted(rows)
    assert any(0 in g[4] for g in GROUPED_CASES)
    assert any(g[0] >= 64 for g in GROUPED_CASES)  # offsets walked from memory, not from lanes
    assert any(max(g[4]) > 256 for g in GROUPED_CASES)


def run_grouped_padded(c):
    """The grouped launch with X rows, W rows and Y rows padded to multiples
    of 8 elements (the library's stride rule), the padding of Y guarded."""
    import torch

    up8 = lambda n: (n + 7) // 8 * 8
    xp = np.zeros((c.T, up8(c.K)), dtype=np.uint16)
    xp[:, :c.K] = c.X
    wp = np.zeros((c.E, c.K, up8(c.N)), dtype=np.uint16)
    wp[:, :, :c.N] = c.W
    X = to_dev(xp, c.dtype)[:, :c.K]
    W = to_dev(wp, c.dtype)[:, :, :c.N]
    off = torch.from_numpy(c.offsets.astype(np.int32)).cuda()
    out = Guarded(c.T, c.N, c.dtype, ld=up8(c.N))
    mg.mg_grouped_gemm(X, W, off, out=out.mat)
    torch.cuda.synchronize()
    return out


@pytest.mark.gpu
@pytest.mark.parametrize("case", GROUPED_CASES, ids=lambda c: "E%d_T%d_%dx%d_%s_%s" % (
    c[0], c[1], c[2], c[3], "bf16" if c[5] else "f16", "int" if c[6] else "float"))
def test_random_grouped_auto_row(orc, _gpu, case):
    E, T, N, K, counts, dtype, integer, seed = case
    c = inputs.random_grouped(E=E, T=T, K=K, N=N, dtype=dtype, seed=seed, counts=np.array(counts), integer=integer,
                              name="random grouped")
    announce("grouped E=%d T=%d N=%d K=%d dt=%d int=%s max count %d" % (E, T, N, K, dtype, integer, max(counts)))
    out = run_grouped_padded(c)
    assert out.guards_intact(), "write outside the output"
    ref, ref_q = orc.grouped_gemm(c.X, c.W, c.offsets, dtype)
    if integer:
        assert_bitexact(out.result(), ref_q, dtype, c.name)
    else:
        assert_tolerance(out.result(), ref, dtype, c.name)
    assert mg.mg_last_kernel() == "gemm_dlds_kernel", (E, T, N, K, mg.mg_last_kernel())


# ---- split-K with the library's split count, and batched products ----------------
SPLITK_SEED = 5
SPLITK_COUNT = 16


def draw_splitk_cases(seed=SPLITK_SEED, count=SPLITK_COUNT):
    """Under-filled outputs over long K: M and N of 16 to 2048 (N a multiple
    of 8, as split-K requires), K of 512 to 32768."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        M = int(np.exp2(rng.uniform(4, 11)))
        N = int(np.exp2(rng.uniform(4, 11))) // 8 * 8
        K = int(np.exp2(rng.uniform(9, 15)))
        if M * N * K > 3e9 or M * K > 2e7 or K * N > 2e7:
            continue
        cases.append((M, N, K, int(rng.integers(0, 2)), bool(rng.integers(0, 2)), int(rng.integers(0, 2**31))))
    return cases


SPLITK_CASES = draw_splitk_cases()


def test_splitk_draws_take_several_split_counts():
    splits = {mg.mg_splitk_choose(M, N, K) for M, N, K, *_ in SPLITK_CASES}
    assert len(splits) >= 3 and max(splits) > 1, sorted(splits)


@pytest.mark.gpu
@pytest.mark.parametrize("case", SPLITK_CASES, ids=lambda c: "%dx%dx%d_%s_%s" % (
    c[0], c[1], c[2], "bf16" if c[3] else "f16", "int" if c[4] else "float"))
def test_random_splitk_chosen_splits(orc, _gpu, case):
    import torch

    M, N, K, dtype, integer, seed = case
    gen = inputs.integer_dense if integer else inputs.random_dense
    c = gen(M, N, K, dtype, seed, name="random splitk")
    splits = mg.mg_splitk_choose(M, N, K)
    announce("splitk %dx%dx%d dt=%d int=%s splits=%d" % (M, N, K, dtype, integer, splits))
    up8 = lambda n: (n + 7) // 8 * 8
    ap = np.zeros((M, up8(K)), dtype=np.uint16)
    ap[:, :K] = c.A
    A = to_dev(ap, dtype)[:, :K]
    B = to_dev(c.B, dtype)
    out = Guarded(M, N, dtype)
    mg.mg_gemm_splitk(A, B, out=out.mat)  # split count and workspace chosen by the library
    torch.cuda.synchronize()
    assert out.guards_intact(), "write outside the output"
    ref, ref_q = orc.gemm(c.A, c.B, dtype)
    if integer:
        assert_bitexact(out.result(), ref_q, dtype, c.name)
    else:
        assert_tolerance(out.result(), ref, dtype, c.name)


BATCHED_SEED = 9
BATCHED_COUNT = 16


def draw_batched_cases(seed=BATCHED_SEED, count=BATCHED_COUNT):
    """1 to 128 entries of 64 to 2048 rows and columns over K of 32 to 512
    (the shapes of attention scores and of small per-head products), with A
    or B shared by every entry (batch stride 0) in about a third of the
    cases each."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        nb = int(np.exp2(rng.uniform(0, 7)))
        M, N = (int(np.exp2(rng.uniform(6, 11))) for _ in range(2))
        K = int(np.exp2(rng.uniform(5, 9)))
        if nb * M * N * K > 3e9 or nb * (M * K + K * N + M * N) > 3e7:
            continue
        share = str(rng.choice(["none", "a", "b"]))
        cases.append((nb, M, N, K, share, int(rng.integers(0, 2)), bool(rng.integers(0, 2)),
                      int(rng.integers(0, 2**31))))
    return cases


BATCHED_CASES = draw_batched_cases()


def test_batched_draws_spread_over_rows():
    rows = {mg.mg_select_config(M, N, K, dt, 0, nb) for nb, M, N, K, _, dt, *_ in BATCHED_CASES}
    assert len(rows) >= 3 and rows <= {0, 1, 2, 3, 4, 6, 8, 9}, sorted(rows)
    assert {c[4] for c in BATCHED_CASES} == {"none", "a", "b"}


@pytest.mark.gpu
@pytest.mark.parametrize("case", BATCHED_CASES, ids=lambda c: "b%d_%dx%dx%d_share%s_%s_%s" % (
    c[0], c[1], c[2], c[3], c[4], "bf16" if c[5] else "f16", "int" if c[6] else "float"))
def test_random_batched_auto_row(orc, _gpu, case):
    import torch

    nb, M, N, K, share, dtype, integer, seed = case
    gen = inputs.integer_dense if integer else inputs.random_dense
    entries = [gen(M, N, K, dtype, seed + b, name="random batched") for b in range(nb)]
    # a shared operand is entry 0's
    A_bits = [entries[0].A if share == "a" else e.A for e in entries]
    B_bits = [entries[0].B if share == "b" else e.B for e in entries]
    announce("batched b=%d %dx%dx%d share=%s dt=%d int=%s" % (nb, M, N, K, share, dtype, integer))
    up8 = lambda n: (n + 7) // 8 * 8

    def stack(bits, rows, cols, one):
        n = 1 if one else nb
        buf = np.zeros((n, rows, up8(cols)), dtype=np.uint16)
        for i in range(n):
            buf[i, :, :cols] = bits[i]
        t = to_dev(buf, dtype)[:, :, :cols]
        return t.expand(nb, -1, -1) if one else t

    A = stack(A_bits, M, K, share == "a")
    B = stack(B_bits, K, N, share == "b")
    out = Guarded(nb * M, N, dtype, ld=up8(N))
    mg.mg_gemm_batched(A, B, out=out.mat.view(nb, M, N))
    torch.cuda.synchronize()
    assert out.guards_intact(), "write outside the output"
    got = out.result().reshape(nb, M, N)
    for b in range(nb):
        ref, ref_q = orc.gemm(A_bits[b], B_bits[b], dtype)
        if integer:
            assert_bitexact(got[b], ref_q, dtype, "batched entry %d" % b)
        else:
            assert_tolerance(got[b], ref, dtype, "batched entry %d" % b)


# ---- convolutions --------------------------------------------------------------
CONV_SEED = 2
CONV_COUNT = 20
F32 = 2


def draw_conv_cases(seed=CONV_SEED, count=CONV_COUNT):
    """NHWC convolutions with kernels of 1 to 7 taps a side, strides 1 to 3,
    padding 0 to 3 and dilation 1 or 2; in_channels a multiple of 64 in about
    half the cases (the implicit GEMM), any count otherwise (im2col, or the
    input itself for an unstrided, unpadded 1x1 kernel); HWIO or OHWI
    weights; fp16, bf16 and, now and then, fp32 (with K = KH KW C a multiple
    of 16, which the fp32 GEMM requires)."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        Nb = int(rng.integers(1, 5))
        H, W = (int(rng.integers(1, 41)) for _ in range(2))
        C = int(rng.choice([64, 128, 192])) if rng.integers(0, 2) else int(rng.integers(1, 97))
        KH, KW = (int(rng.integers(1, 8)) for _ in range(2))
        if rng.integers(0, 4) == 0:
            KH = KW = 1
        stride = tuple(int(v) for v in rng.integers(1, 4, size=2))
        pad = tuple(int(v) for v in rng.integers(0, 4, size=2))
        dil = tuple(int(v) for v in rng.integers(1, 3, size=2))
        if rng.integers(0, 4) == 0:
            stride, pad, dil = (1, 1), (0, 0), (1, 1)
        dt = F32 if rng.integers(0, 6) == 0 else int(rng.integers(0, 2))
        OC = int(rng.integers(1, 33)) * (4 if dt == F32 else 8)
        oh = (H + 2 * pad[0] - dil[0] * (KH - 1) - 1) // stride[0] + 1
        ow = (W + 2 * pad[1] - dil[1] * (KW - 1) - 1) // stride[1] + 1
        if oh < 1 or ow < 1 or Nb * oh * ow * OC * KH * KW * C > 5e8:
            continue
        K = KH * KW * C
        if dt == F32 and K % 16 != 0:  # the fp32 GEMM takes whole 16-element K slices
            continue
        weights = "ohwi" if dt != F32 and K % 8 == 0 and rng.integers(0, 3) == 0 else "hwio"
        cases.append((Nb, H, W, C, OC, KH, KW, stride, pad, dil, dt, weights, bool(rng.integers(0, 2)),
                      bool(rng.integers(0, 2)), int(rng.integers(0, 2**31))))
    return cases


CONV_CASES = draw_conv_cases()


def conv_path(case):
    Nb, H, W, C, OC, KH, KW, stride, pad, dil, dt, *_ = case
    s = mg.Conv2dShape(Nb, H, W, C, OC, KH, KW, stride[0], stride[1], pad[0], pad[1], dil[0], dil[1])
    if mg.mg_conv2d_workspace_bytes(s, dt) > 0:
        return "im2col"
    return "input" if KH == KW == 1 and stride == (1, 1) and pad == (0, 0) else "implicit"


def test_conv_draws_reach_every_path():
    paths = {conv_path(c) for c in CONV_CASES}
    assert paths == {"im2col", "input", "implicit"}, paths
    assert {c[11] for c in CONV_CASES} == {"hwio", "ohwi"}
    assert F32 in {c[10] for c in CONV_CASES}


@pytest.mark.gpu
@pytest.mark.parametrize("case", CONV_CASES, ids=lambda c: "n%d_%dx%dx%d_oc%d_k%dx%d_s%d%d_p%d%d_d%d%d_%s_%s%s%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], *c[7], *c[8], *c[9], ("f16", "bf16", "f32")[c[10]], c[11],
    "_int" if c[12] else "", "_bias" if c[13] else ""))
def test_random_conv2d(orc, _gpu, case):
    from tests.test_gpu_consumers import check, run_conv

    Nb, H, W, C, OC, KH, KW, stride, pad, dil, dt, weights, integer, with_bias, seed = case
    label = "random conv %s (%s)" % (case, conv_path(case))
    announce(label)
    c = inputs.conv_case(Nb, H, W, C, OC, KH, KW, dt, seed=seed, stride=stride, pad=pad, dil=dil, integer=integer,
                         bias=with_bias)
    got, guards = run_conv(c, OC, weights, c.bias)
    assert guards, label + ": write outside the output"
    ref, ref_q = orc.conv2d(c.x, c.w, dt, stride, pad, dil, bias=c.bias, relu=with_bias)
    absref = None
    if dt == F32 and not integer:
        xa = np.abs(orc.decode32(c.x)).astype(np.float32).view(np.uint32)
        wa = np.abs(orc.decode32(c.w)).astype(np.float32).view(np.uint32)
        absref, _ = orc.conv2d(xa, wa, F32, stride, pad, dil)
    check(got, ref, ref_q, dt, integer, label, absref, KH * KW * C)


# ---- transposed operands and attention scores ----------------------------------
TRANSPOSED_SEED = 11
TRANSPOSED_COUNT = 16


def draw_transposed_cases(seed=TRANSPOSED_SEED, count=TRANSPOSED_COUNT):
    """Dense shapes as above with A, B or both handed over as transposed views."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        M = int(np.exp2(rng.uniform(4, 14)))
        N = int(np.exp2(rng.uniform(4, 13)))
        K = int(np.exp2(rng.uniform(5, 12)))
        if M * N * K > 3e9 or M * N * K < 5e7 or M * K > 2e7 or K * N > 2e7:
            continue
        ta, tb = [(1, 0), (0, 1), (1, 1)][int(rng.integers(0, 3))]
        cases.append((M, N, K, ta, tb, int(rng.integers(0, 2)), bool(rng.integers(0, 2)), bool(rng.integers(0, 2)),
                      int(rng.integers(0, 2**31))))
    return cases


TRANSPOSED_CASES = draw_transposed_cases()


def test_transposed_draws_spread_over_rows_and_layouts():
    rows = {mg.mg_select_config(M, N, K, dt) for M, N, K, _, _, dt, *_ in TRANSPOSED_CASES}
    assert len(rows) >= 4 and rows <= {0, 1, 2, 3, 4, 6, 8, 9}, sorted(rows)
    assert {(c[3], c[4]) for c in TRANSPOSED_CASES} == {(1, 0), (0, 1), (1, 1)}


@pytest.mark.gpu
@pytest.mark.parametrize("case", TRANSPOSED_CASES, ids=lambda c: "%dx%dx%d_ta%d_tb%d_%s_%s%s" % (
    c[0], c[1], c[2], c[3], c[4], "bf16" if c[5] else "f16", "int" if c[6] else "float", "_epi" if c[7] else ""))
def test_random_transposed_auto_row(orc, _gpu, case):
    import torch
    from tests.test_gpu_parity import stored_row_major, stored_transposed

    M, N, K, ta, tb, dtype, integer, epi, seed = case
    gen = inputs.integer_dense if integer else inputs.random_dense
    c = gen(M, N, K, dtype, seed, epilogue=epi, name="random transposed")
    announce("transposed %dx%dx%d ta=%d tb=%d dt=%d int=%s epi=%s" % (M, N, K, ta, tb, dtype, integer, epi))
    A = stored_transposed(c.A, dtype) if ta else stored_row_major(c.A, dtype)
    B = stored_transposed(c.B, dtype) if tb else stored_row_major(c.B, dtype)
    out = Guarded(M, N, dtype, ld=(N + 7) // 8 * 8)
    if epi:
        mg.mg_gemm_bias_relu(A, B, to_dev(c.bias, dtype), out=out.mat)
    else:
        mg.mg_gemm(A, B, out=out.mat)
    torch.cuda.synchronize()
    assert out.guards_intact(), "write outside the output"
    ref, ref_q = orc.gemm(c.A, c.B, dtype, bias=c.bias, relu=c.relu)
    if integer:
        assert_bitexact(out.result(), ref_q, dtype, c.name)
    else:
        assert_tolerance(out.result(), ref, dtype, c.name)
    assert mg.mg_last_kernel() == "gemm_dlds_kernel"


ATTENTION_SEED = 4
ATTENTION_COUNT = 12


def draw_attention_cases(seed=ATTENTION_SEED, count=ATTENTION_COUNT):
    """1 to 64 heads, query lengths of 4 to 2048, key lengths a multiple of 8
    up to 2048 (the score rows' stride rule), head dimensions a multiple of 8
    from 8 to 256."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        H = int(np.exp2(rng.uniform(0, 6)))
        Lq = int(np.exp2(rng.uniform(2, 11)))
        Lk = max(8, int(np.exp2(rng.uniform(4, 11))) // 8 * 8)
        d = 8 * int(rng.integers(1, 33))
        if H * Lq * Lk * d > 3e9 or H * Lq * Lk > 3e7:
            continue
        cases.append((H, Lq, Lk, d, int(rng.integers(0, 2)), bool(rng.integers(0, 2)), int(rng.integers(0, 2**31))))
    return cases


ATTENTION_CASES = draw_attention_cases()


def test_attention_draws_spread_over_rows():
    rows = {mg.mg_select_config(Lq, Lk, d, dt, 0, H) for H, Lq, Lk, d, dt, *_ in ATTENTION_CASES}
    assert len(rows) >= 3 and rows <= {0, 1, 2, 3, 4, 6, 8, 9}, sorted(rows)


@pytest.mark.gpu
@pytest.mark.parametrize("case", ATTENTION_CASES, ids=lambda c: "h%d_lq%d_lk%d_d%d_%s_%s" % (
    c[0], c[1], c[2], c[3], "bf16" if c[4] else "f16", "int" if c[5] else "float"))
def test_random_attention_scores(orc, _gpu, case):
    from tests.test_gpu_consumers import check, run_attention

    H, Lq, Lk, d, dtype, integer, seed = case
    label = "random attention %s" % (case,)
    announce(label)
    a = inputs.attention_case(H, Lq, Lk, d, dtype, seed=seed, integer=integer)
    got, guards = run_attention(a)
    assert guards, label + ": write outside the output"
    ref, ref_q = orc.attention_scores(a.Q, a.K, dtype)
    check(got, ref, ref_q, dtype, integer, label)
