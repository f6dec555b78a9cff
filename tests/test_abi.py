"""C-ABI contract checks that need no GPU: the library loads, exports every
function include/mi355gemm.h declares, and rejects bad arguments with the
documented status codes before making any HIP call.  No kernel is launched
here: every call either fails validation or is a documented no-op."""
import ctypes
import os
import re
import subprocess

import pytest

import tiled_matrix_multiplication_gemm_amd as mg
from oracle import layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mi355gemm.h")

OK, INVALID, DTYPE, LAYOUT, MISALIGNED, HIP, BADCFG = range(7)
F16, BF16 = 0, 1
P = 0x10000      # a 16-byte aligned stand-in address; never dereferenced below
S = ctypes.c_void_p(0)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mg_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mg.LIB_PATH):
        pytest.skip("library not built")
    return mg.lib()


def test_header_and_exports_agree(L):
    names = declared_functions()
    assert set(names) == set(mg.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", mg.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(re.findall(r"\bT (mg_[a-z0-9_]+)\b", out.stdout))
    for n in names:
        assert n in exported, n
        assert hasattr(L, n)


def gemm(L, A=P, B=P, C=P, M=64, N=64, K=64, sam=64, sak=1, sbk=64, sbn=1, scm=64, scn=1, din=F16, dout=F16):
    return L.mg_gemm(A, B, C, M, N, K, sam, sak, sbk, sbn, scm, scn, din, dout, S)


def test_status_strings(L):
    for s in range(7):
        assert L.mg_status_string(s).decode().startswith("MG_")
    assert b"unknown" in L.mg_status_string(99)


@pytest.mark.parametrize("kw,status", [
    (dict(A=None), INVALID), (dict(B=None), INVALID), (dict(C=None), INVALID),
    (dict(M=-1), INVALID), (dict(N=-5), INVALID), (dict(K=-1), INVALID),
    (dict(din=3, dout=3), DTYPE), (dict(din=F16, dout=BF16), DTYPE), (dict(din=7, dout=F16), DTYPE),
    (dict(din=2, dout=F16), DTYPE), (dict(din=2, dout=2, sam=66), MISALIGNED), (dict(din=2, dout=2, sak=2), LAYOUT),
    (dict(din=2, dout=2, sam=1, sak=64), LAYOUT), (dict(din=2, dout=2, K=40), LAYOUT), (dict(din=2, dout=2, N=62, sbk=64, scm=64), LAYOUT),
    (dict(sak=2), LAYOUT), (dict(sbn=64), LAYOUT), (dict(scn=0), LAYOUT),
    (dict(sam=32), LAYOUT), (dict(sbk=8), LAYOUT),
    (dict(A=P + 2), MISALIGNED), (dict(B=P + 8), MISALIGNED), (dict(C=P + 4), MISALIGNED),
    (dict(sam=68), MISALIGNED), (dict(scm=100), MISALIGNED),
    # transposed operands (unit stride along M for A, along K for B)
    (dict(sam=1, sak=32), LAYOUT), (dict(sam=1, sak=68), MISALIGNED), (dict(sbk=1, sbn=32), LAYOUT),
    (dict(sbk=1, sbn=68), MISALIGNED),
])
def test_gemm_rejects_bad_arguments(L, kw, status):
    assert gemm(L, **kw) == status


def test_transposed_operands_need_a_direct_row(L):
    # rows without a direct-to-LDS kernel (general-only, K split) refuse transposed operands
    for cid in (5, 7):
        assert L.mg_set_config(cid) == OK
        try:
            assert gemm(L, sam=1, sak=64) == LAYOUT
            assert gemm(L, sbk=1, sbn=64) == LAYOUT
        finally:
            assert L.mg_set_config(-1) == OK


def gemm_batched(L, batch=2, A=P, B=P, C=P, M=64, N=64, K=64, sam=64, sak=1, sbk=64, sbn=1, scm=64, scn=1,
                 sab=4096, sbb=4096, scb=4096, din=F16, dout=F16):
    return L.mg_gemm_batched(A, B, C, batch, M, N, K, sam, sak, sbk, sbn, scm, scn, sab, sbb, scb, din, dout, S)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=-1), INVALID), (dict(sab=-8), INVALID), (dict(scb=-4096), INVALID),
    (dict(scb=64 * 63), LAYOUT), (dict(sab=4100), MISALIGNED), (dict(sbb=12), MISALIGNED),
    (dict(scb=4100), MISALIGNED), (dict(sak=2), LAYOUT), (dict(A=None), INVALID),
])
def test_gemm_batched_rejects_bad_arguments(L, kw, status):
    assert gemm_batched(L, **kw) == status


def test_gemm_batched_empty_batches_are_noops(L):
    assert gemm_batched(L, batch=0, A=None, B=None, C=None) == OK
    assert gemm_batched(L, M=0, A=None, C=None) == OK


def test_splitk_workspace_and_arguments(L):
    assert L.mg_splitk_workspace_bytes(64, 32, 4) == 4 * 64 * 32 * 4
    assert L.mg_splitk_workspace_bytes(0, 32, 4) == 0
    assert L.mg_splitk_workspace_bytes(64, 32, 0) == 0
    W = P + 4096 * 1024

    def splitk(ws=W, nbytes=1 << 20, splits=2, **kw):
        a = dict(M=64, N=64, K=64, sam=64, sak=1, sbk=64, sbn=1, scm=64, scn=1)
        a.update(kw)
        return L.mg_gemm_splitk(P, P, P, ws, nbytes, splits, a["M"], a["N"], a["K"], a["sam"], a["sak"], a["sbk"],
                                a["sbn"], a["scm"], a["scn"], F16, F16, S)

    assert splitk(splits=0) == INVALID
    assert splitk(splits=5000) == INVALID
    assert splitk(ws=None) == INVALID
    assert splitk(nbytes=2 * 64 * 64 * 4 - 1) == INVALID
    assert splitk(ws=W + 8) == MISALIGNED
    assert splitk(sak=2) == LAYOUT
    assert splitk(M=0) == OK
    for cid in (5, 7):  # rows without a direct-to-LDS kernel cannot split
        assert L.mg_set_config(cid) == OK
        try:
            assert splitk() == LAYOUT
        finally:
            assert L.mg_set_config(-1) == OK


def test_splitk_choice_model(L):
    ch = L.mg_splitk_choose
    # outputs that fill the GPU are not split; tall-skinny, large-K ones are
    assert ch(8192, 8192, 8192) == 1 and ch(1024, 1024, 2048) == 1
    assert ch(256, 256, 65536) >= 8 and ch(2048, 2048, 16384) >= 2
    for shape in [(256, 256, 65536), (64, 64, 4096), (512, 512, 32768), (128, 4096, 16384)]:
        s = ch(*shape)
        assert s >= 1 and s & (s - 1) == 0 and (s == 1 or shape[2] // s >= 256)
    assert ch(0, 8, 8) == 1 and ch(8, 8, 0) == 1


def test_f32_only_on_the_plain_gemm(L):
    F32 = 2
    assert gemm_batched(L, din=F32, dout=F32) == DTYPE
    assert L.mg_gemm_splitk(P, P, P, P, 1 << 20, 2, 64, 64, 64, 64, 1, 64, 1, 64, 1, F32, F32, S) == DTYPE
    assert L.mg_prepack_a(P, P, 64, 64, 64, 64, F32, S) == DTYPE


def test_zero_sized_problems_are_noops(L):
    # M == 0 or N == 0: nothing to compute, null pointers are fine
    assert gemm(L, A=None, C=None, M=0) == OK
    assert gemm(L, B=None, C=None, N=0) == OK
    assert gemm(L, A=None, B=None, C=None, M=0, N=0, K=0) == OK


def test_bias_relu_requires_bias(L):
    assert L.mg_gemm_bias_relu(P, P, None, P, 8, 8, 8, 8, 1, 8, 1, 8, 1, F16, F16, S) == INVALID
    assert L.mg_gemm_bias_relu(P, P, None, P, 0, 8, 8, 8, 1, 8, 1, 8, 1, F16, F16, S) == OK


def grouped(L, X=P, W=P, Y=P, off=P, E=4, T=64, N=64, K=64, sxm=64, swe=64 * 64, swk=64, sym=64, dt=F16):
    return L.mg_grouped_gemm(X, W, Y, off, E, T, N, K, sxm, swe, swk, sym, dt, S)


@pytest.mark.parametrize("kw,status", [
    (dict(E=-1), INVALID), (dict(T=-1), INVALID), (dict(off=None), INVALID), (dict(X=None), INVALID),
    (dict(W=None), INVALID), (dict(Y=None), INVALID), (dict(E=0), INVALID), (dict(dt=5), DTYPE),
    (dict(swe=64 * 63), LAYOUT), (dict(swe=64 * 64 + 4), MISALIGNED), (dict(sxm=60), LAYOUT),
    (dict(sym=72 + 1), MISALIGNED), (dict(X=P + 2), MISALIGNED),
])
def test_grouped_rejects_bad_arguments(L, kw, status):
    assert grouped(L, **kw) == status


def test_tile_counts_beyond_31_bits_are_refused(L):
    """Launches are sized in 64 bits and refused (MG_ERR_INVALID_ARG, before
    any HIP call) when their tile count does not fit 31 bits, however the
    count would wrap if narrowed first: a square output of 2^36 rows and
    columns (2^56 tiles), a tile-row count alone past 2^31 (M = 2^45), fp32
    and batched forms, and grouped launches whose token count, expert count
    or column count push the worst-case tile count past 2^31."""
    big = 1 << 36
    assert gemm(L, M=big, N=big, sbk=big, scm=big) == INVALID
    assert gemm(L, M=1 << 45) == INVALID
    assert gemm(L, M=1 << 45, din=2, dout=2) == INVALID
    assert gemm_batched(L, batch=(1 << 31) - 1, M=4096, N=4096, sbk=4096, scm=4096, sab=0, sbb=0,
                        scb=4096 * 4096) == INVALID
    t = (1 << 31) - 1
    assert grouped(L, E=t, T=t) == INVALID
    assert grouped(L, E=2, T=t, N=big, swk=big, swe=64 * big, sym=big) == INVALID


def test_grouped_empty_is_noop(L):
    assert grouped(L, T=0, X=None, Y=None, off=None) == OK
    assert grouped(L, E=0, T=0, X=None, W=None, Y=None, off=None) == OK


def test_prepack_arguments(L):
    assert L.mg_prepack_a(P, P, 64, 64, 64, 48, F16, S) == BADCFG
    assert L.mg_prepack_a(P, None, 64, 64, 64, 64, F16, S) == INVALID
    assert L.mg_prepack_a(P, P + 8, 64, 64, 64, 64, F16, S) == MISALIGNED
    assert L.mg_prepack_a(None, None, 0, 64, 64, 64, F16, S) == OK
    assert L.mg_prepacked_bytes(100, 130, 64, F16) == 3 * 100 * 64 * 2
    assert L.mg_prepacked_bytes(0, 130, 64, F16) == 0
    bk = L.mg_config_bk(8192, 8192, 8192, BF16)
    assert bk in (32, 64)
    # a BK the selected configuration does not use is refused
    assert L.mg_gemm_prepacked(P, 16, P, P, 64, 64, 64, 64, 1, 64, 1, F16, S) == BADCFG


def test_config_table(L):
    n = L.mg_num_configs()
    assert n >= 1
    for i in range(n):
        d = mg.mg_config_info(i)
        assert d["id"] == i
        assert d["bm"] % (32 * d["waves_m"]) == 0 and d["bn"] % (32 * d["waves_n"]) == 0
        assert d["bk"] in (32, 64) and d["stages"] >= 2
        # LDS use follows the pages' budget formula and fits gfx950's 160 KB per CU
        assert d["lds_bytes"] == layout.lds_bytes(d["bm"], d["bn"], d["bk"], 2, d["stages"])
        assert d["lds_bytes"] <= 160 * 1024
        # per-lane accumulator registers of one wave: (BM/Wm)*(BN/Wn)/64 fp32
        acc = (d["bm"] // d["waves_m"]) * (d["bn"] // d["waves_n"]) // 64
        assert acc <= 256
        if d["direct_lds"]:
            assert d["direct_bk"] in (32, 64) and d["direct_stages"] >= 2
            # one ring per wave when the waves split K
            assert d["direct_ksplit"] >= 1
            assert d["direct_lds_bytes"] == d["direct_ksplit"] * layout.lds_bytes(d["bm"], d["bn"], d["direct_bk"], 2,
                                                                                 d["direct_stages"])
            assert d["direct_lds_bytes"] <= 160 * 1024
    with pytest.raises(RuntimeError):
        mg.mg_config_info(n)
    assert L.mg_set_config(n) == BADCFG
    assert L.mg_set_config(-2) == BADCFG
    assert L.mg_set_config(-1) == OK


def test_table_selection_for_the_workloads(L):
    sel = lambda *a: L.mg_select_config(*a)
    big = mg.mg_config_info(sel(8192, 8192, 8192, BF16, 0, 1))
    assert big["bm"] * big["bn"] >= 128 * 128
    mid = mg.mg_config_info(sel(1024, 1024, 2048, F16, 0, 1))
    # a 1024 x 1024 output must still give every CU at least one tile
    assert (1024 // mid["bm"]) * (1024 // mid["bn"]) >= 128
    for cid in range(L.mg_num_configs()):
        assert L.mg_set_config(cid) == OK
        assert L.mg_select_config(8192, 8192, 8192, BF16, 0, 1) == cid
    assert L.mg_set_config(-1) == OK


# ---- GEMM consumers: convolution, im2col, attention scores -------------------
def shape(**kw):
    d = dict(batch=2, height=16, width=16, in_channels=64, out_channels=64, kernel_h=3, kernel_w=3, stride_h=1,
             stride_w=1, pad_h=1, pad_w=1, dilation_h=1, dilation_w=1)
    d.update(kw)
    return mg.Conv2dShape(**d)


def test_conv_output_size(L):
    oh, ow = ctypes.c_int64(), ctypes.c_int64()
    for kw, want in [(dict(), (16, 16)), (dict(stride_h=2, stride_w=2), (8, 8)), (dict(pad_h=0, pad_w=0), (14, 14)),
                     (dict(dilation_h=2, pad_w=0), (14, 14)), (dict(kernel_h=7, kernel_w=1, pad_h=3, pad_w=0), (16, 16)),
                     (dict(height=5, width=6, stride_h=3, stride_w=3, pad_h=0, pad_w=0), (1, 2))]:
        assert L.mg_conv2d_output_hw(ctypes.byref(shape(**kw)), ctypes.byref(oh), ctypes.byref(ow)) == OK
        assert (oh.value, ow.value) == want
    for kw, status in [(dict(kernel_h=0), INVALID), (dict(stride_w=0), INVALID), (dict(dilation_h=0), INVALID),
                       (dict(pad_h=-1), INVALID), (dict(batch=-1), INVALID), (dict(in_channels=-2), INVALID),
                       (dict(height=2, pad_h=0), INVALID),  # a 3-tall kernel does not fit a 2-tall image
                       (dict(height=1 << 30), LAYOUT), (dict(kernel_h=300, kernel_w=300, height=400, width=400), LAYOUT),
                       (dict(batch=1 << 20, height=4096, width=4096), LAYOUT)]:
        assert L.mg_conv2d_output_hw(ctypes.byref(shape(**kw)), None, None) == status, kw
    assert L.mg_conv2d_output_hw(None, None, None) == INVALID


def test_conv_workspace_bytes(L):
    M = 2 * 16 * 16
    assert L.mg_conv2d_workspace_bytes(ctypes.byref(shape()), F16) == 0  # the GEMM gathers from the image
    assert L.mg_conv2d_workspace_bytes(ctypes.byref(shape(in_channels=128)), BF16) == 0
    assert L.mg_conv2d_workspace_bytes(ctypes.byref(shape(in_channels=16)), F16) == M * 144 * 2
    assert L.mg_conv2d_workspace_bytes(ctypes.byref(shape()), 2) == M * 576 * 4  # fp32: im2col + GEMM
    assert L.mg_conv2d_workspace_bytes(ctypes.byref(shape(in_channels=3)), F16) == M * 32 * 2  # 27 -> 32
    assert L.mg_conv2d_workspace_bytes(ctypes.byref(shape(in_channels=3)), 2) == M * 28 * 4  # 27 -> 28
    one = dict(kernel_h=1, kernel_w=1, pad_h=0, pad_w=0)
    assert L.mg_conv2d_workspace_bytes(ctypes.byref(shape(**one)), F16) == 0  # the input is the GEMM's A
    assert L.mg_conv2d_workspace_bytes(ctypes.byref(shape(in_channels=12, **one)), F16) == M * 16 * 2
    assert L.mg_conv2d_workspace_bytes(ctypes.byref(shape(stride_h=2, **one)), F16) == 0  # gathered
    assert L.mg_conv2d_workspace_bytes(ctypes.byref(shape(stride_h=2, in_channels=16, **one)), F16) == 2 * 8 * 16 * 16 * 2
    assert L.mg_conv2d_workspace_bytes(ctypes.byref(shape(kernel_h=0)), F16) == 0
    assert L.mg_conv2d_workspace_bytes(ctypes.byref(shape()), 7) == 0


def im2col(L, s=None, x=P, cols=P, ld=576, dt=F16):
    return L.mg_im2col(ctypes.byref(s or shape()), x, cols, ld, dt, S)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=5), DTYPE), (dict(ld=568), LAYOUT), (dict(ld=580), MISALIGNED), (dict(ld=1 << 27), LAYOUT),
    (dict(x=None), INVALID), (dict(x=P + 8), MISALIGNED), (dict(cols=None), INVALID), (dict(cols=P + 2), MISALIGNED),
    (dict(s=shape(kernel_w=0)), INVALID), (dict(s=shape(batch=0), x=None, cols=None), OK),
    (dict(dt=2, ld=578), MISALIGNED),
])
def test_im2col_rejects_bad_arguments(L, kw, status):
    assert im2col(L, **kw) == status


def conv(L, s=None, x=P, w=P, swk=64, swn=1, bias=None, y=P, ws=P, ws_bytes=1 << 30, dt=F16):
    return L.mg_conv2d(ctypes.byref(s or shape()), x, w, swk, swn, bias, y, ws, ws_bytes, dt, S)


C16 = shape(in_channels=16)  # 16 channels: never gathered by the GEMM, so im2col needs a workspace


@pytest.mark.parametrize("kw,status", [
    (dict(dt=9), DTYPE), (dict(x=None), INVALID), (dict(x=P + 4), MISALIGNED), (dict(w=None), INVALID),
    (dict(y=None), INVALID), (dict(s=C16, ws=None), INVALID), (dict(s=C16, ws_bytes=2 * 256 * 144 * 2 - 1), INVALID),
    (dict(s=C16, ws=P + 8), MISALIGNED), (dict(swk=64, swn=2), LAYOUT), (dict(swk=70, swn=1), MISALIGNED),
    (dict(s=shape(out_channels=4), swk=4), MISALIGNED),  # NHWC rows of 4 fp16 are not 16-byte rows
    (dict(s=shape(in_channels=3), swk=1, swn=27), MISALIGNED),  # OHWI rows of 27 fp16
    (dict(dt=2, swk=1, swn=576), LAYOUT),  # fp32 takes HWIO weights only
    (dict(dt=2, s=shape(in_channels=3)), LAYOUT),  # fp32 K = 27 is not a multiple of 16
    (dict(s=shape(batch=0), x=None, w=None, y=None, ws=None), OK),
    (dict(s=shape(out_channels=0), w=None, y=None, ws=None), OK),
    (dict(s=shape(stride_h=0)), INVALID),
])
def test_conv_rejects_bad_arguments(L, kw, status):
    assert conv(L, **kw) == status


def test_conv_1x1_needs_no_workspace_but_validates_the_gemm(L):
    one = shape(kernel_h=1, kernel_w=1, pad_h=0, pad_w=0)
    # no workspace is needed, so a null one is fine; the GEMM's checks still apply
    assert conv(L, s=one, ws=None, ws_bytes=0, y=None) == INVALID
    assert conv(L, s=one, ws=None, ws_bytes=0, x=P + 8) == MISALIGNED


def attn(L, Q=P, K=P, Sx=P, heads=4, Lq=128, Lk=128, d=64, sqh=128 * 64, sqm=64, skh=128 * 64, skn=64,
         ssh=128 * 128, ssm=128, dt=F16):
    return L.mg_attention_scores(Q, K, Sx, heads, Lq, Lk, d, sqh, sqm, skh, skn, ssh, ssm, dt, S)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=2), DTYPE), (dict(dt=4), DTYPE), (dict(heads=-1), INVALID), (dict(Q=None), INVALID),
    (dict(K=None), INVALID), (dict(Sx=None), INVALID),
    (dict(sqm=72, sqh=128 * 72 + 4), MISALIGNED), (dict(skn=66), MISALIGNED),
    (dict(ssh=100 * 128), LAYOUT),  # score entries of different heads would overlap
    (dict(heads=0, Q=None, K=None, Sx=None), OK), (dict(Lq=0), OK),
])
def test_attention_scores_rejects_bad_arguments(L, kw, status):
    assert attn(L, **kw) == status


def test_conv_workspace_follows_a_forced_row(L):
    # the general-only row cannot gather: the convolution then needs the im2col workspace
    assert L.mg_set_config(5) == OK
    try:
        assert L.mg_conv2d_workspace_bytes(ctypes.byref(shape()), F16) == 2 * 256 * 576 * 2
        assert conv(L, ws=None) == INVALID
    finally:
        L.mg_set_config(-1)
    assert L.mg_conv2d_workspace_bytes(ctypes.byref(shape()), F16) == 0


def test_binding_refuses_host_tensors_before_any_call():
    """Host tensors never reach the library: the binding raises first."""
    import torch

    a, b = torch.zeros(8, 8, dtype=torch.float16), torch.zeros(8, 8, dtype=torch.float16)
    for fn in (lambda: mg.mg_gemm(a, b), lambda: mg.mg_gemm_bias_relu(a, b, torch.zeros(8, dtype=torch.float16)),
               lambda: mg.mg_gemm_splitk(a, b, splits=2), lambda: mg.mg_gemm_batched(a[None], b[None]),
               lambda: mg.mg_attention_scores(a[None], b[None])):
        with pytest.raises(RuntimeError, match="GPU tensors only"):
            fn()


def test_transposed_operands_refused_only_without_a_direct_kernel(L):
    """Row 5 has only the general kernel: forced, it refuses a transposed
    operand before any HIP call (any shape is taken by the table's rows)."""
    try:
        assert L.mg_set_config(5) == OK
        assert gemm(L, sam=1, sak=64, M=60) == LAYOUT
        assert gemm(L, sbk=1, sbn=64, K=40, sam=40) == LAYOUT
    finally:
        L.mg_set_config(-1)
