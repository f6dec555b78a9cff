"""CPU oracle for the tiled GEMM path -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library: the arithmetic
lives in ``gemm_oracle.c`` (plain C, built with gcc), the index bookkeeping
(prepack layout, tile rasterisation, LDS budget) in ``layout.py`` and the
comparisons in ``compare.py``.

Definition followed (see ``gemm_oracle.c`` for the citations):
C[i,j] = sum_k a(i,k) b(k,j) over the exact input values in fp64, k ascending,
then optional + bias[j] and ReLU, kept unrounded (``ref``) and rounded once
round-to-nearest-even to the output type (``ref_q``).

GEMM consumers (FlagOS cross-chip page, section 5.3): a 2-D convolution by
its definition (NHWC input, [KH,KW,C,OC] weights, zero padding, stride,
dilation), and attention scores Q K^T per head on the GEMM oracle.  im2col,
pure data movement, sits in ``layout.py``.

Parity pins: every public function here is pinned by ``tests/test_oracle_*``
against values fixed by the pages or by mathematics (brute force, closed
forms, identities, exhaustive rounding checks).  Performance has no pin.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

F16 = 0
BF16 = 1
F32 = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "liborc.so")
_lock = threading.Lock()
_lib = None

_CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-pthread", "-std=c11"]


def build(force: bool = True, src: str | None = None, out: str | None = None) -> str:
    """Compile the C oracle with gcc into oracle/_build/liborc.so (or `src` into `out`)."""
    os.makedirs(_BUILD_DIR, exist_ok=True)
    target = out or _LIB_PATH
    if force or not os.path.exists(target):
        tmp = target + ".tmp%d" % os.getpid()
        cmd = ["gcc", *_CFLAGS, "-o", tmp, src or _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, target)
    return target


def _configure(lib):
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    i32p = ctypes.POINTER(ctypes.c_int32)
    i64 = ctypes.c_int64
    cint = ctypes.c_int
    lib.orc_decode.restype = ctypes.c_double
    lib.orc_decode.argtypes = [ctypes.c_uint16, cint]
    lib.orc_encode.restype = ctypes.c_uint16
    lib.orc_encode.argtypes = [ctypes.c_double, cint]
    lib.orc_decode_array.restype = None
    lib.orc_decode_array.argtypes = [u16p, f64p, i64, cint]
    lib.orc_encode_array.restype = None
    lib.orc_encode_array.argtypes = [f64p, u16p, i64, cint]
    lib.orc_gemm.restype = cint
    lib.orc_gemm.argtypes = [u16p, u16p, u16p, i64, i64, i64, i64, i64, cint, cint, f64p, u16p, cint]
    lib.orc_gemm_sampled.restype = cint
    lib.orc_gemm_sampled.argtypes = [u16p, u16p, u16p, i64, i64, i64, cint, cint, i64p, i64p, i64,
                                     f64p, u16p, cint]
    lib.orc_grouped_gemm.restype = cint
    lib.orc_grouped_gemm.argtypes = [u16p, u16p, i32p, i64, i64, i64, i64, i64, i64, cint, f64p, u16p, cint]
    u32p = ctypes.POINTER(ctypes.c_uint32)
    lib.orc_decode32.restype = ctypes.c_double
    lib.orc_decode32.argtypes = [ctypes.c_uint32]
    lib.orc_encode32.restype = ctypes.c_uint32
    lib.orc_encode32.argtypes = [ctypes.c_double]
    lib.orc_decode32_array.restype = None
    lib.orc_decode32_array.argtypes = [u32p, f64p, i64]
    lib.orc_encode32_array.restype = None
    lib.orc_encode32_array.argtypes = [f64p, u32p, i64]
    lib.orc_gemm_d.restype = cint
    lib.orc_gemm_d.argtypes = [f64p, f64p, i64, i64, i64, f64p]
    lib.orc_gemm_d_sampled.restype = cint
    lib.orc_gemm_d_sampled.argtypes = [f64p, f64p, i64, i64, i64p, i64p, i64, f64p]
    lib.orc_grouped_sampled.restype = cint
    lib.orc_conv2d_d.restype = cint
    lib.orc_conv2d_d.argtypes = [f64p, f64p] + [i64] * 13 + [i64p, i64p, i64, f64p]
    lib.orc_grouped_sampled.argtypes = [u16p, u16p, i32p, i64, i64, i64, i64, i64, cint, i64p, i64p, i64,
                                        f64p, u16p]
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _configure(ctypes.CDLL(_LIB_PATH))
        return _lib


_active = None  # a library bound by use_library(); None means the built oracle


def use_library(path: str | None):
    """Bind the functions of this module to another build of gemm_oracle.c
    (the tests use this to show that deliberately broken copies fail the
    pins); None restores the real oracle."""
    global _active
    _active = None if path is None else _configure(ctypes.CDLL(path))


def _L():
    return _active if _active is not None else _load()


def _ptr(a: np.ndarray | None, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _bits(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle inputs are raw fp16/bf16 bit patterns (uint16), got %s" % a.dtype)
    return a


MAX_THREADS = 16  # a GPU host's CPU share per GPU; more cores than this are not ours to use


def default_threads() -> int:
    """Threads for the full-output oracle: the cores this process may run on,
    at most MAX_THREADS."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(MAX_THREADS, n))


def decode(bits, dtype: int) -> np.ndarray:
    """Exact value (fp64) of fp16 / bf16 bit patterns."""
    b = _bits(np.asarray(bits, dtype=np.uint16))
    out = np.empty(b.shape, dtype=np.float64)
    _L().orc_decode_array(_ptr(b, ctypes.c_uint16), _ptr(out, ctypes.c_double), b.size, dtype)
    return out


def encode(x, dtype: int) -> np.ndarray:
    """Round fp64 values once, to nearest even, to fp16 / bf16 bit patterns."""
    v = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(v.shape, dtype=np.uint16)
    _L().orc_encode_array(_ptr(v, ctypes.c_double), _ptr(out, ctypes.c_uint16), v.size, dtype)
    return out


def gemm(A, B, dtype: int, bias=None, relu: bool = False, nthreads: int | None = None):
    """Full dense oracle.  A: [M,K] bits, B: [K,N] bits, bias: [N] bits or None.

    Returns (ref fp64 [M,N], ref_q uint16 [M,N])."""
    A = _bits(A)
    B = _bits(B)
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
    bias_b = None if bias is None else _bits(bias)
    if bias_b is not None and bias_b.shape != (N,):
        raise ValueError("bias must have shape (N,)")
    ref = np.zeros((M, N), dtype=np.float64)
    ref_q = np.zeros((M, N), dtype=np.uint16)
    if M and N:
        rc = _L().orc_gemm(_ptr(A, ctypes.c_uint16), _ptr(B, ctypes.c_uint16), _ptr(bias_b, ctypes.c_uint16),
                              M, N, K, K, N, dtype, int(bool(relu)), _ptr(ref, ctypes.c_double),
                              _ptr(ref_q, ctypes.c_uint16), nthreads or default_threads())
        if rc != 0:
            raise MemoryError("oracle gemm failed")
    return ref, ref_q


def gemm_sampled(A, B, dtype: int, rows, cols, bias=None, relu: bool = False, nthreads: int | None = None):
    """Dense oracle at the given (row, col) positions only."""
    A = _bits(A)
    B = _bits(B)
    M, K = A.shape
    _, N = B.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols differ in length")
    if rows.size and (rows.min() < 0 or rows.max() >= M or cols.min() < 0 or cols.max() >= N):
        raise IndexError("sample position outside the output")
    bias_b = None if bias is None else _bits(bias)
    ref = np.zeros(rows.shape, dtype=np.float64)
    ref_q = np.zeros(rows.shape, dtype=np.uint16)
    _L().orc_gemm_sampled(_ptr(A, ctypes.c_uint16), _ptr(B, ctypes.c_uint16), _ptr(bias_b, ctypes.c_uint16),
                             K, K, N, dtype, int(bool(relu)), _ptr(rows, ctypes.c_int64),
                             _ptr(cols, ctypes.c_int64), rows.size, _ptr(ref, ctypes.c_double),
                             _ptr(ref_q, ctypes.c_uint16), nthreads or default_threads())
    return ref, ref_q


def _check_offsets(offsets, T):
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    if off[0] != 0 or off[-1] != T or np.any(np.diff(off) < 0):
        raise ValueError("offsets must start at 0, end at T and be nondecreasing")
    return off


def grouped_gemm(X, W, offsets, dtype: int, nthreads: int | None = None):
    """Full grouped oracle.  X: [T,K] bits, W: [E,K,N] bits, offsets: [E+1]."""
    X = _bits(X)
    W = _bits(W)
    T, K = X.shape
    E, K2, N = W.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    off = _check_offsets(offsets, T)
    if off.shape != (E + 1,):
        raise ValueError("offsets must have E+1 entries")
    ref = np.zeros((T, N), dtype=np.float64)
    ref_q = np.zeros((T, N), dtype=np.uint16)
    _L().orc_grouped_gemm(_ptr(X, ctypes.c_uint16), _ptr(W, ctypes.c_uint16), _ptr(off, ctypes.c_int32),
                             E, N, K, K, K * N, N, dtype, _ptr(ref, ctypes.c_double),
                             _ptr(ref_q, ctypes.c_uint16), nthreads or default_threads())
    return ref, ref_q


def grouped_sampled(X, W, offsets, dtype: int, rows, cols):
    X = _bits(X)
    W = _bits(W)
    T, K = X.shape
    E, _, N = W.shape
    off = _check_offsets(offsets, T)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= T or cols.min() < 0 or cols.max() >= N):
        raise IndexError("sample position outside the output")
    ref = np.zeros(rows.shape, dtype=np.float64)
    ref_q = np.zeros(rows.shape, dtype=np.uint16)
    rc = _L().orc_grouped_sampled(_ptr(X, ctypes.c_uint16), _ptr(W, ctypes.c_uint16), _ptr(off, ctypes.c_int32),
                                     E, K, K, K * N, N, dtype, _ptr(rows, ctypes.c_int64),
                                     _ptr(cols, ctypes.c_int64), rows.size, _ptr(ref, ctypes.c_double),
                                     _ptr(ref_q, ctypes.c_uint16))
    if rc != 0:
        raise ValueError("a sampled row lies in no expert")
    return ref, ref_q


# ---- fp32 -------------------------------------------------------------------
def decode32(bits) -> np.ndarray:
    """Exact values (fp64) of fp32 bit patterns, from the IEEE field definitions."""
    b = np.ascontiguousarray(bits, dtype=np.uint32)
    out = np.empty(b.shape, dtype=np.float64)
    _L().orc_decode32_array(_ptr(b, ctypes.c_uint32), _ptr(out, ctypes.c_double), b.size)
    return out


def encode32(x) -> np.ndarray:
    """fp64 values rounded once to fp32 (ties to even), as bit patterns."""
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint32)
    _L().orc_encode32_array(_ptr(a, ctypes.c_double), _ptr(out, ctypes.c_uint32), a.size)
    return out


def gemm_f32(A, B):
    """fp32 GEMM oracle: A [M,K], B [K,N] fp32 bit patterns (uint32).  Returns
    (ref, ref_q): the k-ascending fp64 sum of the exact products and its
    single RNE rounding to fp32 (bit patterns)."""
    Ad, Bd = decode32(A), decode32(B)
    M, K = Ad.shape
    _, N = Bd.shape
    ref = np.empty((M, N), dtype=np.float64)
    if M and N:
        _L().orc_gemm_d(_ptr(np.ascontiguousarray(Ad), ctypes.c_double), _ptr(np.ascontiguousarray(Bd), ctypes.c_double),
                        M, N, K, _ptr(ref, ctypes.c_double))
    return ref, encode32(ref)


def gemm_f32_sampled(A, B, rows, cols):
    Ad, Bd = np.ascontiguousarray(decode32(A)), np.ascontiguousarray(decode32(B))
    M, K = Ad.shape
    _, N = Bd.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= M or cols.min() < 0 or cols.max() >= N):
        raise IndexError("sample position outside the output")
    ref = np.empty(rows.shape, dtype=np.float64)
    _L().orc_gemm_d_sampled(_ptr(Ad, ctypes.c_double), _ptr(Bd, ctypes.c_double), N, K, _ptr(rows, ctypes.c_int64),
                            _ptr(cols, ctypes.c_int64), rows.size, _ptr(ref, ctypes.c_double))
    return ref, encode32(ref)


# ---- GEMM consumers: 2-D convolution and attention scores -------------------
def _decode_any(bits, dtype: int) -> np.ndarray:
    return decode32(bits) if dtype == F32 else decode(bits, dtype)


def _encode_any(x, dtype: int) -> np.ndarray:
    return encode32(x) if dtype == F32 else encode(x, dtype)


def conv_out_hw(H, W, KH, KW, stride=(1, 1), pad=(0, 0), dil=(1, 1)):
    """Output height and width of a convolution: floor((H + 2p - d (KH - 1) - 1) / s) + 1."""
    oh = (H + 2 * pad[0] - dil[0] * (KH - 1) - 1) // stride[0] + 1
    ow = (W + 2 * pad[1] - dil[1] * (KW - 1) - 1) // stride[1] + 1
    return oh, ow


def conv2d(x, w, dtype: int, stride=(1, 1), pad=(0, 0), dil=(1, 1), bias=None, relu: bool = False,
           rows=None, cols=None):
    """2-D convolution oracle (cross-correlation with zero padding, the
    definition in gemm_oracle.c).  x: NHWC [Nb,H,W,C] bit patterns, w: [KH,KW,C,OC]
    bit patterns, dtype F16 / BF16 / F32.  Returns (ref, ref_q) of shape
    [Nb,OH,OW,OC], or, with `rows` (output row m = (n OH + oh) OW + ow) and
    `cols` (output channel), at those positions only.  Optional + bias[o], then
    ReLU (to +0.0), before the single rounding."""
    Nb, H, W, C = x.shape
    KH, KW, C2, OC = w.shape
    if C2 != C:
        raise ValueError("channel mismatch")
    xd = np.ascontiguousarray(_decode_any(x, dtype))
    wd = np.ascontiguousarray(_decode_any(w, dtype))
    OH, OW = conv_out_hw(H, W, KH, KW, stride, pad, dil)
    if OH < 1 or OW < 1:
        raise ValueError("empty output")
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        if rows.size and (rows.min() < 0 or rows.max() >= Nb * OH * OW or cols.min() < 0 or cols.max() >= OC):
            raise IndexError("sample position outside the output")
        ref = np.empty(rows.shape, dtype=np.float64)
        rp, cp, count = _ptr(rows, ctypes.c_int64), _ptr(cols, ctypes.c_int64), rows.size
        oc_of = cols
    else:
        ref = np.empty((Nb, OH, OW, OC), dtype=np.float64)
        rp = cp = None
        count = 0
        oc_of = None
    rc = _L().orc_conv2d_d(_ptr(xd, ctypes.c_double), _ptr(wd, ctypes.c_double), Nb, H, W, C, OC, KH, KW,
                           stride[0], stride[1], pad[0], pad[1], dil[0], dil[1], rp, cp, count,
                           _ptr(ref, ctypes.c_double))
    if rc != 0:
        raise ValueError("bad convolution parameters (code %d)" % rc)
    if bias is not None:
        bd = _decode_any(bias, dtype)
        ref = ref + (bd[oc_of] if oc_of is not None else bd)
    if relu:
        ref = np.where(ref > 0.0, ref, 0.0)
    return ref, _encode_any(ref, dtype)


def attention_scores(Q, K, dtype: int):
    """Attention scores S[h] = Q[h] K[h]^T for every head h (the QK^T product of
    the FlagOS page, section 5.3), on the GEMM oracle with B = K[h]^T.
    Q [BH,Lq,d], K [BH,Lk,d] 16-bit bit patterns.  Returns (ref, ref_q) [BH,Lq,Lk]."""
    BH, Lq, d = Q.shape
    _, Lk, _ = K.shape
    ref = np.empty((BH, Lq, Lk), dtype=np.float64)
    ref_q = np.empty((BH, Lq, Lk), dtype=np.uint16)
    for h in range(BH):
        ref[h], ref_q[h] = gemm(np.ascontiguousarray(Q[h]), np.ascontiguousarray(K[h].T), dtype)
    return ref, ref_q


def attention_scores_sampled(Q, K, dtype: int, heads, rows, cols):
    """S[h,i,j] = sum_{t ascending} q(h,i,t) k(h,j,t) in fp64 at the listed positions."""
    heads, rows, cols = (np.asarray(v, dtype=np.int64) for v in (heads, rows, cols))
    q = decode(np.ascontiguousarray(Q[heads, rows]), dtype)
    k = decode(np.ascontiguousarray(K[heads, cols]), dtype)
    ref = np.zeros(heads.shape, dtype=np.float64)
    for t in range(q.shape[1]):
        ref += q[:, t] * k[:, t]
    return ref, encode(ref, dtype)
