"""Python binding of libmi355gemm.so (tiled GEMM for one MI355X).

Argument marshalling only: each function takes torch tensors that already
live in GPU memory, passes their pointers, sizes, strides, dtype and torch's
current HIP stream to the C ABI declared in include/mi355gemm.h, and raises
RuntimeError with the library's message on a non-OK status.  All arithmetic
happens in the library's HIP kernels; there is no fallback.  torch is used
for device memory and streams only.

The library is built in-tree (``python -m tiled_matrix_multiplication_gemm_amd.build``)
and loaded on first use; using any entry point without it raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmi355gemm.so")

MG_F16 = 0
MG_BF16 = 1
MG_F32 = 2

_lock = threading.Lock()
_lib = None


class ConfigDesc(ctypes.Structure):
    _fields_ = [
        ("id", ctypes.c_int), ("bm", ctypes.c_int), ("bn", ctypes.c_int), ("bk", ctypes.c_int),
        ("waves_m", ctypes.c_int), ("waves_n", ctypes.c_int), ("stages", ctypes.c_int),
        ("mfma_m", ctypes.c_int), ("mfma_n", ctypes.c_int), ("mfma_k", ctypes.c_int),
        ("group_m", ctypes.c_int), ("xcd_remap", ctypes.c_int), ("lds_bytes", ctypes.c_int),
        ("direct_lds", ctypes.c_int), ("direct_bk", ctypes.c_int), ("direct_stages", ctypes.c_int),
        ("direct_lds_bytes", ctypes.c_int), ("direct_ksplit", ctypes.c_int), ("name", ctypes.c_char_p),
    ]


EXPORTED = (
    "mg_status_string", "mg_gemm", "mg_gemm_bias_relu", "mg_gemm_batched", "mg_gemm_splitk",
    "mg_splitk_workspace_bytes", "mg_splitk_choose", "mg_grouped_gemm", "mg_prepacked_bytes",
    "mg_prepack_a", "mg_config_bk", "mg_gemm_prepacked", "mg_num_configs", "mg_config_info",
    "mg_set_config", "mg_last_config", "mg_select_config", "mg_conv2d_output_hw", "mg_im2col",
    "mg_conv2d_workspace_bytes", "mg_conv2d", "mg_attention_scores", "mg_splitk_noalloc_max_bytes",
    "mg_gemm_splitk_noalloc", "mg_last_kernel", "mg_prepack_uses_to_pay", "mg_set_raster",
)


class Conv2dShape(ctypes.Structure):
    """mg_conv2d_shape of the C ABI."""
    _fields_ = [(n, ctypes.c_int64) for n in (
        "batch", "height", "width", "in_channels", "out_channels", "kernel_h", "kernel_w", "stride_h", "stride_w",
        "pad_h", "pad_w", "dilation_h", "dilation_w")]


def lib() -> ctypes.CDLL:
    """The loaded C library with argument types declared (raises if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmi355gemm.so is not built; run `python -m tiled_matrix_multiplication_gemm_amd.build`")
        import torch  # noqa: F401  -- load torch's HIP runtime first so both share one runtime

        L = ctypes.CDLL(LIB_PATH)
        vp, i64, cint = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.mg_status_string.restype = ctypes.c_char_p
        L.mg_status_string.argtypes = [cint]
        L.mg_gemm.restype = cint
        L.mg_gemm.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, i64, cint, cint, vp]
        L.mg_gemm_bias_relu.restype = cint
        L.mg_gemm_bias_relu.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, i64, cint, cint, vp]
        L.mg_gemm_batched.restype = cint
        L.mg_gemm_batched.argtypes = [vp, vp, vp] + [i64] * 13 + [cint, cint, vp]
        L.mg_splitk_workspace_bytes.restype = ctypes.c_size_t
        L.mg_splitk_workspace_bytes.argtypes = [i64, i64, i64]
        L.mg_splitk_choose.restype = i64
        L.mg_splitk_choose.argtypes = [i64, i64, i64]
        L.mg_gemm_splitk.restype = cint
        L.mg_gemm_splitk.argtypes = [vp, vp, vp, vp, ctypes.c_size_t] + [i64] * 10 + [cint, cint, vp]
        L.mg_splitk_noalloc_max_bytes.restype = ctypes.c_size_t
        L.mg_splitk_noalloc_max_bytes.argtypes = []
        L.mg_gemm_splitk_noalloc.restype = cint
        L.mg_gemm_splitk_noalloc.argtypes = [vp, vp, vp] + [i64] * 10 + [cint, cint, vp]
        L.mg_grouped_gemm.restype = cint
        L.mg_grouped_gemm.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, cint, vp]
        L.mg_prepacked_bytes.restype = ctypes.c_size_t
        L.mg_prepacked_bytes.argtypes = [i64, i64, i64, cint]
        L.mg_prepack_a.restype = cint
        L.mg_prepack_a.argtypes = [vp, vp, i64, i64, i64, i64, cint, vp]
        L.mg_config_bk.restype = i64
        L.mg_config_bk.argtypes = [i64, i64, i64, cint]
        L.mg_gemm_prepacked.restype = cint
        L.mg_gemm_prepacked.argtypes = [vp, i64, vp, vp, i64, i64, i64, i64, i64, i64, i64, cint, vp]
        L.mg_num_configs.restype = cint
        L.mg_num_configs.argtypes = []
        L.mg_config_info.restype = cint
        L.mg_config_info.argtypes = [cint, ctypes.POINTER(ConfigDesc)]
        L.mg_set_config.restype = cint
        L.mg_set_config.argtypes = [cint]
        L.mg_last_config.restype = cint
        L.mg_last_config.argtypes = []
        L.mg_set_raster.restype = cint
        L.mg_set_raster.argtypes = [cint, cint]
        L.mg_prepack_uses_to_pay.restype = i64
        L.mg_prepack_uses_to_pay.argtypes = [i64, i64, i64, cint]
        L.mg_last_kernel.restype = cint
        L.mg_last_kernel.argtypes = []
        L.mg_select_config.restype = cint
        L.mg_select_config.argtypes = [i64, i64, i64, cint, cint, i64]
        shp = ctypes.POINTER(Conv2dShape)
        L.mg_conv2d_output_hw.restype = cint
        L.mg_conv2d_output_hw.argtypes = [shp, ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.mg_im2col.restype = cint
        L.mg_im2col.argtypes = [shp, vp, vp, i64, cint, vp]
        L.mg_conv2d_workspace_bytes.restype = ctypes.c_size_t
        L.mg_conv2d_workspace_bytes.argtypes = [shp, cint]
        L.mg_conv2d.restype = cint
        L.mg_conv2d.argtypes = [shp, vp, vp, i64, i64, vp, vp, vp, ctypes.c_size_t, cint, vp]
        L.mg_attention_scores.restype = cint
        L.mg_attention_scores.argtypes = [vp, vp, vp] + [i64] * 10 + [cint, vp]
        _lib = L
        return L


def _check(status: int) -> None:
    if status != 0:
        raise RuntimeError(lib().mg_status_string(status).decode())


# Per-call helpers.  They run before every launch, so torch objects they
# need are looked up once (dtype codes, the raw-stream accessor) and devices
# are compared as integers.
_DTYPE_CODES = None
_RAW_STREAM = None


def _dtype_code(t) -> int:
    global _DTYPE_CODES
    if _DTYPE_CODES is None:
        import torch

        _DTYPE_CODES = {torch.float16: MG_F16, torch.bfloat16: MG_BF16, torch.float32: MG_F32}
    code = _DTYPE_CODES.get(t.dtype)
    if code is None:
        raise RuntimeError("MG_ERR_UNSUPPORTED_DTYPE: tensor dtype %s is not float16/bfloat16/float32" % t.dtype)
    return code


def _stream(t):
    """torch's current HIP stream on t's device, as a raw handle."""
    global _RAW_STREAM
    if _RAW_STREAM is None:
        import torch

        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        _RAW_STREAM = raw if raw is not None else (lambda d: torch.cuda.current_stream(d).cuda_stream)
    return _RAW_STREAM(t.get_device())


def _require_gpu(*ts):
    """Every tensor on the GPU, all on the first one's device."""
    dev = None
    for t in ts:
        if not t.is_cuda:
            raise RuntimeError("mi355gemm operates on GPU tensors only (got a %s tensor)" % t.device)
        d = t.get_device()
        if dev is None:
            dev = d
        elif d != dev:
            raise RuntimeError("MG_ERR_INVALID_ARG: tensors on different devices (%s, %s)" % (ts[0].device, t.device))


def _same_dtype(ref, *ts):
    for t in ts:
        if t.dtype != ref.dtype:
            raise RuntimeError("MG_ERR_UNSUPPORTED_DTYPE: operands must share one dtype (%s, %s)" % (ref.dtype, t.dtype))


def _check_out(out, shape, like):
    """A caller-supplied output: the exact shape, like's dtype and device,
    and a unit inner stride (the C ABI sees only a pointer and row strides,
    so a smaller or differently typed buffer would be overrun or misread)."""
    _require_gpu(like, out)
    if out.shape != shape:
        raise RuntimeError("MG_ERR_INVALID_ARG: out has shape %s, expected %s" % (tuple(out.shape), tuple(shape)))
    if out.dtype != like.dtype:
        raise RuntimeError("MG_ERR_UNSUPPORTED_DTYPE: out is %s, expected %s" % (out.dtype, like.dtype))
    if shape[-1] > 1 and out.stride(-1) != 1:
        raise RuntimeError("MG_ERR_UNSUPPORTED_LAYOUT: out needs a unit inner stride")


def mg_gemm(a, b, out=None):
    """out[M,N] = a[M,K] @ b[K,N] (fp16/bf16, fp32 accumulation)."""
    _require_gpu(a, b)
    M, K = a.shape
    K2, N = b.shape
    if K2 != K:
        raise RuntimeError("MG_ERR_INVALID_ARG: inner dimensions differ (%d vs %d)" % (K, K2))
    _same_dtype(a, b)
    if out is None:
        import torch

        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    _check_out(out, (M, N), a)
    sa, sb, so = a.stride(), b.stride(), out.stride()
    code = _dtype_code(a)
    _check(lib().mg_gemm(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, sa[0], sa[1], sb[0], sb[1],
                         so[0], so[1], code, code, _stream(a)))
    return out


def mg_gemm_bias_relu(a, b, bias, out=None):
    """out = ReLU(a @ b + bias) in one kernel."""
    _require_gpu(a, b, bias)
    M, K = a.shape
    K2, N = b.shape
    if K2 != K or bias.shape != (N,) or (N > 1 and bias.stride(0) != 1):
        raise RuntimeError("MG_ERR_INVALID_ARG: shapes a[M,K], b[K,N], contiguous bias[N] expected")
    _same_dtype(a, b, bias)
    if out is None:
        import torch

        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    _check_out(out, (M, N), a)
    sa, sb, so = a.stride(), b.stride(), out.stride()
    code = _dtype_code(a)
    _check(lib().mg_gemm_bias_relu(a.data_ptr(), b.data_ptr(), bias.data_ptr(), out.data_ptr(), M, N, K,
                                   sa[0], sa[1], sb[0], sb[1], so[0], so[1], code, code, _stream(a)))
    return out


def mg_gemm_batched(a, b, out=None):
    """out[i] = a[i] @ b[i] for every batch entry i, in one launch.

    a: [batch, M, K], b: [batch, K, N] (either may be an expanded view with
    batch stride 0; each entry row-major or transposed as for mg_gemm)."""
    import torch

    _require_gpu(a, b)
    if a.dim() != 3 or b.dim() != 3 or a.shape[0] != b.shape[0] or a.shape[2] != b.shape[1]:
        raise RuntimeError("MG_ERR_INVALID_ARG: a[batch,M,K] and b[batch,K,N] expected")
    batch, M, K = a.shape
    N = b.shape[2]
    _same_dtype(a, b)
    if out is None:
        out = torch.empty((batch, M, N), dtype=a.dtype, device=a.device)
    _check_out(out, (batch, M, N), a)
    _check(lib().mg_gemm_batched(a.data_ptr(), b.data_ptr(), out.data_ptr(), batch, M, N, K, a.stride(1),
                                 a.stride(2), b.stride(1), b.stride(2), out.stride(1), out.stride(2), a.stride(0),
                                 b.stride(0), out.stride(0), _dtype_code(a), _dtype_code(out), _stream(a)))
    return out


def mg_splitk_workspace_bytes(M: int, N: int, splits: int) -> int:
    return int(lib().mg_splitk_workspace_bytes(M, N, splits))


def mg_splitk_choose(M: int, N: int, K: int) -> int:
    return int(lib().mg_splitk_choose(M, N, K))


def mg_gemm_splitk(a, b, splits: int | None = None, workspace=None, out=None):
    """out = a @ b with K cut into `splits` runs (fp32 partials in `workspace`,
    a device tensor of at least mg_splitk_workspace_bytes(M, N, splits)
    bytes; allocated here through torch when not given).  splits=None takes
    mg_splitk_choose()."""
    import torch

    _require_gpu(a, b)
    M, K = a.shape
    K2, N = b.shape
    if K2 != K:
        raise RuntimeError("MG_ERR_INVALID_ARG: inner dimensions differ (%d vs %d)" % (K, K2))
    _same_dtype(a, b)
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    _check_out(out, (M, N), a)
    if splits is None:
        splits = mg_splitk_choose(M, N, K)
    need = mg_splitk_workspace_bytes(M, N, splits)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=a.device)
    _require_gpu(a, workspace)
    if not workspace.is_contiguous():
        raise RuntimeError("MG_ERR_INVALID_ARG: the workspace must be contiguous")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().mg_gemm_splitk(a.data_ptr(), b.data_ptr(), out.data_ptr(), workspace.data_ptr(), ws_bytes, splits,
                                M, N, K, a.stride(0), a.stride(1), b.stride(0), b.stride(1), out.stride(0),
                                out.stride(1), _dtype_code(a), _dtype_code(out), _stream(a)))
    return out


def mg_splitk_noalloc_max_bytes() -> int:
    return int(lib().mg_splitk_noalloc_max_bytes())


def mg_gemm_splitk_noalloc(a, b, splits: int | None = None, out=None):
    """out = a @ b by split-K with the partials in the library's own scratch
    array (no workspace, nothing allocated by the library; `out` must be
    given by callers that cannot allocate)."""
    import torch

    _require_gpu(a, b)
    M, K = a.shape
    K2, N = b.shape
    if K2 != K:
        raise RuntimeError("MG_ERR_INVALID_ARG: inner dimensions differ (%d vs %d)" % (K, K2))
    _same_dtype(a, b)
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    _check_out(out, (M, N), a)
    if splits is None:
        splits = mg_splitk_choose(M, N, K)
    _check(lib().mg_gemm_splitk_noalloc(a.data_ptr(), b.data_ptr(), out.data_ptr(), splits, M, N, K, a.stride(0),
                                        a.stride(1), b.stride(0), b.stride(1), out.stride(0), out.stride(1),
                                        _dtype_code(a), _dtype_code(out), _stream(a)))
    return out


def mg_grouped_gemm(x, w, offsets, out=None):
    """out[o_e:o_{e+1}] = x[o_e:o_{e+1}] @ w[e] for every expert e (one launch).

    x: [T,K], w: [E,K,N], offsets: int32 device tensor [E+1] (0, ..., T)."""
    import torch

    _require_gpu(x, w, offsets)
    T, K = x.shape
    E, K2, N = w.shape
    if K2 != K or offsets.shape != (E + 1,) or offsets.dtype != torch.int32 or not offsets.is_contiguous():
        raise RuntimeError("MG_ERR_INVALID_ARG: x[T,K], w[E,K,N], contiguous int32 offsets[E+1] expected")
    if w.stride(2) != 1 and N > 1:
        raise RuntimeError("MG_ERR_UNSUPPORTED_LAYOUT: w must have a unit inner stride")
    if w.dtype != x.dtype:
        raise RuntimeError("MG_ERR_UNSUPPORTED_DTYPE: x and w must share a dtype")
    if out is None:
        out = torch.empty((T, N), dtype=x.dtype, device=x.device)
    _check_out(out, (T, N), x)
    if x.stride(1) != 1 and K > 1 or out.stride(1) != 1 and N > 1:
        raise RuntimeError("MG_ERR_UNSUPPORTED_LAYOUT: unit inner strides required")
    _check(lib().mg_grouped_gemm(x.data_ptr(), w.data_ptr(), out.data_ptr(), offsets.data_ptr(), E, T, N, K,
                                 x.stride(0), w.stride(0), w.stride(1), out.stride(0), _dtype_code(x), _stream(x)))
    return out


def mg_prepacked_bytes(M: int, K: int, BK: int, dtype: int = MG_F16) -> int:
    return int(lib().mg_prepacked_bytes(M, K, BK, dtype))


def mg_config_bk(M: int, N: int, K: int, dtype: int = MG_F16) -> int:
    return int(lib().mg_config_bk(M, N, K, dtype))


def mg_prepack_a(a, BK: int, out=None):
    """Blocked copy of a[M,K] as [ceil(K/BK), M, BK] (zero-padded K tail)."""
    import torch

    _require_gpu(a)
    M, K = a.shape
    if out is None:
        out = torch.empty(((K + BK - 1) // BK, M, BK), dtype=a.dtype, device=a.device)
    _check_out(out, ((K + BK - 1) // BK, M, BK), a)
    if not out.is_contiguous():
        raise RuntimeError("MG_ERR_UNSUPPORTED_LAYOUT: the packed output must be contiguous")
    if a.stride(1) != 1 and K > 1:
        raise RuntimeError("MG_ERR_UNSUPPORTED_LAYOUT: unit inner stride required")
    _check(lib().mg_prepack_a(a.data_ptr(), out.data_ptr(), M, K, a.stride(0), BK, _dtype_code(a), _stream(a)))
    return out


def mg_gemm_prepacked(ap, BK: int, b, M: int, K: int, out=None):
    """out[M,N] = A @ b with A given in the blocked layout of mg_prepack_a."""
    import torch

    _require_gpu(ap, b)
    K2, N = b.shape
    if K2 != K:
        raise RuntimeError("MG_ERR_INVALID_ARG: inner dimensions differ")
    _same_dtype(b, ap)
    if not ap.is_contiguous() or ap.numel() < (K + BK - 1) // BK * M * BK:
        raise RuntimeError("MG_ERR_INVALID_ARG: ap must be a contiguous packed [ceil(K/BK), M, BK] tensor")
    if out is None:
        out = torch.empty((M, N), dtype=b.dtype, device=b.device)
    _check_out(out, (M, N), b)
    _check(lib().mg_gemm_prepacked(ap.data_ptr(), BK, b.data_ptr(), out.data_ptr(), M, N, K, b.stride(0),
                                   b.stride(1), out.stride(0), out.stride(1), _dtype_code(b), _stream(b)))
    return out


def mg_prepack_uses_to_pay(M: int, N: int, K: int, dtype: int = MG_F16) -> int:
    """GEMMs sharing one blocked A after which prepacking pays (-1: never)."""
    return int(lib().mg_prepack_uses_to_pay(M, N, K, dtype))


def mg_select_config(M: int, N: int, K: int, dtype: int = MG_F16, grouped: int = 0, batch: int = 1) -> int:
    """The table's row for a dense problem, or a grouped one of `grouped` experts."""
    return int(lib().mg_select_config(M, N, K, dtype, int(grouped), int(batch)))


def mg_num_configs() -> int:
    return int(lib().mg_num_configs())


def mg_config_info(cid: int) -> dict:
    d = ConfigDesc()
    _check(lib().mg_config_info(cid, ctypes.byref(d)))
    out = {f: getattr(d, f) for f, _ in ConfigDesc._fields_}
    out["name"] = out["name"].decode()
    return out


def mg_set_config(cid: int) -> None:
    _check(lib().mg_set_config(cid))


def mg_set_raster(group_m: int = -1, xcd_remap: int = -1) -> None:
    """Process-wide GROUP_M / XCD-renumbering override (-1: the table's)."""
    _check(lib().mg_set_raster(group_m, xcd_remap))


def mg_last_config() -> int:
    return int(lib().mg_last_config())


KERNEL_FAMILIES = {-1: None, 0: "gemm_tile_kernel", 1: "gemm_dlds_kernel", 2: "gemm_kslab_kernel"}


def mg_last_kernel() -> str | None:
    """Kernel family of the last 16-bit GEMM launch in this process."""
    return KERNEL_FAMILIES[int(lib().mg_last_kernel())]




# ---- GEMM consumers --------------------------------------------------------
def _pair(v):
    return (int(v), int(v)) if isinstance(v, int) else (int(v[0]), int(v[1]))


def conv2d_shape(x_shape, kernel, out_channels: int, stride=1, pad=0, dil=1) -> Conv2dShape:
    """The C ABI's convolution shape for an NHWC input of shape x_shape."""
    Nb, H, W, C = (int(v) for v in x_shape)
    (kh, kw), (sh, sw), (ph, pw), (dh, dw) = _pair(kernel), _pair(stride), _pair(pad), _pair(dil)
    return Conv2dShape(Nb, H, W, C, int(out_channels), kh, kw, sh, sw, ph, pw, dh, dw)


def mg_conv2d_output_hw(shape: Conv2dShape):
    oh, ow = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(lib().mg_conv2d_output_hw(ctypes.byref(shape), ctypes.byref(oh), ctypes.byref(ow)))
    return oh.value, ow.value


def mg_conv2d_workspace_bytes(shape: Conv2dShape, dtype: int = MG_F16) -> int:
    return int(lib().mg_conv2d_workspace_bytes(ctypes.byref(shape), dtype))


def mg_im2col(x, kernel, stride=1, pad=0, dil=1, ld: int | None = None, out=None):
    """cols[Nb*OH*OW, ld] of an NHWC tensor x (zero where a tap falls outside
    the image; columns past KH*KW*C zero).  ld defaults to KH*KW*C rounded up
    to whole 16-byte chunks."""
    import torch

    _require_gpu(x)
    if x.dim() != 4 or not x.is_contiguous():
        raise RuntimeError("MG_ERR_UNSUPPORTED_LAYOUT: a contiguous NHWC tensor expected")
    shape = conv2d_shape(x.shape, kernel, 0, stride, pad, dil)
    oh, ow = mg_conv2d_output_hw(shape)
    K = shape.kernel_h * shape.kernel_w * shape.in_channels
    v = 16 // x.element_size()
    if ld is None:
        ld = (K + v - 1) // v * v
    M = shape.batch * oh * ow
    if out is None:
        out = torch.empty((M, ld), dtype=x.dtype, device=x.device)
    _check_out(out, (M, ld), x)
    if out.shape != (M, ld) or not out.is_contiguous():
        raise RuntimeError("MG_ERR_INVALID_ARG: out must be a contiguous [%d, %d] tensor" % (M, ld))
    _check(lib().mg_im2col(ctypes.byref(shape), x.data_ptr(), out.data_ptr(), ld, _dtype_code(x), _stream(x)))
    return out


def mg_conv2d(x, w, stride=1, pad=0, dil=1, bias=None, weight_layout: str = "hwio", workspace=None, out=None):
    """y = conv2d(x, w) as im2col + GEMM (then ReLU(y + bias) when bias is given).

    x: contiguous NHWC [Nb,H,W,C]; w: contiguous [KH,KW,C,OC] ("hwio") or
    [OC,KH,KW,C] ("ohwi"); returns NHWC [Nb,OH,OW,OC].  workspace: a device
    tensor of at least mg_conv2d_workspace_bytes() bytes, allocated here
    through torch when not given."""
    import torch

    _require_gpu(x, w)
    if x.dim() != 4 or w.dim() != 4 or not x.is_contiguous() or not w.is_contiguous():
        raise RuntimeError("MG_ERR_UNSUPPORTED_LAYOUT: contiguous NHWC x and 4-D weights expected")
    if weight_layout == "hwio":
        KH, KW, C, OC = w.shape
    elif weight_layout == "ohwi":
        OC, KH, KW, C = w.shape
    else:
        raise RuntimeError("MG_ERR_INVALID_ARG: weight_layout must be 'hwio' or 'ohwi'")
    if C != x.shape[3] or w.dtype != x.dtype:
        raise RuntimeError("MG_ERR_INVALID_ARG: channel count or dtype of w does not match x")
    shape = conv2d_shape(x.shape, (KH, KW), OC, stride, pad, dil)
    oh, ow = mg_conv2d_output_hw(shape)
    K = KH * KW * C
    swk, swn = (OC, 1) if weight_layout == "hwio" else (1, K)
    if bias is not None:
        _require_gpu(bias)
        if bias.shape != (OC,) or bias.dtype != x.dtype or (OC > 1 and bias.stride(0) != 1):
            raise RuntimeError("MG_ERR_INVALID_ARG: contiguous bias[OC] of x's dtype expected")
    if out is None:
        out = torch.empty((shape.batch, oh, ow, OC), dtype=x.dtype, device=x.device)
    _check_out(out, (shape.batch, oh, ow, OC), x)
    if tuple(out.shape) != (shape.batch, oh, ow, OC) or not out.is_contiguous():
        raise RuntimeError("MG_ERR_INVALID_ARG: out must be a contiguous [%d, %d, %d, %d] tensor"
                           % (shape.batch, oh, ow, OC))
    need = mg_conv2d_workspace_bytes(shape, _dtype_code(x))
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=x.device)
    if workspace is not None:
        _require_gpu(x, workspace)
        if not workspace.is_contiguous():
            raise RuntimeError("MG_ERR_INVALID_ARG: the workspace must be contiguous")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().mg_conv2d(ctypes.byref(shape), x.data_ptr(), w.data_ptr(), swk, swn,
                           bias.data_ptr() if bias is not None else None, out.data_ptr(), ws_ptr, ws_bytes,
                           _dtype_code(x), _stream(x)))
    return out


def mg_attention_scores(q, k, out=None):
    """out[h] = q[h] @ k[h]^T for every head h in one launch.

    q: [heads, Lq, d], k: [heads, Lk, d] with unit stride along d (fp16/bf16);
    returns [heads, Lq, Lk]."""
    import torch

    _require_gpu(q, k)
    if q.dim() != 3 or k.dim() != 3 or q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2]:
        raise RuntimeError("MG_ERR_INVALID_ARG: q[heads,Lq,d] and k[heads,Lk,d] expected")
    H, Lq, d = q.shape
    Lk = k.shape[1]
    if (d > 1 and (q.stride(2) != 1 or k.stride(2) != 1)) or k.dtype != q.dtype:
        raise RuntimeError("MG_ERR_UNSUPPORTED_LAYOUT: unit stride along d and one dtype required")
    if out is None:
        out = torch.empty((H, Lq, Lk), dtype=q.dtype, device=q.device)
    _check_out(out, (H, Lq, Lk), q)
    _check(lib().mg_attention_scores(q.data_ptr(), k.data_ptr(), out.data_ptr(), H, Lq, Lk, d, q.stride(0),
                                     q.stride(1), k.stride(0), k.stride(1), out.stride(0), out.stride(1),
                                     _dtype_code(q), _stream(q)))
    return out


# short names
gemm = mg_gemm
gemm_bias_relu = mg_gemm_bias_relu
gemm_batched = mg_gemm_batched
gemm_splitk = mg_gemm_splitk
grouped_gemm = mg_grouped_gemm
prepack_a = mg_prepack_a
gemm_prepacked = mg_gemm_prepacked
conv2d = mg_conv2d
im2col = mg_im2col
attention_scores = mg_attention_scores
