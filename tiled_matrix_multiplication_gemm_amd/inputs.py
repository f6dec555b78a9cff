"""Seeded synthetic inputs for the GEMM workloads.

This module only draws random numbers and stores them in the input types; it
holds none of the GEMM's arithmetic.  Both the CPU oracle and the GPU path
consume the bit patterns it returns (numpy ``uint16`` arrays of fp16 / bf16
bits), so the two sides always see identical inputs.

Recipe: numpy ``default_rng(seed)`` (PCG64), draws in float64 in the order
A, B, bias (grouped: expert counts, X, W), then one conversion to the input
type.  No public dataset is involved; the shapes and distributions are those
of the five workloads below.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F16 = 0
BF16 = 1


def to_bits(x: np.ndarray, dtype: int) -> np.ndarray:
    """float64 array -> uint16 bit patterns of fp16 (numpy) or bf16 (torch)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    if dtype == F16:
        return x.astype(np.float16).view(np.uint16)
    import torch

    t = torch.from_numpy(x).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


@dataclass
class DenseCase:
    name: str
    M: int
    N: int
    K: int
    dtype: int
    A: np.ndarray
    B: np.ndarray
    bias: np.ndarray | None = None
    relu: bool = False
    integer: bool = False


@dataclass
class GroupedCase:
    name: str
    E: int
    T: int
    N: int
    K: int
    dtype: int
    counts: np.ndarray
    offsets: np.ndarray
    X: np.ndarray
    W: np.ndarray
    integer: bool = False
    meta: dict = field(default_factory=dict)


# name -> (M, N, K, dtype, bias+relu, float-distribution, seeds)
DENSE_WORKLOADS = {
    "gemm_256_f16": dict(M=256, N=256, K=256, dtype=F16, epilogue=False, dist="uniform1",
                         seed_float=101, seed_int=201, seed_sample=301),
    "gemm_1024x1024x2048_f16": dict(M=1024, N=1024, K=2048, dtype=F16, epilogue=False, dist="normal_sqrtk",
                                    seed_float=102, seed_int=202, seed_stress=212, seed_sample=302),
    "gemm_bias_relu_1024x1024x2048_f16": dict(M=1024, N=1024, K=2048, dtype=F16, epilogue=True,
                                              dist="normal_sqrtk", bias_sigma=0.1,
                                              seed_float=103, seed_int=203, seed_sample=303),
    "gemm_8192_bf16": dict(M=8192, N=8192, K=8192, dtype=BF16, epilogue=False, dist="normal_sqrtk",
                           seed_float=104, seed_int=204, seed_sample=304),
}

GROUPED_WORKLOADS = {
    "grouped_moe_e32_t8192_k1024_n4096_f16": dict(E=32, T=8192, K=1024, N=4096, dtype=F16, w_sigma=0.02,
                                                  seed_float=105, seed_int=205, seed_sample=305),
}


def random_dense(M, N, K, dtype, seed, dist="normal_sqrtk", epilogue=False, bias_sigma=0.1,
                 name="custom") -> DenseCase:
    rng = np.random.default_rng(seed)
    if dist == "uniform1":
        A = rng.uniform(-1.0, 1.0, size=(M, K))
        B = rng.uniform(-1.0, 1.0, size=(K, N))
    elif dist == "normal_sqrtk":
        s = 1.0 / np.sqrt(max(K, 1))
        A = rng.standard_normal(size=(M, K)) * s
        B = rng.standard_normal(size=(K, N)) * s
    else:
        raise ValueError(dist)
    bias = rng.standard_normal(size=N) * bias_sigma if epilogue else None
    return DenseCase(name, M, N, K, dtype, to_bits(A, dtype), to_bits(B, dtype),
                     None if bias is None else to_bits(bias, dtype), relu=epilogue)


def integer_dense(M, N, K, dtype, seed, lo=-4, hi=4, epilogue=False, name="custom") -> DenseCase:
    """Entries uniform on the integers lo..hi inclusive (exact in fp16 / bf16)."""
    rng = np.random.default_rng(seed)
    A = rng.integers(lo, hi + 1, size=(M, K)).astype(np.float64)
    B = rng.integers(lo, hi + 1, size=(K, N)).astype(np.float64)
    bias = rng.integers(-4, 5, size=N).astype(np.float64) if epilogue else None
    return DenseCase(name, M, N, K, dtype, to_bits(A, dtype), to_bits(B, dtype),
                     None if bias is None else to_bits(bias, dtype), relu=epilogue, integer=True)


def subnormal_dense(M, N, K, seed, dtype=F16, name="subnormal") -> DenseCase:
    """A whose entries are k * u with k uniform on -4..4 and u the smallest
    subnormal of the type (2^-24 for fp16, 2^-133 for bf16): zero and the
    four smallest subnormals of either sign.  B integers on -4..4.  Every
    product and partial sum is an integer multiple of u below 2^24 of them,
    exact in fp32 (whose own subnormals reach down to 2^-149), so one
    rounding of the exact sum is the only correct output (subnormal itself
    when small enough)."""
    rng = np.random.default_rng(seed)
    u = 2.0 ** -24 if dtype == F16 else 2.0 ** -133
    A = rng.integers(-4, 5, size=(M, K)).astype(np.float64) * u
    B = rng.integers(-4, 5, size=(K, N)).astype(np.float64)
    return DenseCase(name, M, N, K, dtype, to_bits(A, dtype), to_bits(B, dtype), integer=True)


def dense_f32(M, N, K, seed, integer=False, epilogue=False, name="f32"):
    """fp32 inputs as uint32 bit patterns: N(0,1)/sqrt(K) values, or integers
    on -4..4 (exact products and sums); bias N(0, 0.1) or integers."""
    rng = np.random.default_rng(seed)
    if integer:
        A = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
        B = rng.integers(-4, 5, size=(K, N)).astype(np.float32)
        bias = rng.integers(-4, 5, size=N).astype(np.float32) if epilogue else None
    else:
        s = 1.0 / np.sqrt(max(K, 1))
        A = (rng.standard_normal(size=(M, K)) * s).astype(np.float32)
        B = (rng.standard_normal(size=(K, N)) * s).astype(np.float32)
        bias = (rng.standard_normal(size=N) * 0.1).astype(np.float32) if epilogue else None
    return DenseCase(name, M, N, K, 2, A.view(np.uint32), B.view(np.uint32),
                     None if bias is None else bias.view(np.uint32), relu=epilogue, integer=integer)


def dense_workload(name: str, variant: str = "float") -> DenseCase:
    w = DENSE_WORKLOADS[name]
    if variant == "float":
        c = random_dense(w["M"], w["N"], w["K"], w["dtype"], w["seed_float"], w["dist"], w["epilogue"],
                         w.get("bias_sigma", 0.1), name)
    elif variant == "int":
        c = integer_dense(w["M"], w["N"], w["K"], w["dtype"], w["seed_int"], epilogue=w["epilogue"], name=name)
    elif variant == "stress":
        c = integer_dense(w["M"], w["N"], w["K"], w["dtype"], w["seed_stress"], lo=1, hi=4,
                          epilogue=w["epilogue"], name=name)
    else:
        raise ValueError(variant)
    return c


def offsets_from_counts(counts: np.ndarray) -> np.ndarray:
    """Exclusive prefix sum with the total appended: offsets[e] .. offsets[e+1]-1 are expert e's rows."""
    off = np.zeros(len(counts) + 1, dtype=np.int64)
    np.cumsum(counts, out=off[1:])
    return off.astype(np.int32)


def random_grouped(E, T, K, N, dtype, seed, w_sigma=0.02, counts=None, integer=False,
                   name="custom") -> GroupedCase:
    """Token counts ~ Multinomial(T, uniform over E) unless given; X rows sorted by expert."""
    rng = np.random.default_rng(seed)
    if counts is None:
        counts = rng.multinomial(T, [1.0 / E] * E)
    counts = np.asarray(counts, dtype=np.int64)
    if counts.sum() != T or len(counts) != E:
        raise ValueError("counts must have E entries summing to T")
    if integer:
        X = rng.integers(-4, 5, size=(T, K)).astype(np.float64)
        W = rng.integers(-4, 5, size=(E, K, N)).astype(np.float64)
    else:
        X = rng.standard_normal(size=(T, K))
        W = rng.standard_normal(size=(E, K, N)) * w_sigma
    return GroupedCase(name, E, T, N, K, dtype, counts, offsets_from_counts(counts),
                       to_bits(X, dtype), to_bits(W, dtype), integer=integer)


def grouped_workload(name: str, variant: str = "float", counts=None) -> GroupedCase:
    w = GROUPED_WORKLOADS[name]
    seed = w["seed_float"] if variant == "float" else w["seed_int"]
    return random_grouped(w["E"], w["T"], w["K"], w["N"], w["dtype"], seed, w["w_sigma"], counts=counts,
                          integer=(variant == "int"), name=name)


# ---- GEMM consumers ------------------------------------------------------------
# The pages name no convolution or attention workload; the shapes below are a
# mid-network 3x3 convolution stage and one attention layer's scores, with
# He-style weight scaling so that outputs are O(1).
F32 = 2


def _store(x: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float64).astype(np.float32).view(np.uint32)
    return to_bits(x, dtype)


@dataclass
class ConvCase:
    name: str
    x: np.ndarray          # NHWC [Nb,H,W,C] bit patterns
    w: np.ndarray          # [KH,KW,C,OC] bit patterns
    bias: np.ndarray | None
    dtype: int
    stride: tuple
    pad: tuple
    dil: tuple
    integer: bool


def conv_case(Nb, H, W, C, OC, KH, KW, dtype, seed, stride=(1, 1), pad=(0, 0), dil=(1, 1), integer=False,
              bias=False, name="conv") -> ConvCase:
    """x ~ N(0,1), w ~ N(0,1)/sqrt(KH KW C), bias ~ N(0, 0.1); or integers on
    -4..4 (exact sums).  Drawn in the order x, w, bias."""
    rng = np.random.default_rng(seed)
    K = KH * KW * C
    if integer:
        x = rng.integers(-4, 5, size=(Nb, H, W, C)).astype(np.float64)
        w = rng.integers(-4, 5, size=(KH, KW, C, OC)).astype(np.float64)
        b = rng.integers(-4, 5, size=OC).astype(np.float64) if bias else None
    else:
        x = rng.standard_normal(size=(Nb, H, W, C))
        w = rng.standard_normal(size=(KH, KW, C, OC)) / np.sqrt(max(K, 1))
        b = rng.standard_normal(size=OC) * 0.1 if bias else None
    return ConvCase(name, _store(x, dtype), _store(w, dtype), None if b is None else _store(b, dtype), dtype,
                    tuple(stride), tuple(pad), tuple(dil), integer)


@dataclass
class AttentionCase:
    name: str
    Q: np.ndarray  # [heads, Lq, d] bit patterns
    K: np.ndarray  # [heads, Lk, d] bit patterns
    dtype: int
    integer: bool


def attention_case(heads, Lq, Lk, d, dtype, seed, integer=False, name="attention") -> AttentionCase:
    """Q, K ~ N(0,1) / d^(1/4) each (scores of unit variance); or integers on
    -4..4.  Drawn in the order Q, K."""
    rng = np.random.default_rng(seed)
    if integer:
        q = rng.integers(-4, 5, size=(heads, Lq, d)).astype(np.float64)
        k = rng.integers(-4, 5, size=(heads, Lk, d)).astype(np.float64)
    else:
        s = float(d) ** -0.25
        q = rng.standard_normal(size=(heads, Lq, d)) * s
        k = rng.standard_normal(size=(heads, Lk, d)) * s
    return AttentionCase(name, _store(q, dtype), _store(k, dtype), dtype, integer)


# Timed consumer workloads: a 3x3 convolution stage at batch 32 (56x56, 64 ->
# 64 channels) and the scores of one attention layer (batch 8 x 16 heads,
# 2048 tokens, head dimension 128).
CONV_WORKLOAD = dict(Nb=32, H=56, W=56, C=64, OC=64, KH=3, KW=3, stride=(1, 1), pad=(1, 1), dil=(1, 1),
                     dtype=F16, seed_float=106, seed_int=206)
ATTENTION_WORKLOAD = dict(heads=128, L=2048, d=128, dtype=BF16, seed_float=107, seed_int=207)
