"""Comparisons of a GEMM result with the oracle -- TEST INFRASTRUCTURE ONLY.

* bit-exact check for integer-valued inputs (the fp32 accumulation is then
  exact, so the single rounding of the exact sum is the only correct answer);
  +0 and -0 compare equal;
* tolerance check |got - ref| <= atol + rtol*|ref| with ref the unrounded fp64
  oracle value, atol = rtol = 1e-2 for fp16 / bf16 ("Triton study notes",
  section 2.1, which also fixes the order of got and ref) and no NaN / Inf;
* Higham's a-priori bound for floating-point summation (N. J. Higham,
  "Accuracy and Stability of Numerical Algorithms", 2nd ed., section 3.1):
  an fp32 sum of K exact products, in any order, is within
  gamma_K * sum_k |a_ik||b_kj| of the exact value, gamma_n = n u / (1 - n u),
  u = 2^-24; one rounding to the output type adds at most u_out |x|
  (u_out = 2^-11 for fp16, 2^-8 for bf16) and, for fp16, half the subnormal
  spacing 2^-25.  Far tighter than the 1e-2 gate on N(0,1)/sqrt(K) data, it
  catches dropped or doubled k-blocks and a wrong output rounding;
* the seeded 4096-element sample and the deterministic edge set.
"""
from __future__ import annotations

import numpy as np

F16 = 0
BF16 = 1


def to_f64(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Exact fp64 value of fp16 / bf16 bit patterns, through numpy's own types."""
    b = np.asarray(bits, dtype=np.uint16)
    if dtype == F16:
        return b.view(np.float16).astype(np.float64)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bitexact_mismatches(got_bits: np.ndarray, ref_q_bits: np.ndarray) -> np.ndarray:
    """Indices where the bit patterns differ, treating +0 and -0 as equal."""
    g = np.asarray(got_bits, dtype=np.uint16)
    r = np.asarray(ref_q_bits, dtype=np.uint16)
    zero_g = (g & 0x7FFF) == 0
    zero_r = (r & 0x7FFF) == 0
    bad = (g != r) & ~(zero_g & zero_r)
    return np.flatnonzero(bad)


def tolerance_mismatches(got_bits, ref, dtype: int, atol: float = 1e-2, rtol: float = 1e-2) -> np.ndarray:
    got = to_f64(got_bits, dtype)
    ref = np.asarray(ref, dtype=np.float64)
    ok = np.isfinite(got) & (np.abs(got - ref) <= atol + rtol * np.abs(ref))
    return np.flatnonzero(~ok)


def describe(idx, got_bits, ref, dtype, shape=None, limit=5) -> str:
    got = to_f64(got_bits, dtype).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    lines = ["%d mismatching elements" % len(idx)]
    for i in idx[:limit]:
        pos = np.unravel_index(i, shape) if shape is not None else i
        lines.append("  at %s: got %r ref %r" % (pos, got[i], ref[i]))
    return "\n".join(lines)


U_F32 = 2.0 ** -24
U_OUT = {F16: 2.0 ** -11, BF16: 2.0 ** -8}
SUBNORMAL_FLOOR = {F16: 2.0 ** -25, BF16: 0.0}


def gamma(n: int, u: float = U_F32) -> float:
    """gamma_n = n u / (1 - n u), the summation constant (n u < 1)."""
    assert n * u < 1.0
    return n * u / (1.0 - n * u)


def higham_bound(absdot, ref, K: int, dtype: int, abs_bias=None) -> np.ndarray:
    """Bound on |got - ref| for an fp32-accumulated dot product of K exact
    products, rounded once to `dtype`: (1 + u_out) E + u_out |ref| + floor with
    E = gamma_K sum_k |a_k b_k| (gamma_{K+1} and + |bias| when an fp32 bias
    add follows).  ReLU is 1-Lipschitz, so the bound carries through it."""
    absdot = np.asarray(absdot, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if abs_bias is not None:
        E = gamma(K + 1) * (absdot + np.asarray(abs_bias, dtype=np.float64))
    else:
        E = gamma(max(K, 1)) * absdot
    u_out = U_OUT[dtype]
    return (1.0 + u_out) * E + u_out * np.abs(ref) + SUBNORMAL_FLOOR[dtype]


def higham_ratio(got_bits, ref, bound, dtype: int) -> float:
    """max |got - ref| / bound over the elements (inf if any got is not finite)."""
    got = to_f64(got_bits, dtype)
    ref = np.asarray(ref, dtype=np.float64)
    if got.size == 0:
        return 0.0
    if not np.all(np.isfinite(got)):
        return float("inf")
    return float(np.max(np.abs(got - ref) / np.asarray(bound, dtype=np.float64)))


def abs_bits(bits) -> np.ndarray:
    """|x| of fp16 / bf16 bit patterns (sign bit cleared)."""
    return np.asarray(bits, dtype=np.uint16) & np.uint16(0x7FFF)


def sample_positions(M: int, N: int, count: int, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """`count` distinct (row, col) pairs uniform over [0,M) x [0,N), seeded."""
    total = M * N
    count = min(count, total)
    flat = np.random.default_rng(seed).choice(total, size=count, replace=False)
    return (flat // N).astype(np.int64), (flat % N).astype(np.int64)


def edge_positions(M: int, N: int, tile: int = 256, segment_starts=None, cols_per_row: int = 8,
                   seed: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Deterministic edge set: first/last row and column, the last row of each
    tile boundary, and (grouped) the first and last row of every segment."""
    rng = np.random.default_rng(seed)
    rows, cols = [], []
    edge_rows = {0, M - 1} | {r for r in range(tile - 1, M, tile)}
    if segment_starts is not None:
        s = list(segment_starts)
        for a, b in zip(s[:-1], s[1:]):
            if b > a:
                edge_rows |= {a, b - 1}
    edge_cols = {0, N - 1} | {c for c in range(tile - 1, N, tile)}
    for r in sorted(edge_rows):
        cs = set(rng.choice(N, size=min(cols_per_row, N), replace=False).tolist()) | {0, N - 1}
        for c in sorted(cs):
            rows.append(r)
            cols.append(c)
    for c in sorted(edge_cols):
        for r in sorted(set(rng.choice(M, size=min(cols_per_row, M), replace=False).tolist()) | {0, M - 1}):
            rows.append(r)
            cols.append(c)
    pairs = sorted(set(zip(rows, cols)))
    return (np.array([p[0] for p in pairs], dtype=np.int64), np.array([p[1] for p in pairs], dtype=np.int64))
