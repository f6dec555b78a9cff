"""Pins of the comparison gates in oracle/compare.py (CPU only).

Every GPU parity verdict passes through these functions, so each one is fed
inputs whose verdict is fixed by hand: bit patterns one ulp apart, signed
zeros, NaN and Inf, values exactly on and one ulp past the tolerance
|got - ref| <= atol + rtol |ref| ("Triton study notes", section 2.1, which
puts the reference value on the right-hand side), and sample / edge sets
whose contents follow from their definition.  The checks are written as functions of the
module under test so that `test_compare_mutants` can run them against
deliberately broken copies of compare.py and show that each copy fails one.
"""
import importlib.util
import os
import tempfile

import numpy as np
import pytest

from oracle import compare

F16, BF16 = 0, 1
HERE = os.path.dirname(os.path.abspath(__file__))
COMPARE_SRC = os.path.join(os.path.dirname(HERE), "oracle", "compare.py")


def fp16_bits(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


# ---- to_f64 ------------------------------------------------------------------
def check_to_f64(cmp):
    # fp16 fields: sign 1, exponent 5 (bias 15), fraction 10
    f16 = {0x3C00: 1.0, 0xC000: -2.0, 0x3555: 1365 / 4096, 0x0001: 2.0 ** -24, 0x03FF: 1023 * 2.0 ** -24,
           0x0400: 2.0 ** -14, 0x7BFF: 65504.0, 0x8000: -0.0}
    # bf16 fields: sign 1, exponent 8 (bias 127), fraction 7
    bf16 = {0x3F80: 1.0, 0xC040: -3.0, 0x3E2B: 0.1669921875, 0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126,
            0x7F7F: 255 * 2.0 ** 120, 0x4B80: 2.0 ** 24}
    for table, dt in ((f16, F16), (bf16, BF16)):
        bits = np.array(list(table), dtype=np.uint16)
        got = cmp.to_f64(bits, dt)
        assert np.array_equal(got, np.array(list(table.values()))), (dt, got)
    assert np.signbit(cmp.to_f64(np.array([0x8000], np.uint16), F16)[0])
    assert np.all(np.isinf(cmp.to_f64(np.array([0x7C00, 0xFC00], np.uint16), F16)))
    assert np.all(np.isinf(cmp.to_f64(np.array([0x7F80, 0xFF80], np.uint16), BF16)))
    assert np.all(np.isnan(cmp.to_f64(np.array([0x7E00, 0x7FC0], np.uint16), F16)))
    assert np.isnan(cmp.to_f64(np.array([0x7FC0], np.uint16), BF16)[0])


# ---- bit-exact gate -------------------------------------------------------------
def check_bitexact(cmp):
    ref = np.array([0x3C00, 0x4B80, 0xC000, 0x0000, 0x8000, 0x0000, 0x3F80, 0x1234], dtype=np.uint16)
    assert cmp.bitexact_mismatches(ref.copy(), ref).size == 0
    # +0 / -0 in either direction are equal
    got = ref.copy()
    got[3], got[4] = 0x8000, 0x0000
    assert cmp.bitexact_mismatches(got, ref).size == 0
    # one ulp up or down anywhere, including next to zero, is flagged
    for i in range(ref.size):
        for delta in (1, -1):
            g = ref.copy()
            g[i] = np.uint16((int(ref[i]) + delta) & 0xFFFF)
            bad = cmp.bitexact_mismatches(g, ref)
            assert bad.tolist() == [i], (i, delta, bad)
    # the smallest subnormal of either sign is not a zero
    for z in (0x0001, 0x8001):
        g = ref.copy()
        g[5] = z
        assert cmp.bitexact_mismatches(g, ref).tolist() == [5]
    # NaN and Inf where a finite value is expected
    for special in (0x7E00, 0x7FC0, 0x7C00, 0xFF80):
        g = ref.copy()
        g[0] = special
        assert cmp.bitexact_mismatches(g, ref).tolist() == [0]
    # a sign flip of a non-zero value
    g = ref.copy()
    g[1] ^= 0x8000
    assert cmp.bitexact_mismatches(g, ref).tolist() == [1]
    # flat indices of a 2-D input
    g2 = ref.reshape(2, 4).copy()
    g2[1, 2] ^= 0x0400
    assert cmp.bitexact_mismatches(g2, ref.reshape(2, 4)).tolist() == [6]


# ---- tolerance gate -------------------------------------------------------------
def check_tolerance(cmp):
    # exact binary atol / rtol: the bound is computed without rounding
    atol, rtol = 0.25, 0.5
    ref = np.array([2.0, -2.0, 0.0, 8.0])
    # bounds 1.25, 1.25, 0.25, 4.25: got exactly on the bound passes
    on = fp16_bits([3.25, -3.25, 0.25, 12.25])
    assert cmp.tolerance_mismatches(on, ref, F16, atol, rtol).size == 0
    on_low = fp16_bits([0.75, -0.75, -0.25, 3.75])
    assert cmp.tolerance_mismatches(on_low, ref, F16, atol, rtol).size == 0
    # one fp16 ulp past the bound fails (ulps: 3.25 -> 2^-9 ... 12.25 -> 2^-7)
    past = fp16_bits([3.25 + 2.0 ** -9, -3.25 - 2.0 ** -9, 0.25 + 2.0 ** -12, 12.25 + 2.0 ** -7])
    assert cmp.tolerance_mismatches(past, ref, F16, atol, rtol).tolist() == [0, 1, 2, 3]
    past_low = fp16_bits([0.75 - 2.0 ** -11, -0.75 + 2.0 ** -11, -0.25 - 2.0 ** -12, 3.75 - 2.0 ** -9])
    assert cmp.tolerance_mismatches(past_low, ref, F16, atol, rtol).tolist() == [0, 1, 2, 3]
    # the relative part is taken on the reference: |got - ref| = 0.75 is within
    # 0.5 |got| = 0.875 but not within 0.5 |ref| = 0.5
    assert cmp.tolerance_mismatches(fp16_bits([1.75]), np.array([1.0]), F16, 0.0, rtol).tolist() == [0]
    assert cmp.tolerance_mismatches(fp16_bits([1.25]), np.array([1.75]), F16, 0.0, rtol).size == 0
    # non-finite results fail even against a huge reference
    bad = np.array([0x7C00, 0xFC00, 0x7E00], dtype=np.uint16)
    assert cmp.tolerance_mismatches(bad, np.array([1e300, -1e300, 0.0]), F16, 1e300, 1.0).tolist() == [0, 1, 2]
    assert cmp.tolerance_mismatches(np.array([0x7F80, 0x7FC0], np.uint16), np.array([3e38, 0.0]), BF16,
                                    1e300, 1.0).tolist() == [0, 1]
    # ... and even with no bound at all: the gate also requires a finite result
    inf_nan_one = np.array([0x7C00, 0x7E00, 0x3C00], dtype=np.uint16)
    assert cmp.tolerance_mismatches(inf_nan_one, np.zeros(3), F16, np.inf, 0.0).tolist() == [0, 1]
    # the default gate is 1e-2 + 1e-2 |ref|: around ref = 4 the bound is 0.05
    ref4 = np.array([4.0, 4.0, 4.0, 4.0])
    got = fp16_bits([4.046875, 3.953125, 4.0546875, 3.9453125])  # |diff| 0.047, 0.047, 0.055, 0.055
    assert cmp.tolerance_mismatches(got, ref4, F16).tolist() == [2, 3]
    got_bf = np.array([0x4082, 0x4084, 0x4081], dtype=np.uint16)  # bf16 4.0625, 4.125, 4.03125
    assert cmp.tolerance_mismatches(got_bf, np.array([4.0, 4.125, 4.0]), BF16).tolist() == [0]


# ---- sample and edge sets -------------------------------------------------------
def check_sample_positions(cmp):
    M, N = 48, 80
    r, c = cmp.sample_positions(M, N, M * N, seed=11)
    # asked for every position, the sample is the whole grid
    assert sorted(zip(r.tolist(), c.tolist())) == [(i, j) for i in range(M) for j in range(N)]
    r, c = cmp.sample_positions(M, N, 10 * M * N, seed=11)  # clamped to the grid
    assert r.size == M * N
    r, c = cmp.sample_positions(3000, 5000, 4096, seed=7)
    assert r.size == 4096 and len(set(zip(r.tolist(), c.tolist()))) == 4096
    assert r.min() >= 0 and r.max() < 3000 and c.min() >= 0 and c.max() < 5000
    # uniform over the grid: every 1000 x 1000 block is hit (expected ~273 each)
    blocks = np.bincount((r // 1000) * 5 + c // 1000, minlength=15)
    assert blocks.min() > 150, blocks
    r2, c2 = cmp.sample_positions(3000, 5000, 4096, seed=7)
    assert np.array_equal(r, r2) and np.array_equal(c, c2)
    r3, _ = cmp.sample_positions(3000, 5000, 4096, seed=8)
    assert not np.array_equal(r, r3)


def check_edge_positions(cmp):
    M, N = 1000, 600
    r, c = cmp.edge_positions(M, N, tile=256)
    pairs = set(zip(r.tolist(), c.tolist()))
    assert len(pairs) == r.size
    assert r.min() >= 0 and r.max() < M and c.min() >= 0 and c.max() < N
    rows, cols = set(r.tolist()), set(c.tolist())
    assert {0, M - 1, 255, 511, 767} <= rows
    assert {0, N - 1, 255, 511} <= cols
    for corner in ((0, 0), (0, N - 1), (M - 1, 0), (M - 1, N - 1)):
        assert corner in pairs
    # grouped: the first and last row of every non-empty segment
    starts = [0, 100, 100, 357, 800, 1000]
    r, c = cmp.edge_positions(M, N, tile=256, segment_starts=starts)
    rows = set(r.tolist())
    assert {0, 99, 100, 356, 357, 799, 800, 999} <= rows
    assert r.max() < M


CHECKS = [check_to_f64, check_bitexact, check_tolerance, check_sample_positions, check_edge_positions]


@pytest.mark.parametrize("check", CHECKS, ids=lambda f: f.__name__)
def test_compare_gate(check):
    check(compare)


# ---- mutants of compare.py ----------------------------------------------------
MUTANTS = {
    "any zero equals anything": ("bad = (g != r) & ~(zero_g & zero_r)", "bad = (g != r) & ~(zero_g | zero_r)"),
    "zero mask ignores the last bit": ("zero_g = (g & 0x7FFF) == 0", "zero_g = (g & 0x7FFE) == 0"),
    "strict inequality at the bound": ("(np.abs(got - ref) <= atol + rtol * np.abs(ref))",
                                       "(np.abs(got - ref) < atol + rtol * np.abs(ref))"),
    "relative part on got": ("(np.abs(got - ref) <= atol + rtol * np.abs(ref))",
                             "(np.abs(got - ref) <= atol + rtol * np.abs(got))"),
    "non-finite results pass": ("ok = np.isfinite(got) & (", "ok = np.isfinite(ref) & ("),
    "bf16 decoded with a 15-bit shift": ("(b.astype(np.uint32) << 16)", "(b.astype(np.uint32) << 15)"),
    "sample rows divided by M": ("return (flat // N).astype(np.int64), (flat % N).astype(np.int64)",
                                 "return (flat // M).astype(np.int64), (flat % M).astype(np.int64)"),
    "sample drawn with replacement": ("size=count, replace=False)", "size=count, replace=True)"),
    "tile boundary rows off by one": ("{r for r in range(tile - 1, M, tile)}", "{r for r in range(tile, M, tile)}"),
    "segment ends off by one": ("edge_rows |= {a, b - 1}", "edge_rows |= {a, b}"),
}


def test_mutant_table_applies_to_source():
    src = open(COMPARE_SRC).read()
    for name, (old, _) in MUTANTS.items():
        assert src.count(old) == 1, name


def _load_mutant(src, directory):
    path = os.path.join(directory, "compare_mutant.py")
    with open(path, "w") as f:
        f.write(src)
    spec = importlib.util.spec_from_file_location("compare_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_compare_mutants(name):
    old, new = MUTANTS[name]
    src = open(COMPARE_SRC).read()
    with tempfile.TemporaryDirectory() as d:
        mod = _load_mutant(src.replace(old, new), d)
        caught = 0
        for check in CHECKS:
            try:
                check(mod)
            except (AssertionError, ValueError, IndexError):
                caught += 1
        assert caught > 0, "no pin caught the mutant: " + name
