"""Pins of the oracle's fp16 / bf16 decode and round-to-nearest-even encode.

The oracle's conversions are checked against things fixed outside it:
numpy's own float16 / float32 types for decoding, exact rational arithmetic
(fractions.Fraction) over the table of all representable values for the
rounding of every midpoint, and numpy's float64 -> float16 cast on random
doubles.
"""
from fractions import Fraction

import numpy as np
import pytest

F16, BF16 = 0, 1
ALL = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def numpy_decode(bits, dtype):
    if dtype == F16:
        return bits.view(np.float16).astype(np.float64)
    with np.errstate(invalid="ignore"):
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def finite_positive_table(dtype):
    vals = numpy_decode(ALL, dtype)
    keep = np.isfinite(vals) & (vals > 0) & (ALL < 0x8000)
    order = np.argsort(vals[keep], kind="stable")
    return vals[keep][order], ALL[keep][order]


def rne_by_table(x: Fraction, fv, bits, overflow_value: Fraction):
    """Nearest representable value to x > 0, ties to the even bit pattern.

    fv are the exact positive finite values in increasing order, bits their
    patterns; overflow_value is the first power of two beyond the largest
    finite value, and rounding towards it means +Inf."""
    # binary search over the exact values
    lo, hi = 0, len(fv) - 1
    if x <= fv[0]:
        below = Fraction(0)
        below_bits = 0
        above, above_bits = fv[0], int(bits[0])
    elif x >= fv[-1]:
        below, below_bits = fv[-1], int(bits[-1])
        above, above_bits = overflow_value, None
    else:
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if fv[mid] <= x:
                lo = mid
            else:
                hi = mid
        below, below_bits = fv[lo], int(bits[lo])
        above, above_bits = fv[hi], int(bits[hi])
    if x == below:
        return below_bits
    d_lo, d_hi = x - below, above - x
    if d_lo < d_hi:
        return below_bits
    if d_hi < d_lo:
        return "inf" if above_bits is None else above_bits
    # tie: the even one (last fraction bit 0); the overflow side counts as even
    if above_bits is None:
        return "inf"
    return below_bits if below_bits % 2 == 0 else above_bits


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_decode_all_patterns_match_numpy(orc, dtype):
    got = orc.decode(ALL, dtype)
    want = numpy_decode(ALL, dtype)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signs of zeros
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_encode_roundtrip_every_pattern(orc, dtype):
    vals = numpy_decode(ALL, dtype)
    finite = ~np.isnan(vals)
    back = orc.encode(vals[finite], dtype)
    assert np.array_equal(back, ALL[finite])
    nan_back = orc.encode(vals[~finite], dtype)
    assert np.all(np.isnan(numpy_decode(nan_back, dtype)))


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_encode_midpoints_ties_to_even(orc, dtype):
    vals, bits = finite_positive_table(dtype)
    mids = (vals[:-1] + vals[1:]) / 2.0  # exact: neighbours differ by one quantum
    got = orc.encode(mids, dtype)
    # exact expectation: between two neighbours, the tie goes to the even pattern
    lower_even = (bits[:-1] % 2) == 0
    want = np.where(lower_even, bits[:-1], bits[1:])
    assert np.array_equal(got, want)
    # a hair above / below each midpoint goes to the nearer neighbour
    up = orc.encode(np.nextafter(mids, np.inf), dtype)
    dn = orc.encode(np.nextafter(mids, -np.inf), dtype)
    assert np.array_equal(up, bits[1:])
    assert np.array_equal(dn, bits[:-1])
    # negative values mirror the positive ones with the sign bit set
    neg = orc.encode(-mids, dtype)
    assert np.array_equal(neg, want | 0x8000)


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_encode_random_doubles_against_exact_rationals(orc, dtype):
    vals, bits = finite_positive_table(dtype)
    top = Fraction(2) ** (16 if dtype == F16 else 128)
    rng = np.random.default_rng(7)
    lo_exp, hi_exp = (-26, 16) if dtype == F16 else (-135, 128)
    xs = np.ldexp(rng.uniform(1.0, 2.0, size=400), rng.integers(lo_exp, hi_exp, size=400))
    got = orc.encode(xs, dtype)
    fv = [Fraction(float(v)) for v in vals]
    for x, g in zip(xs, got):
        w = rne_by_table(Fraction(float(x)), fv, bits, top)
        if w == "inf":
            assert g == (0x7C00 if dtype == F16 else 0x7F80), x
        else:
            assert int(g) == w, (x, hex(int(g)), hex(w))


def test_encode_f16_matches_numpy_cast_on_random_doubles(orc):
    rng = np.random.default_rng(11)
    xs = np.concatenate([
        rng.standard_normal(400_000),
        rng.standard_normal(300_000) * 1e-5,      # subnormal range
        rng.standard_normal(300_000) * 3e4,       # near overflow
    ])
    with np.errstate(over="ignore"):
        want = xs.astype(np.float16).view(np.uint16)
    got = orc.encode(xs, F16)
    assert np.array_equal(got, want)


def test_overflow_boundaries(orc):
    # fp16: largest finite 65504; the midpoint to 65536 (65520) ties to "even" = Inf
    assert orc.encode([65504.0], F16)[0] == 0x7BFF
    assert orc.encode([65519.99], F16)[0] == 0x7BFF
    assert orc.encode([65520.0], F16)[0] == 0x7C00
    assert orc.encode([-1e9], F16)[0] == 0xFC00
    # bf16: largest finite (2 - 2^-7) * 2^127
    big = (2 - 2 ** -7) * 2.0 ** 127
    assert orc.encode([big], BF16)[0] == 0x7F7F
    assert orc.encode([(2 - 2 ** -8) * 2.0 ** 127], BF16)[0] == 0x7F80
    assert orc.encode([np.inf], BF16)[0] == 0x7F80
    assert orc.encode([-np.inf], F16)[0] == 0xFC00


def test_integer_values_are_exact_and_large_integers_round_to_even(orc):
    ints = np.arange(-2048, 2049, dtype=np.float64)
    assert np.array_equal(orc.decode(orc.encode(ints, F16), F16), ints)
    ints_bf = np.arange(-256, 257, dtype=np.float64)
    assert np.array_equal(orc.decode(orc.encode(ints_bf, BF16), BF16), ints_bf)
    # spacing 2 above 2048 in fp16: 2049 -> 2048 (even), 2051 -> 2052
    assert orc.decode(orc.encode([2049.0, 2051.0], F16), F16).tolist() == [2048.0, 2052.0]
    # spacing 2 above 256 in bf16: 257 -> 256, 259 -> 260
    assert orc.decode(orc.encode([257.0, 259.0], BF16), BF16).tolist() == [256.0, 260.0]
