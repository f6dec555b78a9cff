"""The pins catch plausible mistakes in the oracle.

Each case compiles a copy of oracle/gemm_oracle.c with one deliberate,
plausible mistake (a dropped term, a wrong index, a wrong sign, ties rounded
away from zero, a signed-zero ReLU, a wrong subnormal scale, a wrong expert
weight; in the convolution a dropped dilation, a padding sign, swapped kernel
axes, non-zero padding) into a temporary directory, binds the oracle's Python functions to
it, and checks that at least one pin fails.  The real oracle is rebound
afterwards.  CPU only; nothing here touches the GPU path.
"""
import os
import tempfile

import pytest

import oracle
from tests import test_oracle_gemm as G
from tests import test_oracle_consumers as CV
from tests import test_oracle_rounding as R

SRC = os.path.join(os.path.dirname(oracle.__file__), "gemm_oracle.c")

MUTANTS = {
    "drops the last k term": ("for (int64_t k = 0; k < j->K; ++k) {\n            const double a = arow[k];",
                              "for (int64_t k = 0; k + 1 < j->K; ++k) {\n            const double a = arow[k];"),
    "reads A's row backwards": ("const double a = arow[k];", "const double a = arow[j->K - 1 - k];"),
    "subtracts the bias": ("if (bias) v = v + orc_decode(bias[j], dtype);",
                           "if (bias) v = v - orc_decode(bias[j], dtype);"),
    "rounds ties away from zero": ("double n = rint(ldexp(a, -(int)quantum_exp));",
                                   "double n = round(ldexp(a, -(int)quantum_exp));"),
    "ReLU gives -0.0": ("if (relu) v = (v > 0.0) ? v : 0.0;", "if (relu) v = (v > 0.0) ? v : -0.0;"),
    "wrong subnormal scale": ("v = ldexp((double)frac, 1 - f.bias - f.frac_bits);",
                              "v = ldexp((double)frac, -f.bias - f.frac_bits);"),
    "uses the previous expert's weights": ("double* Wd = decode_matrix(W + e * stride_we, K, N, ldw, dtype);",
                                           "double* Wd = decode_matrix(W + (e > 0 ? e - 1 : 0) * stride_we, K, N, ldw, dtype);"),
    "accumulates in single precision": ("for (int64_t n = 0; n < j->N; ++n) acc[n] += a * brow[n];",
                                        "for (int64_t n = 0; n < j->N; ++n) acc[n] = (float)(acc[n] + (float)(a * brow[n]));"),
    "convolution ignores the dilation": ("const int64_t ih = oh * sh - ph + kh * dh;",
                                         "const int64_t ih = oh * sh - ph + kh;"),
    "convolution pads on the wrong side": ("const int64_t iw = ow * sw - pw + kw * dw;",
                                           "const int64_t iw = ow * sw + pw + kw * dw;"),
    "convolution swaps kh and kw in the weights": ("acc += xv * w[((kh * KW + kw) * C + c) * OC + o];",
                                                   "acc += xv * w[((kw * KH + kh) * C + c) * OC + o];"),
    "convolution pads with ones": ("const double xv = inside ? x[((n * H + ih) * W + iw) * C + c] : 0.0;",
                                   "const double xv = inside ? x[((n * H + ih) * W + iw) * C + c] : 1.0;"),
}

PINS = [
    lambda o: G.test_textbook_2x2(o),
    lambda o: G.test_all_ones_closed_form(o, 3, 5, 256, 0),
    lambda o: G.test_integer_brute_force_is_exact(o, 0),
    lambda o: G.test_agrees_with_numpy_matmul(o),
    lambda o: G.test_epilogue_bias_relu(o),
    lambda o: G.test_grouped_is_concatenation_of_dense(o),
    lambda o: R.test_decode_all_patterns_match_numpy(o, 0),
    lambda o: R.test_encode_midpoints_ties_to_even(o, 0),
    lambda o: R.test_encode_midpoints_ties_to_even(o, 1),
    lambda o: CV.test_conv_worked_examples(o),
    lambda o: CV.test_conv_matches_torch_float64(o, CV.CONV_PARAMS[3], 0),
    lambda o: CV.test_conv_matches_torch_float64(o, CV.CONV_PARAMS[4], 0),
]


def test_mutant_table_applies_to_source():
    src = open(SRC).read()
    for name, (old, _) in MUTANTS.items():
        assert src.count(old) == 1, name


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib = oracle.build(force=True, src=path, out=os.path.join(d, "libmutant.so"))
        failures = 0
        try:
            oracle.use_library(lib)
            for pin in PINS:
                try:
                    pin(oracle)
                except AssertionError:
                    failures += 1
        finally:
            oracle.use_library(None)
        assert failures > 0, "no pin caught the mutant: " + name
