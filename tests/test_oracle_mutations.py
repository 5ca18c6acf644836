"""Planted mistakes in copies of the oracle (CPU only) must each fail at least one pin.

Each mutation rewrites one spot of oracle.c the way a plausible slip would (a dropped
term, a wrong sign, a transposed or mis-indexed operand, an off-by-one exponent, a wrong
constant, truncation instead of rounding), compiles the copy into a temporary library and
runs the pins against it.  The real oracle is never modified.
"""

import os

import pytest

import oracle
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTATIONS = {
    "drop_last_k_term": ("for (int64_t k = 0; k < K; ++k) {\n            double a",
                         "for (int64_t k = 0; k < K - 1; ++k) {\n            double a"),
    "subtract_products": ("c[j] += a * b[j];", "c[j] -= a * b[j];"),
    "nk_layout_not_transposed": ("b_layout == OR_B_KN ? B[k * N + j] : B[j * K + k]",
                                 "B[k * N + j]"),
    "kn_layout_transposed": ("b_layout == OR_B_KN ? B[k * N + j] : B[j * K + k]",
                             "B[j * K + k]"),
    "a_index_transposed": ("decode(A[i * K + k], in_dtype)", "decode(A[k * M + i], in_dtype)"),
    "f16_exponent_off_by_one": ("ldexp((double)(1024 + f), e - 25)",
                                "ldexp((double)(1024 + f), e - 24)"),
    "f16_subnormal_scale": ("ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    "bf16_fraction_bits": ("ldexp((double)(128 + f), e - 134)", "ldexp((double)(256 + f), e - 135)"),
    "round_by_truncation": ("double r = nearbyint(q);", "double r = trunc(q);"),
    "round_half_up": ("double r = nearbyint(q);", "double r = floor(q + 0.5);"),
    "gelu_cubic_decimal_slip": ("0.7978845608 * (x + 0.044715", "0.7978845608 * (x + 0.44715"),
    "gelu_two_over_pi": ("0.7978845608 * (x + 0.044715", "0.6366197724 * (x + 0.044715"),
    "gelu_dropped_cubic": ("(x + 0.044715 * x * x * x)", "(x)"),
    "gelu_exp_sign": ("(1.0 + exp(-2.0 * u))", "(1.0 + exp(2.0 * u))"),
    "gelu_half_dropped": ("return 0.5 * x * (2.0 /", "return x * (2.0 /"),
    "gelu_exp_of_u": ("exp(-2.0 * u)", "exp(-u)"),
    "epilogue_skipped": ("c[j] = oracle_gelu_tanh(c[j]);", "c[j] = c[j];"),
    "relu_as_abs": ("return x > 0.0 ? x : 0.0;", "return fabs(x);"),
    "relu_keeps_negatives": ("return x > 0.0 ? x : 0.0;", "return x < 0.0 ? x : 0.0;"),
    "relu_threshold_one": ("return x > 0.0 ? x : 0.0;", "return x > 1.0 ? x : 0.0;"),
    "relu_skipped": ("c[j] = oracle_relu(c[j]);", "c[j] = c[j];"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.compile_source(str(mutated), str(tmp_path / "liboracle_mut.so"))
    o = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            failed.append(pin.__name__)
        except (RuntimeError, ValueError, OverflowError):
            failed.append(pin.__name__)
        if failed:
            break
    assert failed, f"no pin caught the planted mistake {name}"
