"""Planted mistakes in copies of the comparison metric (CPU only) must each fail a pin.

Each mutation rewrites one spot of oracle/metrics.py the way a plausible slip would: a
wrong fraction width or minimum exponent of an output format, a whole ulp subtracted
instead of half, the ulp or the rounding floor taken of the result instead of the
reference, the wrong error gating a format, a signed difference, a widened relative term
of the elementwise bound, a missing square root in the scale, a doubled tolerance, and
the earlier floor(log2) binade (zero given the spacing of [1, 2), values just below a
power of two given the next binade's).  The copy is loaded as a module of the ``oracle``
package (it imports the oracle's rounding) and the pins in tests/metric_pins.py run
against it.  The real module is never modified.
"""

import importlib.util
import os

import pytest

import oracle
from tests import metric_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "metrics.py")

MUTATIONS = {
    "bf16_fraction_bits_6": ('_FBITS = {"f16": 10, "bf16": 7, "f32": 23}',
                             '_FBITS = {"f16": 10, "bf16": 6, "f32": 23}'),
    "f16_fraction_bits_11": ('_FBITS = {"f16": 10, "bf16": 7, "f32": 23}',
                             '_FBITS = {"f16": 11, "bf16": 7, "f32": 23}'),
    "f32_fraction_bits_24": ('_FBITS = {"f16": 10, "bf16": 7, "f32": 23}',
                             '_FBITS = {"f16": 10, "bf16": 7, "f32": 24}'),
    "f16_emin_off_by_one": ('_EMIN = {"f16": -14, "bf16": -126, "f32": -126}',
                            '_EMIN = {"f16": -15, "bf16": -126, "f32": -126}'),
    "bf16_emin_as_f16": ('_EMIN = {"f16": -14, "bf16": -126, "f32": -126}',
                         '_EMIN = {"f16": -14, "bf16": -14, "f32": -126}'),
    "binade_off_by_one": ("b = np.where(ax > 0, e.astype(np.float64) - 1.0, float(_EMIN[dtype]))",
                          "b = np.where(ax > 0, e.astype(np.float64), float(_EMIN[dtype]))"),
    "zero_in_unit_binade": ("b = np.where(ax > 0, e.astype(np.float64) - 1.0, float(_EMIN[dtype]))",
                            "b = np.where(ax > 0, e.astype(np.float64) - 1.0, 0.0)"),
    "binade_from_log2": ("b = np.where(ax > 0, e.astype(np.float64) - 1.0, float(_EMIN[dtype]))",
                         "b = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))"),
    "whole_ulp_subtracted": ("excess = np.maximum(0.0, d - 0.5 * ulp(C_ref, out_dtype))",
                             "excess = np.maximum(0.0, d - ulp(C_ref, out_dtype))"),
    "ulp_of_result": ("excess = np.maximum(0.0, d - 0.5 * ulp(C_ref, out_dtype))",
                      "excess = np.maximum(0.0, d - 0.5 * ulp(C, out_dtype))"),
    "floor_of_result": ("np.abs(round_to(C_ref, out_dtype) - C_ref)",
                        "np.abs(round_to(C, out_dtype) - C_ref)"),
    "literal_gate_for_16bit": ('gate = err_lit if out_dtype == "f32" else err_q', "gate = err_lit"),
    "quantized_gate_for_f32": ('gate = err_lit if out_dtype == "f32" else err_q', "gate = err_q"),
    "signed_difference": ("d = np.abs(C - C_ref)", "d = C - C_ref"),
    "tolerance_doubled": ('TOL = {"f16": 4e-3, "bf16": 4e-3, "f32": 1e-4}',
                          'TOL = {"f16": 8e-3, "bf16": 8e-3, "f32": 1e-4}'),
    "scale_without_sqrt": ("return math.sqrt(max(K, 1)) * max_abs_a * max_abs_b",
                           "return max(K, 1) * max_abs_a * max_abs_b"),
    "elementwise_rel_times_4": ("EW_REL = 2.0 ** -16", "EW_REL = 2.0 ** -14"),
    "elementwise_whole_ulp": ("bound = 0.5 * ulp(g[fin], out_dtype)", "bound = ulp(g[fin], out_dtype)"),
    "elementwise_rel_of_result": ("EW_REL * np.abs(g[fin])", "EW_REL * np.abs(y[fin]) * 4"),
    "elementwise_nan_ignored": (
        '"ok": excess <= 0.0 and bool(np.array_equal(nan_y, nan_g)) and inf_ok',
        '"ok": excess <= 0.0 and inf_ok'),
}


def _load(path, name):
    spec = importlib.util.spec_from_file_location(f"oracle.{name}", path)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_metric_mutation_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = tmp_path / f"metrics_{name}.py"
    path.write_text(src.replace(old, new))
    m = _load(str(path), f"metrics_{name}")
    failed = []
    for pin in metric_pins.ALL_PINS:
        try:
            pin(m)
        except AssertionError:
            failed.append(pin.__name__)
            break
    assert failed, f"no pin caught the planted mistake {name}"


def test_unmutated_copy_passes(tmp_path):
    # the loader itself does not make pins fail
    path = tmp_path / "metrics_copy.py"
    path.write_text(open(SRC).read())
    m = _load(str(path), "metrics_copy")
    for pin in metric_pins.ALL_PINS:
        pin(m)
