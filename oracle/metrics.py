"""Error metrics for comparing a GEMM result with the oracle -- TEST INFRASTRUCTURE.

Scale of the bound: s = sqrt(K) * max|A| * max|B|.

* ``err_lit`` = max |C - C_ref| / s, the literal bound (4e-3 for a 16-bit
  output, 1e-4 for an fp32 output).
* ``floor``   = max |round_out(C_ref) - C_ref| / s, what a correctly rounded
  output of the exact result would already score on err_lit.
* ``err_q``   = max max(0, |C - C_ref| - ulp_out(C_ref)/2) / s, the error in
  excess of the output format's own rounding.  For a bf16 output at K = 8192
  the literal bound is below the rounding floor (|C| reaches 128 and beyond,
  where half an ulp is 0.5 against an allowance of 4e-3 * sqrt(8192) = 0.36),
  so the gate for 16-bit outputs is err_q; err_lit is always reported beside it.
"""

from __future__ import annotations

import math

import numpy as np

from . import round_to

TOL = {"f16": 4e-3, "bf16": 4e-3, "f32": 1e-4}

_FBITS = {"f16": 10, "bf16": 7, "f32": 23}
_EMIN = {"f16": -14, "bf16": -126, "f32": -126}


def ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the output format at |x|: 2^(e - p) for |x| in the binade [2^e, 2^(e+1)),
    p the format's fraction bits; the subnormal spacing 2^(emin - p) below the normal range
    and at zero.  The binade comes from frexp, which is exact (a floor of log2 rounds up
    into the next binade just below a power of two)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(ax)                     # ax = f 2^e with 0.5 <= f < 1: binade e - 1
    b = np.where(ax > 0, e.astype(np.float64) - 1.0, float(_EMIN[dtype]))
    b = np.maximum(b, _EMIN[dtype])
    return np.exp2(b - _FBITS[dtype])


def scale(K: int, max_abs_a: float, max_abs_b: float) -> float:
    return math.sqrt(max(K, 1)) * max_abs_a * max_abs_b


def compare(C: np.ndarray, C_ref: np.ndarray, out_dtype: str, s: float) -> dict:
    """Return err_lit, err_q, floor, and pass/fail at the tolerance for out_dtype."""
    C = np.asarray(C, dtype=np.float64)
    C_ref = np.asarray(C_ref, dtype=np.float64)
    if C.shape != C_ref.shape:
        raise ValueError(f"shape mismatch {C.shape} vs {C_ref.shape}")
    if s <= 0:
        s = 1.0
    if C.size == 0:
        return {"err_lit": 0.0, "err_q": 0.0, "floor": 0.0, "tol": TOL[out_dtype], "ok": True,
                "nonfinite": 0}
    nonfinite = int(np.count_nonzero(~np.isfinite(C)))
    d = np.abs(C - C_ref)
    err_lit = float(np.max(d)) / s
    floor = float(np.max(np.abs(round_to(C_ref, out_dtype) - C_ref))) / s
    excess = np.maximum(0.0, d - 0.5 * ulp(C_ref, out_dtype))
    err_q = float(np.max(excess)) / s
    tol = TOL[out_dtype]
    gate = err_lit if out_dtype == "f32" else err_q
    return {"err_lit": err_lit, "err_q": err_q, "floor": floor, "tol": tol,
            "ok": bool(nonfinite == 0 and gate <= tol), "nonfinite": nonfinite}


# Standalone elementwise GELU (fp32 evaluation, round to nearest even):
#   |y - g| <= ulp_out(g)/2 + EW_REL |g| + EW_ABS
# with g the exact (double) gelu of the stored input.  EW_REL bounds the fp32
# evaluation: the exponent argument -2 log2(e) u carries ~3 roundings, and an
# argument error of d moves exp2 by ln(2) |t| d relatively, |t| <= 128 before the
# fp32 exponent overflows: 128 * 0.69 * 3 * 2^-24 + 2 * 2^-24 < 2^-16.  EW_ABS covers
# the far negative side where exp2 overflows and the fp32 result is 0 while the
# exact value is a (sub)normal below 2^-120.
EW_REL = 2.0 ** -16
EW_ABS = 2.0 ** -120


def compare_elementwise(y: np.ndarray, g: np.ndarray, out_dtype: str) -> dict:
    """Worst excess over the elementwise GELU bound (<= 0 passes), NaN agreement, and
    the fraction of results equal to the correctly rounded exact value."""
    y = np.asarray(y, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    nan_y, nan_g = np.isnan(y), np.isnan(g)
    fin = ~nan_g & np.isfinite(g)
    inf_ok = bool(np.all(y[np.isinf(g)] == g[np.isinf(g)]))
    d = np.abs(y[fin] - g[fin])
    bound = 0.5 * ulp(g[fin], out_dtype) + EW_REL * np.abs(g[fin]) + EW_ABS
    excess = float(np.max(d - bound)) if d.size else -1.0
    exact = float(np.mean(y[fin] == round_to(g[fin], out_dtype))) if d.size else 1.0
    return {"excess": excess, "nan_match": bool(np.array_equal(nan_y, nan_g)), "inf_ok": inf_ok,
            "exact_frac": exact, "ok": excess <= 0.0 and bool(np.array_equal(nan_y, nan_g)) and inf_ok}
