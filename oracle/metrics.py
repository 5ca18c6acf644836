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
    """Spacing of the output format at |x| (binade-wise; subnormal spacing below)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, _EMIN[dtype])
    return np.exp2(e - _FBITS[dtype])


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
