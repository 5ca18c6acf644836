"""Pins for the comparison metric (oracle/metrics.py): checks against facts that do not come
from metrics.py.

The GPU parity gate is whatever ``metrics.compare`` and ``metrics.compare_elementwise``
say, so a slip there (a wrong fraction width, a whole ulp subtracted instead of half, a
widened relative term) would loosen every parity test at once.  Each pin takes a metrics
module and raises AssertionError when it disagrees with:
  * the spacing of the output formats, read off Python's own IEEE codecs (``struct``
    'e' for binary16, 'f' for binary32 and bfloat16 as its top half) and
    ``numpy.spacing`` for binary32;
  * correctly rounded results from those codecs (a correctly rounded output has no
    error in excess of half an ulp, so its err_q is exactly 0);
  * results built by hand whose excess over the bound is known exactly in binary.
The same pins run against the real module (tests/test_metric_pins.py) and against
copies of it with planted mistakes (tests/test_metric_mutations.py), each of which
must fail at least one pin.
"""

from __future__ import annotations

import math
import struct

import numpy as np

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def _f16_values(bits):
    return np.array([struct.unpack("<e", struct.pack("<H", int(b)))[0] for b in bits])


def _bf16_values(bits):
    return np.array([struct.unpack("<f", struct.pack("<I", int(b) << 16))[0] for b in bits])


def _positive_finite(dtype):
    """Sorted positive finite values of a 16-bit format (zero included), from struct."""
    vals = _f16_values(ALL16[:0x8000]) if dtype == "f16" else _bf16_values(ALL16[:0x8000])
    vals = vals[np.isfinite(vals)]
    return np.sort(vals)


def _round_f16(x):
    """Round doubles to binary16, nearest-even, through Python's IEEE half packer."""
    return np.array([struct.unpack("<e", struct.pack("<e", float(v)))[0] for v in x])


def _round_bf16(x, vals):
    """Round doubles to bfloat16 by brute force over the sorted positive values, ties to
    the even pattern (the pattern's parity is its index's parity among the positives)."""
    out = []
    for v in x:
        a = abs(float(v))
        i = int(np.searchsorted(vals, a))
        if i >= len(vals):
            r = math.inf
        elif vals[i] == a or i == 0:
            r = vals[i]
        else:
            lo, hi = vals[i - 1], vals[i]
            if a - lo < hi - a:
                r = lo
            elif a - lo > hi - a:
                r = hi
            else:
                r = lo if (i - 1) % 2 == 0 else hi
        out.append(math.copysign(r, v))
    return np.array(out)


# ---------------------------------------------------------------------------
# ulp()
# ---------------------------------------------------------------------------

def pin_ulp_spacing_16bit(m):
    """For every positive finite fp16 and bf16 value v below the largest one, ulp(v) is the
    gap to the next value, and so is ulp of any x in [v, next) and of -x; subnormal and
    zero arguments give the subnormal spacing (2^-24 for fp16, 2^-133 for bf16)."""
    r = np.random.Generator(np.random.PCG64(31))
    for dtype, sub in (("f16", 2.0 ** -24), ("bf16", 2.0 ** -133)):
        vals = _positive_finite(dtype)
        gaps = np.diff(vals)
        lo = vals[:-1]
        got = m.ulp(lo, dtype)
        # the gap above v is the binade's spacing except where v is the last value of its
        # binade (the next one starts a new binade with twice the spacing): there the gap
        # equals the spacing too, since next = v + spacing(v) = 2^(e+1)
        assert np.array_equal(got, gaps), dtype
        assert np.array_equal(m.ulp(-lo, dtype), gaps), dtype
        inside = lo + r.random(lo.size) * gaps
        inside = np.minimum(inside, np.nextafter(vals[1:], 0))
        assert np.array_equal(m.ulp(inside, dtype), gaps), dtype
        # the largest double below each next value (binade tops included) is still in [v, next)
        top = np.nextafter(vals[1:], 0)
        assert np.array_equal(m.ulp(top, dtype), gaps), dtype
        assert float(m.ulp(np.array([0.0]), dtype)[0]) == sub, dtype
        assert float(m.ulp(np.array([sub * 0.5]), dtype)[0]) == sub, dtype


def pin_ulp_spacing_f32(m):
    """binary32: ulp(x) equals numpy.spacing of x rounded down to binary32, across normal
    binades, at powers of two, and in the subnormal range (2^-149)."""
    r = np.random.Generator(np.random.PCG64(32))
    x = r.uniform(1.0, 2.0, 4000) * np.exp2(r.integers(-125, 127, 4000))
    x32 = x.astype(np.float32)
    # the float32 value at or below x has the same binade as x unless x rounded up to a
    # power of two; use the values themselves so the binade is unambiguous
    xs = x32.astype(np.float64)
    assert np.array_equal(m.ulp(xs, "f32"), np.spacing(x32).astype(np.float64))
    p2 = np.exp2(np.arange(-126, 127, dtype=np.float64))
    assert np.array_equal(m.ulp(p2, "f32"), np.spacing(p2.astype(np.float32)).astype(np.float64))
    tiny = np.array([2.0 ** -140, 2.0 ** -149, 0.0])
    assert np.all(m.ulp(tiny, "f32") == 2.0 ** -149)


def pin_scale(m):
    """s = sqrt(K) max|A| max|B|; K = 0 is treated as 1 (empty sums have no error)."""
    assert m.scale(8192, 1.0, 1.0) == math.sqrt(8192.0)
    assert m.scale(4096, 2.0, 0.5) == 64.0
    assert m.scale(1000, 2.0, 4.0) == math.sqrt(1000.0) * 8.0
    assert m.scale(0, 2.0, 3.0) == 6.0


# ---------------------------------------------------------------------------
# compare()
# ---------------------------------------------------------------------------

def _refs(dtype, n, seed):
    """Unrounded values spread over many binades of the format (like a GEMM's C_ref)."""
    r = np.random.Generator(np.random.PCG64(seed))
    hi = 15 if dtype == "f16" else 40
    lo = -20 if dtype == "f16" else -40
    return r.choice([-1.0, 1.0], n) * r.uniform(1.0, 2.0, n) * np.exp2(r.integers(lo, hi, n))


def pin_compare_correctly_rounded(m):
    """A correctly rounded output (Python's codecs) has err_q = 0 exactly, err_lit equal
    to its own largest rounding error, and floor equal to err_lit; a 16-bit one passes."""
    bvals = _positive_finite("bf16")
    for dtype in ("f16", "bf16", "f32"):
        ref = _refs(dtype, 3000, 41)
        if dtype == "f16":
            got = _round_f16(ref)
        elif dtype == "bf16":
            got = _round_bf16(ref, bvals)
        else:
            got = ref.astype(np.float32).astype(np.float64)
        s = 3.0
        res = m.compare(got, ref, dtype, s)
        worst = float(np.max(np.abs(got - ref))) / s
        assert res["err_q"] == 0.0, (dtype, res)
        assert res["err_lit"] == worst, (dtype, res, worst)
        assert res["floor"] == worst, (dtype, res, worst)
        assert res["nonfinite"] == 0, (dtype, res)
        # 16-bit outputs are gated on err_q; fp32 outputs on err_lit, which these large
        # values exceed
        assert res["ok"] is (dtype != "f32"), (dtype, res)


def pin_compare_one_ulp_off(m):
    """An output one ulp away from an exactly representable reference value v has excess
    half an ulp of v: err_q = ulp(v) / (2 s) exactly, with ulp(v) read off the codecs;
    the rest of the output is exact."""
    for dtype in ("f16", "bf16"):
        vals = _positive_finite(dtype)
        # interior values of a few binades (the neighbours share v's spacing), and the top
        # value of the binade below 2, whose upper neighbour 2.0 has twice its spacing: the
        # allowance is half an ulp of the reference, not of the output
        top = float(vals[int(np.searchsorted(vals, 2.0)) - 1])
        for v in (1.5, 96.0, 0.1875, 384.0, top):
            i = int(np.searchsorted(vals, v))
            assert vals[i] == v
            gap = float(vals[i + 1]) - v if v != top else 2.0 - top
            for nb in (float(vals[i + 1]), float(vals[i - 1])):
                ref = np.array([v, 1.0, -2.0, 0.5])
                got = ref.copy()
                got[0] = nb
                s = 2.0
                res = m.compare(got, ref, dtype, s)
                d = abs(nb - v)
                assert res["err_q"] == (d - gap / 2.0) / s, (dtype, v, nb, res)
                assert res["err_lit"] == d / s, (dtype, v, nb, res)
                assert res["floor"] == 0.0, (dtype, v, res)


def pin_compare_gate(m):
    """16-bit outputs are gated on err_q <= 4e-3, fp32 outputs on err_lit <= 1e-4 (the
    bounds the parity tests use); a non-finite output fails whatever its error."""
    assert m.TOL == {"f16": 4e-3, "bf16": 4e-3, "f32": 1e-4}
    # fp32: err_lit exactly at the bound passes, the next double above fails, and an error
    # inside half an fp32 ulp of 2^20 but above 1e-4 fails (err_q does not gate fp32)
    ref = np.array([0.0, 2.0 ** 20])
    assert m.compare(np.array([1e-4, 2.0 ** 20]), ref, "f32", 1.0)["ok"]
    assert not m.compare(np.array([np.nextafter(1e-4, 1.0), 2.0 ** 20]), ref, "f32", 1.0)["ok"]
    res = m.compare(np.array([0.0, 2.0 ** 20 + 0.01]), ref, "f32", 1.0)
    assert res["err_q"] == 0.0 and not res["ok"], res
    # 16-bit: references whose half ulp (2^-7) exceeds the bound, so err_lit is above 4e-3
    # whatever the excess; an excess of half the bound passes, one and a half fails
    for dtype, r0 in (("f16", 16.0), ("bf16", 2.0)):
        half = 2.0 ** -7
        ref = np.array([r0, 1.0])
        for frac, ok in ((0.5, True), (1.5, False)):
            got = np.array([r0 + half + frac * 4e-3, 1.0])
            res = m.compare(got, ref, dtype, 1.0)
            assert res["ok"] is ok, (dtype, frac, res)
            assert abs(res["err_q"] - frac * 4e-3) <= 1e-12, (dtype, res)
            assert res["err_lit"] > 4e-3, (dtype, res)
    ref = np.array([1.0, 2.0, 4.0])
    bad = np.array([1.0, np.nan, 4.0])
    res = m.compare(bad, ref, "f32", 1.0)
    assert res["nonfinite"] == 1 and not res["ok"]
    res = m.compare(np.array([1.0, np.inf, 4.0]), ref, "bf16", 1.0)
    assert res["nonfinite"] == 1 and not res["ok"]
    # an empty result passes; a shape mismatch raises
    assert m.compare(np.zeros((0, 3)), np.zeros((0, 3)), "bf16", 1.0)["ok"]
    try:
        m.compare(np.zeros((2, 3)), np.zeros((3, 2)), "f32", 1.0)
    except ValueError:
        pass
    else:
        raise AssertionError("shape mismatch not reported")


# ---------------------------------------------------------------------------
# compare_elementwise()
# ---------------------------------------------------------------------------

def pin_elementwise_bound(m):
    """The standalone GELU's bound |y - g| <= ulp(g)/2 + 2^-16 |g| + 2^-120: results built
    in binary at g = 1 (ulp 2^-10 fp16, 2^-7 bf16) and g = -3 (ulp 2^-9 / 2^-6) sit
    exactly on it (pass) or a little outside (fail: 2^-40 beyond it, twice the relative
    term, a whole ulp)."""
    assert m.EW_REL == 2.0 ** -16 and m.EW_ABS == 2.0 ** -120
    for dtype, p in (("f16", 10), ("bf16", 7)):
        for g0, e in ((1.0, 0), (-3.0, 1)):
            sgn = math.copysign(1.0, g0)
            half = 2.0 ** (e - p - 1)
            rel = 2.0 ** -16 * abs(g0)
            g = np.array([g0])
            # at the bound: 2^-120 is below the spacing of doubles near the bound, so the
            # excess is exactly 0
            inside = np.array([g0 + sgn * (half + rel)])
            res = m.compare_elementwise(inside, g, dtype)
            assert res["ok"] and res["excess"] == 0.0, (dtype, g0, res)
            for y in (g0 + sgn * (half + rel + 2.0 ** -40),
                      g0 + sgn * (half + 2 * rel),
                      g0 + sgn * 2 * half):
                res = m.compare_elementwise(np.array([y]), g, dtype)
                assert not res["ok"] and res["excess"] > 0, (dtype, g0, y, res)
    # the far negative tail: an exact (sub)normal below 2^-120 against a 0 result passes
    # only through the absolute term
    g = np.array([-(2.0 ** -121)])
    assert m.compare_elementwise(np.array([0.0]), g, "f32")["ok"]
    assert not m.compare_elementwise(np.array([0.0]), np.array([-(2.0 ** -100)]), "f32")["ok"]


def pin_elementwise_specials(m):
    """NaN must meet NaN, +inf must meet +inf, and the exact fraction counts results equal
    to the correctly rounded value."""
    g = np.array([np.nan, np.inf, 1.0, 2.0])
    assert m.compare_elementwise(np.array([np.nan, np.inf, 1.0, 2.0]), g, "bf16")["ok"]
    assert not m.compare_elementwise(np.array([0.0, np.inf, 1.0, 2.0]), g, "bf16")["ok"]
    assert not m.compare_elementwise(np.array([np.nan, 65504.0, 1.0, 2.0]), g, "f16")["ok"]
    assert not m.compare_elementwise(np.array([np.nan, np.inf, np.nan, 2.0]), g, "bf16")["ok"]
    res = m.compare_elementwise(np.array([1.0, 2.0 + 2.0 ** -6, 4.0, 8.0]),
                                np.array([1.0, 2.0, 4.0, 8.0]), "bf16")
    assert res["exact_frac"] == 0.75


ALL_PINS = [
    pin_ulp_spacing_16bit,
    pin_ulp_spacing_f32,
    pin_scale,
    pin_compare_correctly_rounded,
    pin_compare_one_ulp_off,
    pin_compare_gate,
    pin_elementwise_bound,
    pin_elementwise_specials,
]
