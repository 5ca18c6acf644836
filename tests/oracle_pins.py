"""Pins for the CPU oracle: checks against facts that do not come from the oracle.

Each pin takes an ``oracle.Oracle`` instance and raises AssertionError when the
oracle disagrees with the closed form, the independent codec, the exact
rational sum or the page's printed value it is compared with.  The same pins
run against the real oracle (tests/test_oracle_pins.py) and against copies of
it with planted mistakes (tests/test_oracle_mutations.py), which must fail at
least one pin.
"""

from __future__ import annotations

import decimal
import math
import os
import struct
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def _rng(seed=0):
    return np.random.Generator(np.random.PCG64(seed))


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------------------
# codecs
# ---------------------------------------------------------------------------

def pin_f16_decode_exhaustive(o):
    """All 65,536 binary16 patterns against Python's IEEE half codec (struct 'e')."""
    got = o.decode(ALL16, "f16")
    ref = np.array([struct.unpack("<e", struct.pack("<H", int(b)))[0] for b in ALL16])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert math.copysign(1.0, got[0x8000]) == -1.0


def pin_bf16_decode_exhaustive(o):
    """All 65,536 bfloat16 patterns: bf16 is the top half of an IEEE binary32."""
    got = o.decode(ALL16, "bf16")
    ref = np.array([struct.unpack("<f", struct.pack("<I", int(b) << 16))[0] for b in ALL16])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def _finite_sorted(o, dtype):
    vals = o.decode(ALL16, dtype)
    pos = vals[(ALL16 < 0x8000) & np.isfinite(vals)]
    bits = ALL16[(ALL16 < 0x8000) & np.isfinite(vals)]
    order = np.argsort(pos, kind="stable")
    return pos[order], bits[order]


def pin_f16_encode(o):
    """Round trip of every finite half, ties-to-even at every midpoint, overflow."""
    vals, bits = _finite_sorted(o, "f16")
    assert np.array_equal(o.encode(vals, "f16"), bits)
    assert np.array_equal(o.encode(-vals, "f16"), bits | 0x8000)
    mids = (vals[:-1] + vals[1:]) / 2.0  # exact in double
    got = o.encode(mids, "f16")
    ref = np.array([struct.unpack("<H", struct.pack("<e", float(m)))[0] for m in mids])
    assert np.array_equal(got, ref)
    # a hair off each midpoint goes to the nearer neighbour
    above = np.nextafter(mids, np.inf)
    below = np.nextafter(mids, -np.inf)
    assert np.array_equal(o.encode(above, "f16"), bits[1:])
    assert np.array_equal(o.encode(below, "f16"), bits[:-1])
    # overflow: 65504 is the largest half; its half-ulp above (65520) rounds to inf
    assert int(o.encode(np.array([65519.99]), "f16")[0]) == 0x7BFF
    assert int(o.encode(np.array([65520.0]), "f16")[0]) == 0x7C00
    assert int(o.encode(np.array([-1e9]), "f16")[0]) == 0xFC00
    # random doubles against struct's correctly rounded pack
    x = _rng(1).uniform(-60000, 60000, 2000) * np.exp2(_rng(2).integers(-30, 1, 2000))
    ref = np.array([struct.unpack("<H", struct.pack("<e", float(v)))[0] for v in x])
    assert np.array_equal(o.encode(x, "f16"), ref)


def _nearest_even_ref(x, vals, bits):
    """Brute-force nearest of the sorted finite positive values, ties to the even pattern."""
    out = []
    for v in x:
        a = abs(v)
        i = int(np.searchsorted(vals, a))
        if i == 0:
            r = bits[0]
        elif i >= len(vals):
            r = None
        else:
            lo, hi = vals[i - 1], vals[i]
            if a == hi:
                r = bits[i]
            elif a - lo < hi - a:
                r = bits[i - 1]
            elif a - lo > hi - a:
                r = bits[i]
            else:
                r = bits[i - 1] if bits[i - 1] % 2 == 0 else bits[i]
        out.append(int(r) | (0x8000 if v < 0 else 0))
    return np.array(out, dtype=np.uint16)


def pin_bf16_encode(o):
    """Round trip, midpoints to even, brute-force nearest on random doubles, overflow."""
    vals, bits = _finite_sorted(o, "bf16")
    assert np.array_equal(o.encode(vals, "bf16"), bits)
    mids = (vals[:-1] + vals[1:]) / 2.0
    got = o.encode(mids, "bf16")
    even = np.where(bits[:-1] % 2 == 0, bits[:-1], bits[1:])
    assert np.array_equal(got, even)
    assert np.array_equal(o.encode(np.nextafter(mids, np.inf), "bf16"), bits[1:])
    assert np.array_equal(o.encode(np.nextafter(mids, -np.inf), "bf16"), bits[:-1])
    r = _rng(3)
    x = r.standard_normal(3000) * np.exp2(r.integers(-140, 120, 3000))
    assert np.array_equal(o.encode(x, "bf16"), _nearest_even_ref(x, vals, bits))
    # largest finite bf16 is (2 - 2^-7) * 2^127; anything at or above its half-ulp above is inf
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127
    assert int(o.encode(np.array([big]), "bf16")[0]) == 0x7F7F
    assert int(o.encode(np.array([big + 2.0 ** 119]), "bf16")[0]) == 0x7F80


def pin_f32_encode(o):
    """double -> binary32 against numpy's correctly rounded cast."""
    r = _rng(4)
    x = r.standard_normal(20000) * np.exp2(r.integers(-160, 120, 20000))
    got = o.encode(x, "f32")
    ref = x.astype(np.float32).view(np.uint32)
    assert np.array_equal(got, ref)


def pin_xla_bf16_constants(o):
    """The XLA:GPU emitters page prints its GELU constants after rounding to bf16."""
    for inp, printed, exact in _golden_rows("xla_gelu_bf16_constants.txt"):
        v = float(o.round_to(np.array([float(inp)]), "bf16")[0])
        assert v == float(exact), (inp, v, exact)
        # the page prints the bf16 value to 6 significant digits; the printed number
        # lies within that precision of v and itself rounds to the same bf16 value
        p = float(printed)
        assert abs(v - p) <= 5e-6 * abs(v), (inp, v, printed)
        assert float(o.round_to(np.array([p]), "bf16")[0]) == v


# ---------------------------------------------------------------------------
# GELU
# ---------------------------------------------------------------------------

def pin_gelu(o):
    """gelu(0)=0, odd-part identity, limits, and distance to the exact (erf) GELU."""
    x = np.linspace(-12, 12, 4801)
    g = o.gelu(x)
    assert o.gelu(np.array([0.0]))[0] == 0.0
    # 0.5x(1+t(x)) - 0.5(-x)(1+t(-x)) = x because tanh is odd
    gm = o.gelu(-x)
    assert np.max(np.abs((g - gm) - x)) <= 1e-14 * 12
    # gelu(x) -> x for x >> 0 and -> 0 for x << 0
    assert np.all(np.abs(o.gelu(np.array([10.0, 20.0, 40.0])) - [10.0, 20.0, 40.0]) < 1e-12)
    assert np.all(np.abs(o.gelu(np.array([-10.0, -20.0, -40.0]))) < 1e-12)
    # the tanh form approximates x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)); its largest
    # deviation is 4.73e-4 (near |x| = 2.2), so a wrong constant or a dropped term that
    # moves it further than 5e-4 fails here
    exact = np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in x])
    dev = np.max(np.abs(g - exact))
    assert 4.5e-4 < dev < 5e-4, dev
    # the constant is sqrt(2/pi) to 10 digits (the Triton notes' comment, golden file)
    consts = {k: float(v) for k, v in _golden_rows("gelu_formula.txt")}
    assert abs(consts["sqrt_2_over_pi"] - math.sqrt(2.0 / math.pi)) < 1e-15
    # gelu is increasing above its minimum near x = -0.75 and its minimum is about -0.17
    assert -0.18 < g.min() < -0.16
    # the literal form 0.5 x (1 + tanh u) with Python's tanh, where it is well
    # conditioned (1 + tanh u >= 2e-3)
    for v in np.linspace(-3.0, 12.0, 301):
        u = 0.7978845608 * (v + 0.044715 * v ** 3)
        assert abs(o.gelu(np.array([v]))[0] - 0.5 * v * (1.0 + math.tanh(u))) <= 1e-14
    # the negative tail, where 1 + tanh u cancels in double: the literal definition in
    # 120-digit decimal arithmetic (1 + tanh u ~ 1e-50 at x = -13), tanh from its
    # exponential definition
    with decimal.localcontext() as ctx:
        ctx.prec = 120
        for v in (-4.0, -5.5, -6.9375, -7.0625, -8.0, -9.5, -11.0, -13.0):
            d = decimal.Decimal(v)
            u = decimal.Decimal("0.7978845608") * (d + decimal.Decimal("0.044715") * d ** 3)
            e2 = (2 * u).exp()
            ref = decimal.Decimal("0.5") * d * (1 + (e2 - 1) / (e2 + 1))
            got = o.gelu(np.array([v]))[0]
            # the rounding of u in double moves exp(-2u) by ~2|u| 2^-53 relatively
            rel = decimal.Decimal(1e-15) * (1 + abs(u))
            assert abs(decimal.Decimal(got) - ref) <= abs(ref) * rel, (v, got, ref)


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------

def _enc(o, x, dtype):
    return o.encode(np.asarray(x, dtype=np.float64), dtype)


def _store_b(b_kn_bits, layout):
    """Put a logical [K,N] pattern matrix into the stored layout."""
    return np.ascontiguousarray(b_kn_bits if layout == "kn" else b_kn_bits.T)


def pin_identity(o):
    """A = I gives C = B_e exactly; B_e = I gives C = A exactly (both dtypes, both layouts)."""
    r = _rng(5)
    for dtype in ("f16", "bf16"):
        for layout in ("kn", "nk"):
            K, N = 24, 13
            eye = _enc(o, np.eye(K), dtype)
            Bv = r.uniform(-3, 3, (K, N))
            Bb = _enc(o, Bv, dtype)
            C = o.gemm(eye, _store_b(Bb, layout), K, N, K, dtype, layout)
            assert np.array_equal(C, o.decode(Bb, dtype))
            M = 11
            Ab = _enc(o, r.uniform(-3, 3, (M, K)), dtype)
            C = o.gemm(Ab, _store_b(_enc(o, np.eye(K), dtype), layout), M, K, K, dtype, layout)
            assert np.array_equal(C, o.decode(Ab, dtype))


def pin_all_ones(o):
    """All-ones A and B: every C[i,j] is exactly K."""
    for K in (1, 7, 64, 1000):
        for layout in ("kn", "nk"):
            A = _enc(o, np.ones((5, K)), "f16")
            B = _enc(o, np.ones((K, 6)), "f16")
            C = o.gemm(A, _store_b(B, layout), 5, 6, K, "f16", layout)
            assert np.all(C == K)


def pin_rank1(o):
    """A[i,k] = u_i, B[k,j] = v_j gives C = K u_i v_j exactly (products exact in double)."""
    r = _rng(6)
    for dtype in ("f16", "bf16"):
        M, N, K = 9, 7, 96
        u = o.decode(_enc(o, r.uniform(-2, 2, M), dtype), dtype)
        v = o.decode(_enc(o, r.uniform(-2, 2, N), dtype), dtype)
        A = _enc(o, np.repeat(u[:, None], K, axis=1), dtype)
        Bkn = _enc(o, np.repeat(v[None, :], K, axis=0), dtype)
        for layout in ("kn", "nk"):
            C = o.gemm(A, _store_b(Bkn, layout), M, N, K, dtype, layout)
            assert np.array_equal(C, K * np.outer(u, v))


def pin_brute_force(o):
    """Tiny shapes against the exact rational sum (fractions), within gamma_K sum|a||b|."""
    r = _rng(7)
    u = 2.0 ** -53
    for (M, N, K) in ((1, 1, 1), (2, 3, 4), (7, 5, 9), (3, 7, 2), (5, 1, 8)):
        for dtype in ("f16", "bf16"):
            for layout in ("kn", "nk"):
                vals = r.uniform(-4, 4, (M, K)) * np.exp2(r.integers(-12, 4, (M, K)))
                Ab = _enc(o, vals, dtype)
                Bkn = _enc(o, r.uniform(-4, 4, (K, N)) * np.exp2(r.integers(-12, 4, (K, N))),
                           dtype)
                Ad, Bd = o.decode(Ab, dtype), o.decode(Bkn, dtype)
                C = o.gemm(Ab, _store_b(Bkn, layout), M, N, K, dtype, layout)
                gam = K * u / (1 - K * u)
                for i in range(M):
                    for j in range(N):
                        exact = sum(Fraction(Ad[i, k]) * Fraction(Bd[k, j]) for k in range(K))
                        mag = sum(abs(Ad[i, k] * Bd[k, j]) for k in range(K))
                        assert abs(Fraction(C[i, j]) - exact) <= Fraction(gam * mag) + 0, \
                            (M, N, K, dtype, layout, i, j)


def pin_layout_equivalence(o):
    """NN on B equals TN on the transposed storage of the same B, bitwise."""
    r = _rng(8)
    M, N, K = 17, 23, 31
    Ab = _enc(o, r.uniform(-1, 1, (M, K)), "bf16")
    Bkn = _enc(o, r.uniform(-1, 1, (K, N)), "bf16")
    C1 = o.gemm(Ab, Bkn, M, N, K, "bf16", "kn")
    C2 = o.gemm(Ab, np.ascontiguousarray(Bkn.T), M, N, K, "bf16", "nk")
    assert np.array_equal(C1, C2)
    # and it is not symmetric in a wrong way: swapping the roles of A and B changes C
    C3 = o.gemm(np.ascontiguousarray(Bkn.T), np.ascontiguousarray(Ab.T), N, M, K, "bf16", "kn")
    assert np.array_equal(C3, C1.T)


def pin_zero_padding(o):
    """Out-of-range elements contribute exactly zero: the leading block of the zero-padded
    problem equals the unpadded result, bitwise (the Triton matmul loads masked tails as 0)."""
    r = _rng(9)
    M, N, K = 13, 11, 21
    Mp, Np, Kp = 16, 16, 32
    Av = np.zeros((Mp, Kp))
    Av[:M, :K] = r.uniform(-1, 1, (M, K))
    Bv = np.zeros((Kp, Np))
    Bv[:K, :N] = r.uniform(-1, 1, (K, N))
    Ab, Bb = _enc(o, Av, "f16"), _enc(o, Bv, "f16")
    for layout in ("kn", "nk"):
        Cp = o.gemm(Ab, _store_b(Bb, layout), Mp, Np, Kp, "f16", layout)
        C = o.gemm(np.ascontiguousarray(Ab[:M, :K]), _store_b(np.ascontiguousarray(Bb[:K, :N]),
                   layout), M, N, K, "f16", layout)
        assert np.array_equal(Cp[:M, :N], C)
        assert np.all(Cp[M:, :] == 0) and np.all(Cp[:, N:] == 0)


def pin_rows_and_epilogue(o):
    """Row subsets equal the full result; the GELU epilogue is gelu() of the plain result."""
    r = _rng(10)
    M, N, K = 12, 9, 40
    Ab = _enc(o, r.normal(0, 1, (M, K)), "bf16")
    Bb = _enc(o, r.normal(0, 1, (N, K)), "bf16")
    C = o.gemm(Ab, Bb, M, N, K, "bf16", "nk")
    sub = o.gemm(Ab, Bb, M, N, K, "bf16", "nk", rows=[11, 0, 5])
    assert np.array_equal(sub, C[[11, 0, 5]])
    G = o.gemm(Ab, Bb, M, N, K, "bf16", "nk", epilogue="gelu_tanh")
    assert np.array_equal(G, o.gelu(C))
    # K = 0: the empty sum is 0 and gelu(0) = 0
    Z = o.gemm(np.zeros((3, 0), np.uint16), np.zeros((0, 4), np.uint16), 3, 4, 0, "f16", "kn",
               epilogue="gelu_tanh")
    assert np.all(Z == 0)


def pin_relu(o):
    """ReLU epilogue (the Triton lecture notes' matmul kernel, maximum(acc, 0)): with A = I
    it is max(b, 0) of every element of B exactly; relu(c) - relu(-c) = c, so the ReLU
    results for A and -A differ by exactly the plain result; relu of the empty sum is 0."""
    r = _rng(12)
    K, N = 16, 21
    Bv = r.uniform(-3, 3, (K, N))
    Bv[0, :5] = 0.0
    for dtype in ("f16", "bf16"):
        Bb = _enc(o, Bv, dtype)
        eye = _enc(o, np.eye(K), dtype)
        for layout in ("kn", "nk"):
            C = o.gemm(eye, _store_b(Bb, layout), K, N, K, dtype, layout, epilogue="relu")
            Bd = o.decode(Bb, dtype)
            assert np.array_equal(C, np.where(Bd > 0, Bd, 0.0))
            assert np.any(C == 0) and np.any(C > 0)
    M, N, K = 10, 13, 37
    Av = r.normal(0, 1, (M, K))
    Ab, Anb = _enc(o, Av, "bf16"), _enc(o, -Av, "bf16")
    Bb = _enc(o, r.normal(0, 1, (K, N)), "bf16")
    plain = o.gemm(Ab, Bb, M, N, K, "bf16", "kn")
    pos = o.gemm(Ab, Bb, M, N, K, "bf16", "kn", epilogue="relu")
    neg = o.gemm(Anb, Bb, M, N, K, "bf16", "kn", epilogue="relu")
    assert np.array_equal(pos - neg, plain)
    assert np.all(pos >= 0) and np.any(plain < 0)
    Z = o.gemm(np.zeros((2, 0), np.uint16), np.zeros((0, 3), np.uint16), 2, 3, 0, "f16", "kn",
               epilogue="relu")
    assert np.all(Z == 0)


def pin_gelu_elementwise(o):
    """The standalone GELU on stored elements: 0 -> 0; for bf16 x >= 8 the exact result
    rounds back to x itself (gelu(x) = x sigmoid(2u) with 1 - sigmoid(2u) < 2^-40), for
    x <= -12 to -0 (|gelu(x)| < 2^-400); the fp32 path decodes binary32 exactly."""
    for dtype in ("f16", "bf16"):
        vals = np.array([0.0, 8.0, 9.5, 100.0, 1000.0, -12.0, -20.0, -1000.0])
        bits = _enc(o, vals, dtype)
        g = o.gelu_elementwise(bits, dtype)
        out = o.encode(g, dtype)
        assert out[0] == 0
        assert np.array_equal(out[1:5], bits[1:5])
        assert np.all(out[5:] == 0x8000)
    x32 = np.array([0.5, -0.5, 3.0], dtype=np.float32)
    g = o.gelu_elementwise(x32.view(np.uint32), "f32")
    assert np.array_equal(g, o.gelu(x32.astype(np.float64)))


def pin_small_exact_integers(o):
    """Integer-valued inputs: C equals numpy's integer matmul exactly (no rounding anywhere)."""
    r = _rng(11)
    M, N, K = 19, 14, 57
    Ai = r.integers(-8, 9, (M, K))
    Bi = r.integers(-8, 9, (K, N))
    for dtype in ("f16", "bf16"):
        Ab, Bb = _enc(o, Ai, dtype), _enc(o, Bi, dtype)
        for layout in ("kn", "nk"):
            C = o.gemm(Ab, _store_b(Bb, layout), M, N, K, dtype, layout)
            assert np.array_equal(C, (Ai @ Bi).astype(np.float64))


ALL_PINS = [
    pin_f16_decode_exhaustive,
    pin_bf16_decode_exhaustive,
    pin_f16_encode,
    pin_bf16_encode,
    pin_f32_encode,
    pin_xla_bf16_constants,
    pin_gelu,
    pin_identity,
    pin_all_ones,
    pin_rank1,
    pin_brute_force,
    pin_layout_equivalence,
    pin_zero_padding,
    pin_rows_and_epilogue,
    pin_relu,
    pin_gelu_elementwise,
    pin_small_exact_integers,
]
