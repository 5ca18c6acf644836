"""CPU oracle for C[M,N] = epi(A[M,K] @ B) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  It shares nothing with the GPU path: its C
source (``oracle.c``) decodes fp16/bf16 patterns exactly, sums every output in
IEEE double with k ascending, applies the tanh-GELU in double and rounds to the
output format to nearest-even.  See ``oracle.c`` for the definition it follows
and the passages of the pages it cites.

Pins (all in ``tests/test_oracle_*.py``): exhaustive codec checks against
Python's ``struct`` IEEE codecs, identity / all-ones / rank-1 closed forms,
exact-rational brute force on tiny shapes, layout equivalence, zero-padding
invariance, GELU identities and its distance to the erf GELU, and the bf16
constants that the XLA:GPU emitters page prints (``tests/golden/``).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DTYPES = {"f16": 0, "bf16": 1, "f32": 2}
LAYOUTS = {"kn": 0, "nk": 1}
EPILOGUES = {"none": 0, "gelu_tanh": 1, "relu": 2}


def compile_source(src: str, out: str) -> str:
    """Compile an oracle C source file into a shared library (gcc, OpenMP, no FMA)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O3", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", src, "-o", tmp,
           "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so."""
    if not force and os.path.exists(_LIB):
        return _LIB
    return compile_source(_SRC, _LIB)


class Oracle:
    """ctypes view of one build of liboracle.so (the tests also load mutated copies)."""

    def __init__(self, path: str = _LIB):
        L = ctypes.CDLL(path)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        L.oracle_decode_array.restype = None
        L.oracle_decode_array.argtypes = [u16p, i64, ctypes.c_int, f64p]
        L.oracle_encode_array.restype = None
        L.oracle_encode_array.argtypes = [f64p, i64, ctypes.c_int, ctypes.c_void_p]
        L.oracle_gelu_array.restype = None
        L.oracle_gelu_array.argtypes = [f64p, i64, f64p]
        L.oracle_gemm_rows.restype = ctypes.c_int
        L.oracle_gemm_rows.argtypes = [u16p, u16p, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.POINTER(ctypes.c_int64), i64, f64p]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_num_threads.argtypes = []
        self.lib = L
        self.path = path

    def decode(self, bits: np.ndarray, dtype: str) -> np.ndarray:
        """Exact decode of fp16/bf16 bit patterns to float64."""
        b = _u16(bits)
        out = np.empty(b.shape, dtype=np.float64)
        self.lib.oracle_decode_array(b.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)), b.size,
                                     DTYPES[dtype],
                                     out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
        return out

    def encode(self, x: np.ndarray, dtype: str) -> np.ndarray:
        """Round float64 values to fp16/bf16/f32 (nearest-even); returns bit patterns."""
        xd = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(xd.shape, dtype=np.uint32 if dtype == "f32" else np.uint16)
        self.lib.oracle_encode_array(xd.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                     xd.size, DTYPES[dtype], out.ctypes.data_as(ctypes.c_void_p))
        return out

    def round_to(self, x: np.ndarray, dtype: str) -> np.ndarray:
        """Values of x after rounding to the output format, as float64."""
        bits = self.encode(x, dtype)
        if dtype == "f32":
            return bits.view(np.float32).astype(np.float64)
        return self.decode(bits, dtype)

    def gelu(self, x: np.ndarray) -> np.ndarray:
        xd = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty_like(xd)
        self.lib.oracle_gelu_array(xd.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), xd.size,
                                   out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
        return out

    def gelu_elementwise(self, x_bits: np.ndarray, dtype: str) -> np.ndarray:
        """The standalone GELU on stored elements: exact decode, gelu in double.
        x_bits are uint16 patterns (f16/bf16) or uint32 patterns (f32); returns the
        unrounded double results (self.encode gives the correctly rounded patterns)."""
        if dtype == "f32":
            x = np.ascontiguousarray(x_bits, dtype=np.uint32).view(np.float32).astype(np.float64)
        else:
            x = self.decode(np.ascontiguousarray(x_bits, dtype=np.uint16), dtype)
        return self.gelu(x)

    def gemm(self, A_bits: np.ndarray, B_bits: np.ndarray, M: int, N: int, K: int,
             in_dtype: str, b_layout: str, epilogue: str = "none",
             rows: Optional[Sequence[int]] = None) -> np.ndarray:
        """C = epi(A @ B_e) in float64 (all rows, or the listed rows in that order)."""
        A = _u16(A_bits)
        B = _u16(B_bits)
        if A.size != M * K:
            raise ValueError("A has the wrong size")
        if B.size != K * N:
            raise ValueError("B has the wrong size")
        if rows is None:
            nrows, rows_p, keep = M, None, None
        else:
            keep = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
            nrows = keep.size
            rows_p = keep.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        out = np.empty((nrows, N), dtype=np.float64)
        rc = self.lib.oracle_gemm_rows(A.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)),
                                       B.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)), M, N, K,
                                       DTYPES[in_dtype], LAYOUTS[b_layout], EPILOGUES[epilogue],
                                       rows_p, nrows,
                                       out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
        if rc != 0:
            raise RuntimeError(f"oracle_gemm_rows failed with code {rc}")
        return out

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())


def _u16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected uint16 bit patterns, got {a.dtype}")
    return a


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build()
        _default = Oracle(_LIB)
    return _default


def decode(bits, dtype):
    return default().decode(bits, dtype)


def encode(x, dtype):
    return default().encode(x, dtype)


def round_to(x, dtype):
    return default().round_to(x, dtype)


def gelu(x):
    return default().gelu(x)


def gelu_elementwise(x_bits, dtype):
    return default().gelu_elementwise(x_bits, dtype)


def gemm(A_bits, B_bits, M, N, K, in_dtype, b_layout, epilogue="none", rows=None):
    return default().gemm(A_bits, B_bits, M, N, K, in_dtype, b_layout, epilogue, rows)


def num_threads() -> int:
    return default().num_threads()
