"""Seeded synthetic inputs for the tiled GEMM C[M,N] = A[M,K] @ B.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It only *draws* inputs; it contains none of the GEMM's arithmetic
(no decoding, no products, no sums).  Matrices are returned as raw 16-bit
patterns (``numpy.uint16``) so that both sides decode the very same bits.

Recipe (the pages fix no RNG):
  * ``numpy.random.Generator(PCG64(seed))`` draws float64 values, which are
    rounded float64 -> float32 (numpy, round-to-nearest-even) -> fp16/bf16
    (round-to-nearest-even).
  * A uses seed 42 and B seed 43, echoing the Pallas pipelining guide's
    Hopper matmul example, which draws both operands from ``key(42)``.
  * B is drawn directly in its stored shape: ``[K, N]`` for the "nn" layout,
    ``[N, K]`` for the "nk" (transpose_B) layout of the TileLang pipelined
    GEMM tutorial's ``matmul_auto``.
  * ``normal(0, s)`` means standard deviation ``s``.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Tuple

import numpy as np

SEED_A = 42
SEED_B = 43

F16 = "f16"
BF16 = "bf16"
F32 = "f32"
B_KN = "kn"  # B stored row-major [K, N]  ("NN")
B_NK = "nk"  # B stored row-major [N, K]  ("TN", transpose_B)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    in_dtype: str
    out_dtype: str
    b_layout: str
    epilogue: str  # "none" | "gelu_tanh" | "relu"
    dist: Tuple  # ("uniform", lo, hi) | ("normal", sigma) | ("unit",) == uniform [0, 1)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    def describe(self) -> str:
        lay = "B[K,N] (NN)" if self.b_layout == B_KN else "B[N,K] (transpose_B)"
        epi = {"none": "", "gelu_tanh": ", fused tanh-GELU", "relu": ", fused ReLU"}[self.epilogue]
        return (f"{self.in_dtype} GEMM M={self.M} N={self.N} K={self.K}, A[M,K], {lay}, "
                f"inputs {self.dist}, fp32 accumulate, {self.out_dtype} output{epi}")


# The five workloads of the benchmark table plus the Pallas guide's Hopper
# example shape (m = 132*128, n = 4*128, k = 10*64, uniform [0, 1) fp16) and a
# matmul + ReLU case after the Triton lecture notes.
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in (
        Workload("tn_f16_256", 256, 256, 256, F16, F16, B_NK, "none", ("uniform", -1.0, 1.0)),
        Workload("tn_f16_4096", 4096, 4096, 4096, F16, F16, B_NK, "none", ("normal", 1.0)),
        Workload("nn_bf16_8192", 8192, 8192, 8192, BF16, BF16, B_KN, "none", ("uniform", -1.0, 1.0)),
        Workload("tn_f16_3000x5000x1000_f32out", 3000, 5000, 1000, F16, F32, B_NK, "none",
                 ("uniform", -1.0, 1.0)),
        Workload("nn_bf16_3072x4096x4096_gelu", 3072, 4096, 4096, BF16, BF16, B_KN, "gelu_tanh",
                 ("normal", 0.02)),
        Workload("pallas_hopper_example", 132 * 128, 4 * 128, 10 * 64, F16, F16, B_KN, "none",
                 ("unit",)),
        # The Triton lecture notes' matmul + ReLU (B stored [K,N], fp32 output; the notes
        # give no size, this one spans 8 x 8 tiles of 256).
        Workload("nn_f16_2048x2048x1024_relu_f32out", 2048, 2048, 1024, F16, F32, B_KN, "relu",
                 ("uniform", -1.0, 1.0)),
        # The same 8192^3 problem in fp16 (the metric's wording names fp16).
        Workload("nn_f16_8192", 8192, 8192, 8192, F16, F16, B_KN, "none", ("uniform", -1.0, 1.0)),
        # ... and with B stored [N,K] (transpose_B, the other layout the pages use).
        Workload("tn_f16_8192", 8192, 8192, 8192, F16, F16, B_NK, "none", ("uniform", -1.0, 1.0)),
    )
}


def _draw(shape, dist, seed) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    kind = dist[0]
    if kind == "uniform":
        x = rng.uniform(dist[1], dist[2], size=shape)
    elif kind == "normal":
        x = rng.standard_normal(size=shape) * dist[1]
    elif kind == "unit":
        x = rng.random(size=shape)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return x.astype(np.float32)


def float32_to_bits(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to fp16/bf16 (nearest-even) and return the bit patterns."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == F16:
        return x32.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        u = x32.view(np.uint32).astype(np.uint64)
        # nearest-even on the 16 dropped bits (inputs are finite)
        u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return u.astype(np.uint16)
    raise ValueError(dtype)


def make_matrix(shape, dtype: str, dist, seed: int) -> np.ndarray:
    return float32_to_bits(_draw(shape, dist, seed), dtype)


def make_inputs(w: Workload, seed_a: int = SEED_A, seed_b: int = SEED_B):
    """Return (A_bits [M,K], B_bits [K,N] or [N,K]) as uint16 arrays."""
    a = make_matrix((w.M, w.K), w.in_dtype, w.dist, seed_a)
    b_shape = (w.K, w.N) if w.b_layout == B_KN else (w.N, w.K)
    b = make_matrix(b_shape, w.in_dtype, w.dist, seed_b)
    return a, b


def custom(M, N, K, in_dtype=F16, out_dtype=F16, b_layout=B_NK, epilogue="none",
           dist=("uniform", -1.0, 1.0), name=None) -> Workload:
    return Workload(name or f"custom_{M}x{N}x{K}", M, N, K, in_dtype, out_dtype, b_layout,
                    epilogue, dist)
