"""Helpers for the GPU tests: move seeded inputs to the device, run the C ABI,
bring C back, and compare with the oracle (test infrastructure)."""

from __future__ import annotations

import numpy as np

import oracle
from oracle import metrics
import software_pipelined_tiled_gemm_amd as spg
import workloads as W


def torch_dev():
    import torch
    return torch.device("cuda:0")


def to_dev(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(torch_dev())


def alloc_c(w: W.Workload, fill=0):
    import torch
    if w.out_dtype == W.F32:
        return torch.full((w.M, w.N), float(fill), dtype=torch.float32, device=torch_dev())
    return torch.full((w.M, w.N), int(fill), dtype=torch.int16, device=torch_dev())


def c_values(C, w: W.Workload, rows=None) -> np.ndarray:
    """Device C -> float64 values (optionally only some rows)."""
    import torch
    t = C if rows is None else C[torch.as_tensor(np.asarray(rows), device=C.device)]
    h = t.cpu().numpy()
    if w.out_dtype == W.F32:
        return h.astype(np.float64)
    return oracle.decode(h.view(np.uint16), w.out_dtype)


def c_values_raw(raw: np.ndarray, w: W.Workload) -> np.ndarray:
    """Host copy of C (int16 bits or float32) -> float64 values."""
    if w.out_dtype == W.F32:
        return raw.astype(np.float64)
    return oracle.decode(raw.view(np.uint16), w.out_dtype)


def run(w: W.Workload, a_bits, b_bits, force=None, C=None, autotune=False):
    import torch
    A, B = to_dev(a_bits), to_dev(b_bits)
    if C is None:
        C = alloc_c(w)
    with spg.Gemm(w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.b_layout, w.epilogue, force) as g:
        if autotune:
            g.autotune(A, B, C, reps=3)
        g(A, B, C)
        cfg = g.config()
    torch.cuda.synchronize()
    return C, cfg


def scale_of(w: W.Workload, a_bits, b_bits) -> float:
    ma = float(np.abs(oracle.decode(a_bits, w.in_dtype)).max()) if a_bits.size else 0.0
    mb = float(np.abs(oracle.decode(b_bits, w.in_dtype)).max()) if b_bits.size else 0.0
    return metrics.scale(w.K, ma, mb)


def check(w: W.Workload, a_bits, b_bits, got: np.ndarray, rows=None) -> dict:
    ref = oracle.gemm(a_bits, b_bits, w.M, w.N, w.K, w.in_dtype, w.b_layout, w.epilogue, rows)
    r = metrics.compare(got, ref, w.out_dtype, scale_of(w, a_bits, b_bits))
    assert r["ok"], f"{w.describe()}: {r}"
    return r
