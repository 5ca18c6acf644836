"""Python binding of the MI355X software-pipelined tiled GEMM (C ABI in include/spgemm.h)
and of the standalone elementwise GELU (include/spgelu.h).

Argument marshalling only: every step of C = epi(A . B) runs in the HIP
kernels of ``libspgemm.so``.  PyTorch is used by callers for device memory and
streams; this module accepts torch tensors (device pointer + current stream are
taken from them) or raw integer device pointers.

If the shared library has not been built, importing works but every call raises
``GemmError`` -- there is no CPU fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspgemm.so")
# The poison library: the same C ABI built with -DSPG_POISON from a subset of the
# configurations, every released ring region overwritten with NaN (a race detector
# for the GPU tests; build.build_poison()).
POISON_LIB_PATH = os.path.join(_HERE, "libspgemm_poison.so")

GEMM_OK = 0
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "out of memory",
          4: "HIP runtime error", 5: "internal error"}
DTYPES = {"f16": 0, "bf16": 1, "f32": 2}
B_LAYOUTS = {"kn": 0, "nk": 1}
EPILOGUES = {"none": 0, "gelu_tanh": 1, "relu": 2}
STAGING = {0: "direct", 1: "vgpr", 2: "direct-spread", 3: "producer-wave", 4: "direct-a-deep",
           5: "direct-late-release", 6: "direct-b-deep", 7: "vgpr-any-alignment"}


class GemmError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)} (status {status})")
        self.status = status


class TileConfig(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32),
                ("block_k", ctypes.c_int32), ("stages", ctypes.c_int32),
                ("wave_m", ctypes.c_int32), ("wave_n", ctypes.c_int32),
                ("swizzle", ctypes.c_int32), ("group_m", ctypes.c_int32),
                ("xcd_remap", ctypes.c_int32), ("staging", ctypes.c_int32),
                ("lookahead", ctypes.c_int32), ("schedule", ctypes.c_int32),
                ("persistent", ctypes.c_int32), ("store", ctypes.c_int32),
                ("mfma", ctypes.c_int32)]

    def __init__(self, **kw):
        kw.setdefault("lookahead", 1)
        super().__init__(**kw)

    def as_dict(self):
        return {k: int(getattr(self, k)) for k, _ in self._fields_}

    @classmethod
    def from_dict(cls, d):
        c = cls()
        for k, _ in cls._fields_:
            setattr(c, k, int(d.get(k, 1 if k == "lookahead" else 0)))
        return c

    def __repr__(self):
        d = self.as_dict()
        return (f"TileConfig({d['block_m']}x{d['block_n']}x{d['block_k']}, S={d['stages']}, "
                f"wave {d['wave_m']}x{d['wave_n']}, swizzle={d['swizzle']}, "
                f"group_m={d['group_m']}, xcd_remap={d['xcd_remap']}, "
                f"staging={STAGING.get(d['staging'], d['staging'])}, lookahead={d['lookahead']}, "
                f"schedule={('manual', 'compiler', 'ping-pong')[d['schedule']] if 0 <= d['schedule'] <= 2 else d['schedule']}"
                f"{', persistent' if d['persistent'] else ''}{', direct store' if d['store'] else ''}"
                f"{', mfma 16x16x32' if d['mfma'] == 16 else ''})")


EXPORTED = ("gemm_create", "gemm_run", "gemm_destroy", "gemm_get_config", "gemm_launch_config",
            "gemm_autotune",
            "gemm_num_configs", "gemm_list_config", "gemm_lds_bytes", "gemm_status_string",
            "gemm_last_hip_error", "gemm_wait_timeouts", "gelu_run")

_lib = None
_poison_lib = None


def lib():
    """Load libspgemm.so (raises GemmError if it is missing: no fallback path exists)."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def poison_lib():
    """Load libspgemm_poison.so, the race-detecting test build of the same C ABI."""
    global _poison_lib
    if _poison_lib is None:
        _poison_lib = _load(POISON_LIB_PATH)
    return _poison_lib


def _load(path):
    if not os.path.exists(path):
        raise GemmError(5, f"HIP library {path} is not built (run __graft_entry__.build())")
    # PyTorch-ROCm ships its own libamdhip64 / libhsa-runtime64.  Load it first so this
    # library binds (by soname) to that same HIP runtime instead of a second copy from
    # /opt/rocm: two HIP runtimes in one process do not share devices.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.gemm_create.restype = ctypes.c_int
    L.gemm_create.argtypes = [ctypes.POINTER(vp), i64, i64, i64, ctypes.c_int, ctypes.c_int,
                              ctypes.c_int, ctypes.c_int, ctypes.POINTER(TileConfig)]
    L.gemm_run.restype = ctypes.c_int
    L.gemm_run.argtypes = [vp, vp, vp, vp, vp]
    L.gemm_destroy.restype = ctypes.c_int
    L.gemm_destroy.argtypes = [vp]
    L.gemm_get_config.restype = ctypes.c_int
    L.gemm_get_config.argtypes = [vp, ctypes.POINTER(TileConfig)]
    L.gemm_launch_config.restype = ctypes.c_int
    L.gemm_launch_config.argtypes = [vp, vp, vp, vp, ctypes.POINTER(TileConfig)]
    L.gemm_autotune.restype = ctypes.c_int
    L.gemm_autotune.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    L.gemm_num_configs.restype = i32
    L.gemm_num_configs.argtypes = []
    L.gemm_list_config.restype = ctypes.c_int
    L.gemm_list_config.argtypes = [i32, ctypes.POINTER(TileConfig)]
    L.gemm_lds_bytes.restype = i64
    L.gemm_lds_bytes.argtypes = [ctypes.POINTER(TileConfig)]
    L.gemm_status_string.restype = ctypes.c_char_p
    L.gemm_status_string.argtypes = [ctypes.c_int]
    L.gemm_last_hip_error.restype = ctypes.c_char_p
    L.gemm_last_hip_error.argtypes = []
    L.gemm_wait_timeouts.restype = ctypes.c_int
    L.gemm_wait_timeouts.argtypes = [ctypes.POINTER(ctypes.c_uint32), i32]
    L.gelu_run.restype = ctypes.c_int
    L.gelu_run.argtypes = [vp, vp, i64, ctypes.c_int, vp]
    return L


def _check(status: int, what: str):
    if status != GEMM_OK:
        if status == 4:
            what = f"{what} [{gemm_last_hip_error()}]"
        raise GemmError(status, what)


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())  # torch tensor


def _stream(stream, *tensors) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else int(stream.cuda_stream)
    for t in tensors:
        if t is not None and not isinstance(t, int) and getattr(t, "is_cuda", False):
            import torch
            return int(torch.cuda.current_stream(t.device).cuda_stream)
    return None


# ---- the C entry points, same names --------------------------------------------------

def gemm_create(M: int, N: int, K: int, in_dtype: str = "bf16", out_dtype: str = "bf16",
                b_layout: str = "kn", epilogue: str = "none",
                force: Optional[TileConfig] = None) -> int:
    h = ctypes.c_void_p()
    st = lib().gemm_create(ctypes.byref(h), M, N, K, DTYPES[in_dtype], DTYPES[out_dtype],
                           B_LAYOUTS[b_layout], EPILOGUES[epilogue],
                           ctypes.byref(force) if force is not None else None)
    _check(st, "gemm_create")
    return int(h.value)


def gemm_run(handle: int, A, B, C, stream=None) -> None:
    st = lib().gemm_run(handle, _ptr(A), _ptr(B), _ptr(C), _stream(stream, A, B, C))
    _check(st, "gemm_run")


def gemm_destroy(handle: Optional[int]) -> None:
    _check(lib().gemm_destroy(handle), "gemm_destroy")


def gemm_get_config(handle: int) -> TileConfig:
    c = TileConfig()
    _check(lib().gemm_get_config(handle, ctypes.byref(c)), "gemm_get_config")
    return c


def gemm_launch_config(handle: int, A, B, C) -> TileConfig:
    """The configuration gemm_run would launch with these operands (their alignment)."""
    c = TileConfig()
    _check(lib().gemm_launch_config(handle, _ptr(A), _ptr(B), _ptr(C), ctypes.byref(c)),
           "gemm_launch_config")
    return c


def gemm_autotune(handle: int, A, B, C, stream=None, reps: int = 10) -> float:
    us = ctypes.c_double()
    st = lib().gemm_autotune(handle, _ptr(A), _ptr(B), _ptr(C), _stream(stream, A, B, C), reps,
                             ctypes.byref(us))
    _check(st, "gemm_autotune")
    return float(us.value)


def gemm_num_configs() -> int:
    return int(lib().gemm_num_configs())


def gemm_list_config(index: int) -> TileConfig:
    c = TileConfig()
    _check(lib().gemm_list_config(index, ctypes.byref(c)), "gemm_list_config")
    return c


def gemm_lds_bytes(cfg: TileConfig) -> int:
    return int(lib().gemm_lds_bytes(ctypes.byref(cfg)))


def gemm_status_string(status: int) -> str:
    return lib().gemm_status_string(status).decode()


def gemm_last_hip_error() -> str:
    return lib().gemm_last_hip_error().decode()


def gemm_wait_timeouts(reset: bool = False) -> int:
    """Bounded waits of the wave-specialized ring that gave up on the current device
    (synchronizes the device; reset clears the count after reading it)."""
    n = ctypes.c_uint32()
    _check(lib().gemm_wait_timeouts(ctypes.byref(n), 1 if reset else 0), "gemm_wait_timeouts")
    return int(n.value)


def gelu_run(x, y, n: int, dtype: str = "bf16", stream=None) -> None:
    """y[i] = gelu(x[i]) for n contiguous elements of dtype (include/spgelu.h)."""
    st = lib().gelu_run(_ptr(x), _ptr(y), n, DTYPES[dtype], _stream(stream, x, y))
    _check(st, "gelu_run")


class Gemm:
    """RAII wrapper around one plan: ``with Gemm(M, N, K, ...) as g: g(A, B, C)``."""

    def __init__(self, M, N, K, in_dtype="bf16", out_dtype="bf16", b_layout="kn",
                 epilogue="none", force: Optional[TileConfig] = None):
        self.M, self.N, self.K = M, N, K
        self.in_dtype, self.out_dtype, self.b_layout, self.epilogue = (
            in_dtype, out_dtype, b_layout, epilogue)
        self.handle = gemm_create(M, N, K, in_dtype, out_dtype, b_layout, epilogue, force)

    def __call__(self, A, B, C, stream=None):
        gemm_run(self.handle, A, B, C, stream)
        return C

    def config(self) -> TileConfig:
        return gemm_get_config(self.handle)

    def launch_config(self, A, B, C) -> TileConfig:
        return gemm_launch_config(self.handle, A, B, C)

    def autotune(self, A, B, C, stream=None, reps=10) -> float:
        return gemm_autotune(self.handle, A, B, C, stream, reps)

    def close(self):
        if self.handle:
            gemm_destroy(self.handle)
            self.handle = 0

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
