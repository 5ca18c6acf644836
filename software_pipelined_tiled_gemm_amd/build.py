"""Build libspgemm.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

The kernel instantiations are spread over csrc/gemm_tu*.hip so that they compile
in parallel; csrc/gemm.hip holds the GEMM's host side (C ABI, variant table) and
csrc/gelu.hip the standalone elementwise GELU (include/spgelu.h).
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libspgemm.so")

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in any generated code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def _jobs() -> int:
    n = os.cpu_count() or 4
    for var in ("MAX_JOBS", "CMAKE_BUILD_PARALLEL_LEVEL"):
        if os.environ.get(var, "").isdigit():
            n = min(n, int(os.environ[var]))
    return max(1, min(n, 16))


def build(out: str = OUT, extra=()) -> str:
    sources = ([os.path.join(CSRC, "gemm.hip"), os.path.join(CSRC, "gelu.hip")]
               + sorted(glob.glob(os.path.join(CSRC, "gemm_tu*.hip"))))
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory(prefix="spgemm_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = ["hipcc", *FLAGS, *extra, *inc, "-c", src, "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-4000:]}")
            return obj
        with ThreadPoolExecutor(max_workers=_jobs()) as pool:
            objs = list(pool.map(compile_one, sources))
        tmp_out = out + ".tmp"
        subprocess.run(["hipcc", *FLAGS, "-shared", *objs, "-o", tmp_out], check=True)
        os.replace(tmp_out, out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
