"""Build libspgemm.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

The kernel instantiations listed in csrc/variants.inc are spread over translation
units by the first field of each line: csrc/gemm_unit.hip is compiled once per unit
number (with -DSPG_UNIT_IS_<n>=~,1 selecting that unit's lines), so the units compile
in parallel.  csrc/gemm.hip holds the GEMM's host side (C ABI, variant table) and
csrc/gelu.hip the standalone elementwise GELU (include/spgelu.h).
"""

from __future__ import annotations

import os
import re
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


def units() -> list:
    """Unit numbers that appear as the first field of an SPG_V line of variants.inc."""
    with open(os.path.join(CSRC, "variants.inc")) as fh:
        found = {int(m.group(1)) for m in re.finditer(r"^SPG_V\((\d+),", fh.read(), re.M)}
    return sorted(found)


def build(out: str = OUT, extra=()) -> str:
    unit_src = os.path.join(CSRC, "gemm_unit.hip")
    # (source, object name, defines): the host side, the GELU, and one object per unit
    jobs = [(os.path.join(CSRC, "gemm.hip"), "gemm.o", []),
            (os.path.join(CSRC, "gelu.hip"), "gelu.o", [])]
    jobs += [(unit_src, f"gemm_unit{u}.o", [f"-DSPG_UNIT_IS_{u}=~,1"]) for u in units()]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory(prefix="spgemm_build_") as tmp:
        def compile_one(job):
            src, name, defs = job
            obj = os.path.join(tmp, name)
            cmd = ["hipcc", *FLAGS, *extra, *defs, *inc, "-c", src, "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-4000:]}")
            return obj
        with ThreadPoolExecutor(max_workers=_jobs()) as pool:
            objs = list(pool.map(compile_one, jobs))
        tmp_out = out + ".tmp"
        subprocess.run(["hipcc", *FLAGS, "-shared", *objs, "-o", tmp_out], check=True)
        os.replace(tmp_out, out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
