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
POISON_OUT = os.path.join(HERE, "libspgemm_poison.so")
# Units of the poison library (a test instrument: -DSPG_POISON turns the ring's released
# regions into NaN; see kPoison in csrc/gemm_kernels.hpp): every direct-to-LDS ring
# (S = 2..5 with 32x32x16, the 16x16x32 tiles, the A-deep and B-deep rings, release
# delay 1, persistent tiles), the wave-specialized ring and the register-staged
# misaligned mode, which also covers every configuration the shape heuristic picks.
POISON_UNITS = (8, 14, 21, 23, 24, 25, 26, 27, 28, 29, 30, 31, 32, 33, 34, 35)

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


def build(out: str = OUT, extra=(), poison: bool = False) -> str:
    """Compile the library; poison=True builds the poison library from POISON_UNITS."""
    unit_src = os.path.join(CSRC, "gemm_unit.hip")
    us = [u for u in units() if u in POISON_UNITS] if poison else units()
    keep = [f"-DSPG_KEEP_{u}=~,1" for u in us] if poison else []
    pdef = ["-DSPG_POISON"] if poison else []
    # (source, object name, defines): the host side, the GELU, and one object per unit
    jobs = [(os.path.join(CSRC, "gemm.hip"), "gemm.o", pdef + keep),
            (os.path.join(CSRC, "gelu.hip"), "gelu.o", [])]
    jobs += [(unit_src, f"gemm_unit{u}.o", pdef + [f"-DSPG_UNIT_IS_{u}=~,1"]) for u in us]
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


def build_poison(out: str = POISON_OUT) -> str:
    return build(out, poison=True)


if __name__ == "__main__":
    if sys.argv[1:2] == ["--poison"]:
        print(build_poison())
    else:
        print(build(*sys.argv[1:2]))
