"""Build libspgemm.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "gemm.hip")
OUT = os.path.join(HERE, "libspgemm.so")

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in any generated code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def build(out: str = OUT, extra=()) -> str:
    tmp = out + ".tmp"
    cmd = ["hipcc", *FLAGS, *extra, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(HERE, "csrc"), SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
