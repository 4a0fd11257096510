"""Build liboba.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run ``python -m communication_compressed_optimizer_02_amd.build``; the
library is written next to this file.  Host-only planning code is compiled
by the host compiler; HIP sources by hipcc with:
  * ``-ffp-contract=off``: no product is fused into a following add, so the
    binary32 operation order of the method is kept exactly;
  * ``-fhip-fp32-correctly-rounded-divide-sqrt``: correctly rounded division
    and square root (HIP's default, stated explicitly);
  * ``-Xclang -target-feature -Xclang -packed-fp32-ops``: no packed fp32
    instructions are generated.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "liboba.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]
# one translation unit per pass, plus the C ABI
HIP_SOURCES = ("warmup.hip", "compress.hip", "scales.hip", "server.hip", "update.hip",
               "small.hip", "api.hip")


def hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    inc = [f"-I{INCLUDE}", f"-I{CSRC}"]
    objs = []

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)

    o = os.path.join(obj_dir, "layout.o")
    run(["g++", *HOST_FLAGS, *inc, "-c", os.path.join(CSRC, "layout.cpp"), "-o", o])
    objs.append(o)
    for src in HIP_SOURCES:
        o = os.path.join(obj_dir, src.replace(".hip", ".o"))
        run([hipcc(), *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", o])
        objs.append(o)
    tmp = LIB + ".tmp"
    run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
