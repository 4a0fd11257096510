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
# streaming probes of the HBM (bench.py's ceiling measurement; not the method)
CALIB_SRC = os.path.join(HERE, "calib", "hbm_stream.hip")
CALIB_LIB = os.path.join(HERE, "libhbmstream.so")
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
    tmp = CALIB_LIB + ".tmp"
    run([hipcc(), *HIP_FLAGS, *inc, "-shared", CALIB_SRC, "-o", tmp])
    os.replace(tmp, CALIB_LIB)
    return LIB


def resource_usage(out_md: str) -> str:
    """Compile every HIP source with the compiler's kernel-resource-usage
    remarks and write a table of each kernel's registers, LDS and occupancy
    (waves per SIMD as the compiler computes it) to out_md."""
    import re
    import tempfile

    rows = []
    inc = [f"-I{INCLUDE}", f"-I{CSRC}"]
    with tempfile.TemporaryDirectory() as tmp:
        for src in HIP_SOURCES:
            r = subprocess.run([hipcc(), *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o",
                                os.path.join(tmp, "x.o"),
                                "-Rpass-analysis=kernel-resource-usage"],
                               check=True, capture_output=True, text=True)
            cur = None
            for line in r.stderr.splitlines():
                m = re.search(r"remark:\s+Function Name: (\S+)", line)
                if m:
                    cur = {"file": src, "name": m.group(1)}
                    rows.append(cur)
                    continue
                m = re.search(r"remark:\s+([A-Za-z][A-Za-z /\[\]]*?): (\S+) \[", line)
                if m and cur is not None:
                    cur[m.group(1).strip()] = m.group(2)
    demangled = subprocess.run(["c++filt"], input="\n".join(r["name"] for r in rows),
                               capture_output=True, text=True).stdout.splitlines()
    for r, dn in zip(rows, demangled):
        dn = dn.replace("(anonymous namespace)::", "")
        r["kernel"] = re.sub(r"\(.*", "", dn).replace("void ", "", 1)
    keys = ("VGPRs", "AGPRs", "TotalSGPRs", "ScratchSize [bytes/lane]", "LDS Size [bytes/block]",
            "Occupancy [waves/SIMD]", "SGPRs Spill", "VGPRs Spill")
    L = ["# Kernel resources on gfx950 (compiler remarks)", "",
         "Written by `python -m communication_compressed_optimizer_02_amd.build --resource-usage "
         "profiles/kernel_resources_gfx950.md`: every HIP source compiled with the library's flags",
         "and `-Rpass-analysis=kernel-resource-usage`.  Occupancy is the compiler's: waves per "
         "SIMD that the register and LDS use allow (at most 8 on gfx950; 512 VGPRs per SIMD lane "
         "are shared by the resident waves).", "",
         "| kernel | file | " + " | ".join(keys) + " |", "|---|---|" + "---|" * len(keys)]
    for r in sorted(rows, key=lambda r: (r["file"], r["kernel"])):
        L.append(f"| `{r['kernel']}` | {r['file']} | " + " | ".join(r.get(k, "—") for k in keys)
                 + " |")
    with open(out_md, "w") as f:
        f.write("\n".join(L) + "\n")
    return out_md


if __name__ == "__main__":
    if "--resource-usage" in sys.argv:
        print(resource_usage(sys.argv[sys.argv.index("--resource-usage") + 1]))
    else:
        print(build(verbose="-v" in sys.argv))
