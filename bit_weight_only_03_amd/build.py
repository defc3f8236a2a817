"""Build libw4a16.so (all HIP sources under csrc/) for gfx950 with hipcc.

    python -m bit_weight_only_03_amd.build

The library is built in-tree next to this file.  Packed-fp32 instructions are
disabled for the device code (-packed-fp32-ops); hipcc's host pass prints a
harmless warning that it does not know that feature.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libw4a16.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


# Per-source device flags.  The 4-bit GEMV kernel takes the arguments every
# wave needs first as leading scalars and pointers (ten arguments, 14
# dwords; the W16A16, ternary and M-tiled kernels likewise); this option compiles them as
# preloaded into SGPRs at wave launch,
# which saves each wave a scalar load before its first memory access
# (measured 0.25-0.3 us per call on the qkv and o_proj shapes).  The code
# object keeps a prologue that loads them itself where the firmware does not
# preload.
SOURCE_FLAGS = {"w4_gemv.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=10"],
                "w16_gemv.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=10"],
                "w2t.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=10"],
                "w4_gemm.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=10"]}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(HERE, "_build", os.path.basename(src) + ".o")
    cmd = [HIPCC, "-c", "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           *SOURCE_FLAGS.get(os.path.basename(src), []),
           "-Wall", "-Wno-unused-function", "-o", obj, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if errs.strip() and verbose:
        print(errs, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel) and link the shared library; always
    rebuilds."""
    os.makedirs(os.path.join(HERE, "_build"), exist_ok=True)
    srcs = sources()
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", "0")) or os.cpu_count() or 1, 8))
    with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
        objs = list(pool.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
