"""Build libocg.so (HIP, gfx950) in-tree with hipcc.

    python communication_overlapped_gemm_amd/build.py

(run as a file: importing the package loads libocg.so, which this builds)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libocg.so")
SOURCES = ["kernels.hip", "attention.hip", "api.cpp"]
# Per-source code-generation options. The attention kernel keeps its MFMA
# accumulators in VGPRs (VGPR form): the softmax reads every score with VALU
# instructions, which cannot take accumulation registers, and in the default
# form each one would be moved through a VGPR per key block (the GEMM kernels
# measured slower in that form). Its maxima assume no NaN inputs, so fmaxf
# needs no quieting of its operands.
SOURCE_FLAGS = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"]}

# Packed-fp32 instructions are disabled (v_pk_*_f32 forms are not trusted on
# the test machines); hipcc's host pass warns that it does not know the
# feature, which is harmless.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    # m0 is listed as clobbered by the direct-to-LDS load asm; the compiler
    # warns because m0 is reserved, and uses m0 nowhere else in these kernels.
    "-Wno-inline-asm",
    "-D__HIP_PLATFORM_AMD__",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "unknown target feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l and "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source to an object (with its own options), in
    parallel, then link libocg.so."""
    from concurrent.futures import ThreadPoolExecutor
    tmp = os.path.join(PKG, "_build")
    os.makedirs(tmp, exist_ok=True)
    objs = [os.path.join(tmp, s + ".o") for s in SOURCES]
    cmds = [[hipcc(), *FLAGS, *SOURCE_FLAGS.get(s, []), "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"], verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
