"""Ahead-of-time build of the gfx950 HIP library ``libmoe_ragged_bf16.so``.

One ``hipcc`` invocation compiles the kernels and the C ABI for gfx950 only and
links them into the package directory.  Run ``python -m moe_ragged_bf16_amd.build``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmoe_ragged_bf16.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["grouped_gemm_kernels.hip", "capi.cpp"]

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # the accumulate epilogue and the split reduction are plain IEEE adds
    "-ffp-contract=off",
    # never emit packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def build(verbose: bool = False) -> str:
    """Compile the library (always) and return its path."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC]
    for s in SOURCES:
        cmd += ["-x", "hip", os.path.join(CSRC, s)]
    cmd += ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building %s" % LIB_NAME)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


C_SMOKE_SRC = os.path.join(ROOT, "tests", "c_abi_smoke.cpp")
C_SMOKE_BIN = os.path.join(ROOT, "tests", "c_abi_smoke")


def build_c_smoke(verbose: bool = False) -> str:
    """Compile the C++ caller of the C ABI used by the tests (host code only,
    linked against the library with a relative rpath)."""
    cmd = [hipcc(), "-O2", "-std=c++17", "-I", INCLUDE, C_SMOKE_SRC, "-L", PKG_DIR, "-lmoe_ragged_bf16",
           "-Wl,-rpath,$ORIGIN/../moe_ragged_bf16_amd", "-o", C_SMOKE_BIN]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building %s" % C_SMOKE_BIN)
    return C_SMOKE_BIN


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_c_smoke(verbose=True))
