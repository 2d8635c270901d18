"""Ahead-of-time build of the gfx950 HIP library ``libmoe_ragged_bf16.so``.

One ``hipcc`` invocation compiles the kernels and the C ABI for gfx950 only and
links them into the package directory.  Run ``python -m moe_ragged_bf16_amd.build``.
"""
from __future__ import annotations

import os
import re
import shutil
import tempfile
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
    # never emit packed fp32 arithmetic (v_pk_add/mul/fma_f32).  The feature
    # belongs to the gfx950 device pass; the host pass prints that it does not
    # know it and ignores it.  check_no_packed_fp32() verifies the result.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # export only the entry points the public header marks MDG_API
    "-fvisibility=hidden",
]

LLVM_BIN = "/opt/rocm/llvm/bin"
DEVICE_TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
PACKED_FP32 = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")


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
    try:
        check_no_packed_fp32(tmp)
    except Exception:
        os.unlink(tmp)
        raise
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def device_assembly(lib_path: str = LIB_PATH) -> str:
    """AMD assembly of the gfx950 code object built into `lib_path` (its
    .hip_fatbin section, unbundled and disassembled with ROCm's LLVM tools)."""
    with tempfile.TemporaryDirectory() as d:
        fat = os.path.join(d, "fatbin.bin")
        co = os.path.join(d, "gfx950.co")
        for cmd in ([os.path.join(LLVM_BIN, "llvm-objcopy"), "--dump-section", ".hip_fatbin=" + fat, lib_path],
                    [os.path.join(LLVM_BIN, "clang-offload-bundler"), "--unbundle", "--type=o", "--input=" + fat,
                     "--targets=" + DEVICE_TARGET, "--output=" + co]):
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                raise RuntimeError("extracting the gfx950 code object failed: " + res.stderr)
        res = subprocess.run([os.path.join(LLVM_BIN, "llvm-objdump"), "-d", co], capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("llvm-objdump failed: " + res.stderr)
        return res.stdout


def check_no_packed_fp32(lib_path: str = LIB_PATH) -> int:
    """Raises if the built device code holds a packed fp32 add, multiply or
    fma; returns the number of MFMA instructions seen (a sanity count)."""
    asm = device_assembly(lib_path)
    bad = [ln.strip() for ln in asm.splitlines() if PACKED_FP32.search(ln)]
    if bad:
        raise RuntimeError("packed fp32 arithmetic in the gfx950 code: %d instructions, e.g. %s" % (len(bad), bad[0]))
    return sum(1 for ln in asm.splitlines() if "v_mfma" in ln)


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
