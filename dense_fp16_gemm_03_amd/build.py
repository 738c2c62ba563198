"""Build libgemm_f16.so (hipcc, gfx950) in the package directory.

    python -m dense_fp16_gemm_03_amd.build [--asm] [--vendor]

``--asm`` also writes the gfx950 assembly of the kernels to ``_build/`` so
register, spill and LDS figures can be read from it. ``--vendor`` also builds
libvendor_hipblaslt.so, the hipBLASLt context arm bench.py --vendor times.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libgemm_f16.so")
ASM_DIR = os.path.join(ROOT, "_build")
SOURCES = [os.path.join(CSRC, "gemm_kernels.hip"), os.path.join(CSRC, "gemm_api.cpp"),
           os.path.join(CSRC, "gemm_noalloc.hip")]
# hipBLASLt context arm (measurement only; see vendor/hipblaslt_arm.cpp).
VENDOR_SOURCE = os.path.join(PKG, "vendor", "hipblaslt_arm.cpp")
VENDOR_LIBRARY = os.path.join(PKG, "libvendor_hipblaslt.so")
ARCH = "gfx950"

# Packed-fp32 VALU forms are kept out of the generated code (this flag is a
# target feature of the device pass; the host pass warns that it ignores it).
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-DNDEBUG", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: install ROCm or put hipcc on PATH")
    return path


def build(asm: bool = False, verbose: bool = False) -> str:
    tmp = LIBRARY + ".tmp"
    cmd = [hipcc(), *COMMON_FLAGS, "-shared", *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    if asm:
        emit_asm(verbose)
    return LIBRARY


def build_vendor(verbose: bool = False) -> str:
    """The hipBLASLt context arm: host code only, linked against hipBLASLt."""
    tmp = VENDOR_LIBRARY + ".tmp"
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = [hipcc(), "-O2", "-std=c++17", "-fPIC", "-shared", VENDOR_SOURCE,
           f"-L{rocm}/lib", "-lhipblaslt", f"-Wl,-rpath,{rocm}/lib", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, VENDOR_LIBRARY)
    return VENDOR_LIBRARY


def emit_asm(verbose: bool = False) -> str:
    """Device assembly of the kernels (gfx950) into _build/gemm_kernels-gfx950.s."""
    os.makedirs(ASM_DIR, exist_ok=True)
    out = os.path.join(ASM_DIR, f"gemm_kernels-{ARCH}.s")
    cmd = [hipcc(), *COMMON_FLAGS, "--cuda-device-only", "-S", SOURCES[0], "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    build(asm="--asm" in sys.argv, verbose=True)
    print(LIBRARY)
    if "--vendor" in sys.argv:
        print(build_vendor(verbose=True))
