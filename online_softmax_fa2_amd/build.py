"""Build libosfa.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: ``python -m online_softmax_fa2_amd.build`` (or ``build_library()``).
Compiles every source under ``csrc/`` into ``_build/`` and links
``online_softmax_fa2_amd/_lib/libosfa.so``.  Always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libosfa.so")

ARCH = "gfx950"
SOURCES = ["api.cpp", "attn_fwd.hip", "attn_fwd_fp8.hip", "attn_bwd.hip", "decode.hip", "softmax.hip"]
# Packed FP32 ops are disabled for all device code: hipcc -O3 would
# otherwise form v_pk_* float32 instructions by itself.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# -fno-honor-nans where maxima of scores dominate the VALU work: the kernels
# never produce or test NaN (non-finite inputs are out of contract), and it
# lets fmaxf chains become v_max3_f32 with no NaN-quieting copies.  Not for
# decode.hip: there it makes the compiler keep twice the VGPRs (half the
# occupancy of an HBM-bound kernel).
NNAN_SOURCES = {"attn_fwd.hip", "attn_fwd_fp8.hip", "attn_bwd.hip", "softmax.hip"}
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libosfa.so)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + DEVICE_FLAGS
    if src in NNAN_SOURCES:
        cmd.append("-fno-honor-nans")
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build_library(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)
