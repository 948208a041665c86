"""Builds libfa_mi355x.so (the gfx950 kernels and their C ABI) in-tree.

hipcc compiles the device code for gfx950 only.  Packed fp32 VALU instructions
are disabled for device code (``-packed-fp32-ops``); the host pass warns that
it does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libfa_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"
KERNEL_SOURCES = ("fa_fwd_f16.hip", "fa_fwd_f16_ks.hip", "fa_fwd_f32.hip", "fa_fwd_kvcache.hip", "fa_fwd_fp8.hip", "fa_bwd.hip")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build_library(verbose: bool = False, extra_flags=()) -> str:
    """Compile the kernels and the C ABI into LIB_PATH; returns that path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    common = ["-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, *extra_flags]
    objs = []
    for src in KERNEL_SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        _run([cc, f"--offload-arch={ARCH}", *common, "-fno-honor-nans",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    aobj = os.path.join(BUILD_DIR, "fa_api.o")
    _run([cc, *common, "-Wall", "-c", os.path.join(CSRC, "fa_api.cpp"), "-o", aobj], verbose)
    tmp = LIB_PATH + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, aobj, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


CALIB_SOURCE = "calib_mfma.hip"
CALIB_LIB_PATH = os.path.join(PKG, "libfa_calib.so")


def build_calibration_library(verbose: bool = False) -> str:
    """Compile the roofline calibration kernel (bench.py --calibrate) into its
    own small library, separate from the attention library."""
    tmp = CALIB_LIB_PATH + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          os.path.join(CSRC, CALIB_SOURCE), "-o", tmp], verbose)
    os.replace(tmp, CALIB_LIB_PATH)
    return CALIB_LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
    print(build_calibration_library(verbose=True))
