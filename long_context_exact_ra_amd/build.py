"""Compile the HIP sources of the ring-attention share library into libra.so.

Run as `python -m long_context_exact_ra_amd.build`.  Objects go to
long_context_exact_ra_amd/_build/, the library to long_context_exact_ra_amd/libra.so.
Every device source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libra.so")
SOURCES = ["ra_api.cpp", "fwd_bf16.hip", "fwd_f32.hip", "util.hip", "bwd_bf16.hip",
           "fwd_fp8.hip", "fp8_quant.hip", "noalloc.hip"]
ARCH = "gfx950"
NO_NAN_SOURCES = {"fwd_bf16.hip", "fwd_fp8.hip"}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def common_flags(src: str = "") -> list[str]:
    flags = [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
             "-Wno-unused-result", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    if src in NO_NAN_SOURCES:
        # Inputs are finite by contract: max/min need no NaN quieting, so row maxima
        # compile to plain v_max3_f32.
        flags += ["-fno-honor-nans", "-mno-amdgpu-ieee"]
    return flags


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *common_flags(src), "-c", *lang, os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
