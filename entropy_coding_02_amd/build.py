"""Build libkvc.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m entropy_coding_02_amd.build [--force]

Flags: -O3, no FP contraction (the quantizer's fp32 steps are each rounded
on their own), correctly rounded fp32 division, packed-fp32 instructions off.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvc.so")
SOURCES = ["kvc_abi.hip", "kvc_quantize.hip", "kvc_cdf.hip", "kvc_encode.hip", "kvc_decode.hip",
           "kvc_container.hip", "kvc_int8.hip", "kvc_delta.hip"]
ARCH = os.environ.get("KVC_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-std=c++17", "-O3", f"--offload-arch={ARCH}", "-fPIC", "-Wall",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _deps():
    hdrs = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    return hdrs + [os.path.join(ROOT, "include", "kvc.h")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(os.path.basename(src))[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile every HIP source and link libkvc.so.  Always rebuilds unless
    force=False and the library is newer than every source."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    if not force and os.path.exists(LIB):
        newest = max(os.path.getmtime(f) for f in srcs + _deps())
        if os.path.getmtime(LIB) >= newest:
            return LIB
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(force="--no-force" not in sys.argv, verbose=True)
