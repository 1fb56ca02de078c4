"""Build libqgemv_q4.so for gfx950 with hipcc (in-tree, no JIT cache).

    python gemm_qgemv_q4_amd/build.py          # builds gemm_qgemv_q4_amd/lib/libqgemv_q4.so

(Run it as a script: importing it through the package would first load the
library that it is about to replace.)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIBNAME = "libqgemv_q4.so"
ARCH = os.environ.get("QG_OFFLOAD_ARCH", "gfx950")

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    "-ffp-contract=off",                 # every fused multiply-add is written out explicitly
    "-mcode-object-version=5",
    # packed FP32 instructions (v_pk_*_f32) are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # leading scalar kernel arguments are preloaded into scalar registers
    # (the K-sliced GEMV passes what a single-part launch needs that way)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libqgemv_q4)")


def build(verbose: bool = True) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    out = os.path.join(LIBDIR, LIBNAME)
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "api.hip"), "-o", tmp]
    t0 = time.time()
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode})")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out} in {time.time() - t0:.1f}s")
    build_read_probe(verbose)
    return out


def build_read_probe(verbose: bool = True) -> str:
    """libqg_read.so: the streaming-read probe that bench.py times as a read
    ceiling beside each memory-bound workload (not part of the product ABI)."""
    out = os.path.join(LIBDIR, "libqg_read.so")
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, os.path.join(CSRC, "stream_read.hip"), "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed for the read probe ({res.returncode})")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build()
