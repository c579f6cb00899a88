"""Build libkda.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Usage: python -m chunked_gated_delta_09_amd.build   (or build() from Python)
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libkda.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["kda_api.cpp", "kda_fwd.hip", "kda_scan.hip", "kda_bwd.hip", "kda_noalloc.hip"]
ARCH = "gfx950"

# Packed fp32 VALU instructions are disabled: plain float code is compiled to scalar VALU ops.
HIP_FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-mcode-object-version=5", "-fPIC", "-fvisibility=hidden",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             # MFMA accumulators in ordinary VGPRs: kernels with more than 256 registers per
             # lane would otherwise keep them in AGPRs and copy them to VGPRs for every VALU use
             "-mllvm", "-amdgpu-mfma-vgpr-form", "-I", INCLUDE, "-I", CSRC]


def _hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), "hipcc"):
        if os.path.isabs(cand) and os.path.exists(cand):
            return cand
    return "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc()] + HIP_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libkda.so next to this file. Always rebuilds."""
    os.makedirs(OBJDIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-mcode-object-version=5", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
