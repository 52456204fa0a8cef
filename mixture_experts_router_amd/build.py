"""Build libmoe_amd.so: the HIP kernels and the C ABI, for gfx950 only.

    python -m mixture_experts_router_amd.build

Every source is compiled with hipcc --offload-arch=gfx950 into _build/, then
linked into mixture_experts_router_amd/libmoe_amd.so (in-tree, so the built
library travels with the source tree).
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_amd.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["router.hip", "sort.hip", "gemv.hip", "gemm.hip", "gemm_w4.hip", "gemm_w56.hip", "gemm_w8.hip",
           "gemm_w16.hip", "gemm_wf4.hip", "combine.hip", "moe_abi.cpp"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    # packed fp32 instructions stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, r.stdout, r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
