"""Builds libmoe.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m mixture_experts_layer_10_amd.build

Each translation unit is compiled separately (the router with
-ffp-contract=off, so that its float32 steps are single IEEE operations),
then linked into mixture_experts_layer_10_amd/libmoe.so.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["moe_api.hip", "route.hip", "dispatch.hip", "gemm.hip", "gemm_big.hip", "gemm_pf.hip", "gemm_fp8.hip", "gemm_mx.hip", "combine.hip", "load_stats.hip", "peak.hip", "gemm_cores.hip"]
EXTRA = {"route.hip": ["-ffp-contract=off"]}


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe.so)")


def common_flags():
    return ["--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-Wall",
            "-Wno-unused-function", "-Wno-unused-variable",
            # Packed-fp32 instructions are kept out of every code object.
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(PKG, "..", "include")]


def _compile(src):
    cc = hipcc()
    obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
    cmd = [cc, *common_flags(), *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=True):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
