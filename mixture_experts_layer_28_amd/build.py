"""Build libmoe.so (HIP kernels for gfx950 + the C ABI) in place.

    python -m mixture_experts_layer_28_amd.build

Each source is compiled by hipcc into ``_build/`` in parallel, then linked
into ``mixture_experts_layer_28_amd/libmoe.so``.  Packed FP32 instructions
are switched off for device code (``-packed-fp32-ops``).  No fast-math:
NaN propagation and denormals are part of the routing contract.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmoe.so")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["moe_abi.cpp", "route.hip", "route_sigmoid.hip", "dispatch.hip",
           "gemm.hip", "gemm_big.hip", "combine.hip", "router_weights.hip",
           "backward.hip"]
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature",
                "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
          "-I" + os.path.join(ROOT, "include")]


def _compile(src):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC] + COMMON + DEVICE_FLAGS + ["-c", os.path.join(CSRC, src),
                                             "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (
            src, " ".join(cmd), r.stderr))
    return obj


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950"] + objs + [
        "-o", tmp]
    try:
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd),
                                                         r.stderr))
        # every symbol must resolve: a kernel whose host stub went missing
        # shows up here rather than at the first call
        import ctypes
        ctypes.CDLL(tmp)
        os.replace(tmp, OUT)
    finally:
        if os.path.exists(tmp):
            os.remove(tmp)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build()
    sys.exit(0)
