"""Build libecf8.so (host encoder + gfx950 decode kernels) in-tree with hipcc.

Usage: python -m lossless_entropy_coded_ecf8_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libecf8.so")
ARCH = os.environ.get("ECF8_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# hipcc flags for all HIP code: gfx950 only, packed-FP32 instructions disabled.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-result", "-I" + INCLUDE]


def sources():
    return [os.path.join(CSRC, f) for f in ("ecf8_host.cpp", "ecf8_decode.hip", "ecf8_encode.hip", "ecf8v_host.cpp",
                                                "ecf8v_decode.hip", "hbm_copy.hip")]


def build(verbose: bool = False, extra=None) -> str:
    """Compile every source and link libecf8.so (always rebuilds)."""
    objs = []
    for src in sources():
        obj = os.path.join(CSRC, os.path.basename(src) + ".o")
        cmd = [HIPCC] + HIP_FLAGS + (extra or [])
        if src.endswith(".hip"):
            cmd += ["-x", "hip"]
        cmd += ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs + ["-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
