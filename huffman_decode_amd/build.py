"""Build libdf11.so in-tree: host codec (g++) + gfx950 decode kernel (hipcc)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdf11.so")
ARCH = os.environ.get("DF11_OFFLOAD_ARCH", "gfx950")

HOST_SOURCES = ["df11_host.cpp"]
HIP_SOURCES = ["df11_decode.hip"]

# Packed FP32 VALU forms are kept out of every HIP object.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-command-line-argument"]
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-pthread", "-Wall", "-Wextra"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def build_library(verbose: bool = False) -> str:
    """Compile every source (always) and link libdf11.so atomically."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run(["g++", *HOST_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src),
              "-o", obj], verbose)
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run(["hipcc", *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src),
              "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", *objs, "-o", tmp],
         verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
