"""Build libdf11.so in-tree: host codec (g++) + gfx950 decode kernel (hipcc).

Beside the library it writes libdf11.kernels.json: a hash of each kernel's
machine code (its disassembly, addresses dropped), so that measurements taken
on one build can tell whether a later build still runs the same kernel.
"""
from __future__ import annotations

import hashlib
import json
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdf11.so")
KERNELS_JSON = os.path.join(PKG, "libdf11.kernels.json")
LLVM_BIN = "/opt/rocm/lib/llvm/bin"
ARCH = os.environ.get("DF11_OFFLOAD_ARCH", "gfx950")

HOST_SOURCES = ["df11_host.cpp"]
HIP_SOURCES = ["df11_decode.hip", "df11_ceiling.hip"]

HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
             "-Wno-unused-command-line-argument"]
# Packed FP32 VALU forms are kept out of the device code.  The feature is
# switched off in a device-only pass (the host compiler does not know it);
# the host pass then embeds that pass's code object.
DEVICE_ONLY_FLAGS = ["--cuda-device-only", "-Xclang", "-target-feature", "-Xclang",
                     "-packed-fp32-ops"]
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-pthread", "-Wall", "-Wextra"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def _kernel_hashes(fatbin: str) -> dict:
    """{kernel name: sha256[:16] of its instructions} for the gfx950 code
    object inside a device-only compile's bundle."""
    co = fatbin + ".co"
    subprocess.check_call([os.path.join(LLVM_BIN, "clang-offload-bundler"), "--unbundle",
                           "--type=o", f"--input={fatbin}",
                           f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}", f"--output={co}"])
    dis = subprocess.check_output([os.path.join(LLVM_BIN, "llvm-objdump"), "-d",
                                   "--no-show-raw-insn", "--no-leading-addr", "--demangle", co],
                                  text=True)
    out, name, lines = {}, None, []

    def flush():
        if name is not None:
            out[name] = hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]

    for line in dis.splitlines():
        m = re.match(r"^<(.+)>:$", line.strip())
        if m:
            flush()
            # "void (anonymous namespace)::df11_gemm_kernel<1>(...)" -> "df11_gemm_kernel<1>"
            sym = m.group(1).replace("(anonymous namespace)::", "").replace("void ", "")
            name, lines = re.sub(r"\(.*$", "", sym), []
            continue
        ins = line.split("//", 1)[0].strip()
        if ins:
            lines.append(ins)
    flush()
    return out


def build_library(verbose: bool = False) -> str:
    """Compile every source (always) and link libdf11.so atomically."""
    os.makedirs(BUILD, exist_ok=True)
    objs, hashes = [], {}
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run(["g++", *HOST_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src),
              "-o", obj], verbose)
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        fatbin = os.path.join(BUILD, src + ".hipfb")
        inc = ["-I", INCLUDE, "-I", CSRC]
        _run(["hipcc", *HIP_FLAGS, *DEVICE_ONLY_FLAGS, *inc, "-c", os.path.join(CSRC, src),
              "-o", fatbin], verbose)
        _run(["hipcc", *HIP_FLAGS, "--cuda-host-only", "-Xclang", "-fcuda-include-gpubinary",
              "-Xclang", fatbin, *inc, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
        hashes.update(_kernel_hashes(fatbin))
    tmp = LIB + ".tmp%d" % os.getpid()
    _run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", *objs, "-o", tmp],
         verbose)
    os.replace(tmp, LIB)
    with open(KERNELS_JSON + ".tmp", "w") as f:
        json.dump(hashes, f, indent=1, sort_keys=True)
    os.replace(KERNELS_JSON + ".tmp", KERNELS_JSON)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
