"""Build step for the C ABI test program: compiles df11_roundtrip.c with the
plain C compiler against include/df11.h, the in-tree libdf11.so and the HIP
runtime's C API.  Run by __graft_entry__.build() after the library."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
EXE = os.path.join(HERE, "df11_roundtrip")


def build_roundtrip(verbose: bool = False) -> str:
    pkg = os.path.join(ROOT, "huffman_decode_amd")
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "df11_roundtrip.c"), "-o", EXE + ".tmp",
           "-L", pkg, "-l:libdf11.so", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../huffman_decode_amd:" + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build_roundtrip(verbose=True))
