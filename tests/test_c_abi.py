"""The library used from C alone: tests/c_abi/df11_roundtrip.c includes only
include/df11.h and the HIP runtime's C API, links libdf11.so, and encodes,
decodes and checks seeded BF16 weights with no Python or torch in the process.
On the CPU it runs its host half (histogram, code book, table image, sizes,
encode); on the GPU the whole round trip, bit for bit against the original
words, with a misaligned output refused first and the status word left 0."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_abi", "df11_roundtrip")


def _run(*args, timeout=120, build_if_missing=False):
    if not os.path.exists(EXE) and build_if_missing:  # the host half only: a CPU compile
        import sys
        sys.path.insert(0, os.path.dirname(HERE))
        from tests.c_abi.build import build_roundtrip
        build_roundtrip()
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: build it with __graft_entry__.build()")
    print(f"[c_abi] df11_roundtrip {' '.join(args)}", flush=True)
    return subprocess.run([EXE, *args], capture_output=True, text=True, timeout=timeout)


@pytest.mark.parametrize("n,seed", [(1, 1), (65, 2), (200_003, 5)])
def test_c_program_host_half(n, seed):
    r = _run("--host", str(n), str(seed), build_if_missing=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "df11_roundtrip host ok" in r.stdout


@pytest.mark.gpu
@pytest.mark.parametrize("n,seed", [(1, 1), (4097, 3), (3_000_017, 11)])
def test_c_program_round_trip_on_the_gpu(n, seed):
    r = _run(str(n), str(seed))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 words differ, status 0" in r.stdout and "df11_roundtrip ok" in r.stdout
