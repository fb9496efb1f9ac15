"""The host half of libdf11 and the CPU oracle under sanitizers.

tests/sanitize/sanitize_driver.cpp runs the host codec (histogram, code book,
tables, sizes, the threaded encoder at 1 and 8 threads, the tile layout
helpers) against the oracle on seeded inputs and walks the error paths.  It
is built here with g++ twice from the sources: with AddressSanitizer and
UndefinedBehaviorSanitizer, and with ThreadSanitizer (the encoder's threads
OR the words they share with their neighbours atomically).  Each build must
run clean: exit status 0 and no sanitizer report.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES_C = [os.path.join(ROOT, "oracle", "df11_oracle.c")]
SOURCES_CXX = [os.path.join(ROOT, "huffman_decode_amd", "csrc", "df11_host.cpp"),
               os.path.join(ROOT, "tests", "sanitize", "sanitize_driver.cpp")]
INCLUDES = ["-I", os.path.join(ROOT, "include"), "-I",
            os.path.join(ROOT, "huffman_decode_amd", "csrc")]

CONFIGS = {
    "address_undefined": (["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-omit-frame-pointer"],
                          {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=1",
                           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}),
    "thread": (["-fsanitize=thread"], {"TSAN_OPTIONS": "halt_on_error=1"}),
}


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_host_codec_and_oracle_run_clean_under_sanitizer(tmp_path, name):
    flags, env_extra = CONFIGS[name]
    objs = []
    for src in SOURCES_C:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", *flags, "-c", src, "-o", obj])
        objs.append(obj)
    for src in SOURCES_CXX:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.check_call(["g++", "-O1", "-g", "-std=c++17", "-pthread", *flags, *INCLUDES,
                               "-c", src, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "driver")
    subprocess.check_call(["g++", *flags, "-pthread", *objs, "-o", exe])
    env = dict(os.environ, **env_extra)
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "WARNING: ThreadSanitizer",
                   "ERROR: LeakSanitizer"):
        assert marker not in out, out[-4000:]
    assert "0 failed checks" in out
