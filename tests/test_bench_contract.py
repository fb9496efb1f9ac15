"""bench.py's host-side parts, on the CPU: the refusal of more than one GPU,
the algorithmic byte count behind `value` and `roofline.achieved`, and the
CPU baseline leg (the oracle, bit-exact, with its core count, and the
oracle's encoder checked against the host encoder's arrays)."""
import dataclasses
import importlib.util
import json
import os
import subprocess
import sys

import numpy as np

import huffman_decode_amd as hd
from huffman_decode_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_algorithmic_bytes_count_each_array_once():
    """Bytes read: the code bits, one 5-bit gap per 64-bit slice plus the
    sentinel, one u32 position per block plus the sentinel, one
    sign|mantissa byte per weight and the tables; written: two bytes per
    weight.  Each figure fits inside the array the encoder produced (those
    carry padding and guards)."""
    bench = _bench()
    for n, kind in ((1, "normal"), (4097, "normal"), (300_001, "normal"), (65_536, "single")):
        enc = hd.encode(wl.random_small(n, 11, kind))
        s = enc.sizes
        nb = int(s.n_blocks)
        rd, wr = bench.algorithmic_bytes(enc)
        code = -(-int(s.total_bits) // 8)
        gaps = -(-5 * (64 * nb + 1) // 8)
        assert wr == 2 * n
        assert rd == code + gaps + 4 * (nb + 1) + n + int(s.lut_bytes)
        assert code <= enc.stream.nbytes and gaps <= enc.gaps.nbytes
        assert 4 * (nb + 1) <= enc.block_pos.nbytes and n <= enc.signmant.nbytes
        # blocks of 4096 code bits: exactly enough of them for the codes
        assert 4096 * (nb - 1) < int(s.total_bits) <= 4096 * nb


def test_cpu_baseline_is_the_oracle_and_checks_its_result():
    bench = _bench()
    w = wl.random_small(200_003, 12, "normal")
    wlx = wl.Workload("small", w)
    enc = hd.encode(w)
    got = bench.cpu_baseline(wlx, enc)
    assert got["kind"] == "oracle" and got["bit_exact"] is True
    assert 1 <= got["cores"] <= 16 and got["one_core"]["cores"] == 1
    assert got["value"] > 0 and got["unit"] == "GB/s" and "small" in got["sample"]
    assert got["encode_one_core"]["same_arrays_as_host_encoder"] is True
    # a flipped code bit must show: the check compares with the original words
    stream = enc.stream.copy()
    stream[len(stream) // 3] ^= np.uint8(0x10)
    bad = bench.cpu_baseline(wlx, dataclasses.replace(enc, stream=stream))
    assert bad["bit_exact"] is False
    assert bad["encode_one_core"]["same_arrays_as_host_encoder"] is False
