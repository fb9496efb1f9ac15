"""Pins for the CPU oracle: each test checks it against something other than itself.

Sources: the page "DFloat11: lossless BFloat16 compression" (ai-infrastructure.net)
-- its printed worked example (golden file), the entropy bound it states, and the
chunk-decode premise of its two-phase kernel -- plus mathematics (Kraft equality,
brute-force optimal prefix codes, Fibonacci closed forms, the BF16 definition) and
a small example derived by hand.
"""
import itertools
import math
import os

import numpy as np
import pytest

import oracle
from huffman_decode_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(None, 1)
            vals[key] = rest
    return vals


def _kraft_units(lengths, unit_bits=40):
    """Kraft sum scaled by 2**unit_bits, exact in integers."""
    return sum(1 << (unit_bits - int(l)) for l in lengths if l > 0)


# ------------------------------------------------------------ BF16 fields

def test_split_join_exhaustive():
    """join(split(w)) == w for all 65536 BF16 patterns."""
    w = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    e, sm = oracle.split_bf16(w)
    assert np.array_equal(oracle.join_bf16(e, sm), w)
    # each (exponent, sign|mantissa) pair appears exactly once
    assert np.unique(e.astype(np.uint32) * 256 + sm).size == 1 << 16


def test_split_fields_against_bf16_definition():
    """BF16 = sign | 8-bit biased exponent (bias 127) | 7-bit mantissa."""
    import torch
    vals = torch.tensor([1.0, -2.0, 0.5, 3.0, -0.0, 2.0 ** -126, 1.5 * 2.0 ** 10],
                        dtype=torch.bfloat16)
    w = vals.view(torch.int16).numpy().view(np.uint16)
    e, sm = oracle.split_bf16(w)
    assert e.tolist() == [127, 128, 126, 128, 0, 1, 137]
    # sign in the top bit of the raw byte; 3.0 = 1.1b -> mantissa 0x40; 1.5 -> 0x40
    assert sm.tolist() == [0x00, 0x80, 0x00, 0x40, 0x80, 0x00, 0x40]


# ------------------------------------------------- the page's worked example

def _page_inputs():
    rng = np.random.default_rng(0)
    w = wl.to_bf16(rng.normal(0.0, 0.02, 200_000).astype(np.float32))
    u = rng.integers(0, 256, 200_000).astype(np.uint8)
    q = wl.to_bf16((rng.integers(-127, 128, 200_000) * (0.02 / 127)).astype(np.float32))
    return w, u, q


def _bits_per_weight(w):
    e, _ = oracle.split_bf16(w)
    h = oracle.histogram(e)
    ln = oracle.huffman_lengths(h)
    return 8.0 + oracle.average_length(h, ln)


def test_page_worked_example_statistics():
    g = _golden("p3_worked_example.txt")
    w, u, q = _page_inputs()
    e, sm = oracle.split_bf16(w)
    h = oracle.histogram(e)
    ln = oracle.huffman_lengths(h)
    H = oracle.entropy_bits(h)
    avg = oracle.average_length(h, ln)
    assert int((h > 0).sum()) == int(g["distinct_exponents"])
    assert f"{H:.3f}" == g["exponent_entropy_bits"]
    assert f"{avg:.3f}" == g["avg_code_length_bits"]
    assert int(ln.max()) == int(g["max_code_length"])
    assert f"{8.0 + avg:.3f}" == g["bits_per_weight"]
    assert f"{(8.0 + avg) / 16 * 100:.1f}" == g["compressed_percent_of_bf16"]
    assert f"{oracle.entropy_bits(np.bincount(sm, minlength=256)):.3f}" == g["signmant_entropy_bits"]
    # flat table over the longest code: 2**max entries of (symbol byte, length byte)
    assert 2 * (1 << int(ln.max())) // 1024 == int(g["flat_lut_kib"])
    # hierarchy of 256-entry tables; the page's tables hold 1+1+2 bytes per entry
    nt = oracle.count_subtables(ln, 8)
    assert nt == int(g["hier_tables"])
    assert f"{nt * 256 * 4 / 1024:.2f}" == g["hier_tables_kib"]
    # entropy bound stated on the page: H <= avg < H + 1
    assert H <= avg < H + 1.0

    # uniform exponents degenerate to an 8-bit code; one u32 offset per 4096 weights
    uh = oracle.histogram(u)
    uavg = oracle.average_length(uh, oracle.huffman_lengths(uh))
    assert f"{8.0 + uavg:.3f}" == g["uniform_bits_per_weight"]
    assert f"{8.0 + uavg + 32.0 / 4096:.3f}" == g["uniform_bits_per_weight_with_offsets"]
    # single exponent: 1-bit code
    d = np.full(1000, 0x3E, np.uint8)
    dh = oracle.histogram(d)
    assert f"{8.0 + oracle.average_length(dh, oracle.huffman_lengths(dh)):.3f}" == \
        g["single_bits_per_weight"]
    # int8-rounded tensor
    assert f"{_bits_per_weight(q):.3f}" == g["int8_bits_per_weight"]
    _, word_counts = np.unique(q, return_counts=True)
    assert f"{oracle.entropy_bits(word_counts):.3f}" == g["int8_word_entropy_bits"]


def test_page_worked_example_roundtrip_chunks_and_corruption():
    g = _golden("p3_worked_example.txt")
    w, _, _ = _page_inputs()
    e, sm = oracle.split_bf16(w)
    ln = oracle.huffman_lengths(oracle.histogram(e))
    stream, total = oracle.encode_bits(e, ln)
    dec, end = oracle.decode(stream, total, 0, e.size, ln)
    assert end == total
    assert np.array_equal(oracle.join_bf16(dec, sm), w)
    assert w.size == int(g["roundtrip_weights"])

    # independent decoders started at every 4096th code give the serial result
    starts = np.concatenate([[0], np.cumsum(ln[e].astype(np.int64))])[::4096]
    starts = starts[:-1] if e.size % 4096 == 0 else starts
    parts = []
    for i, s in enumerate(starts.tolist()):
        cnt = min(4096, e.size - 4096 * i)
        part, _ = oracle.decode(stream, total, s, cnt, ln)
        parts.append(part)
    assert np.array_equal(np.concatenate(parts), e)
    assert len(starts) == int(g["chunks"])
    assert 4 * len(starts) == int(g["chunk_offset_array_bytes"])

    # one flipped bit desynchronises the decoder
    k = int(g["flipped_bit"])
    bad = stream.copy()
    bad[k >> 3] ^= np.uint8(1 << (k & 7))
    dec_bad, _ = oracle.decode(bad, total, 0, e.size, ln)
    assert int((dec_bad != e).sum()) == int(g["corrupted_weights"])


# ------------------------------------------------------------ hand example

def test_hand_example():
    g = _golden("hand_example.txt")
    seq = np.array([int(x) for x in g["sequence"].split()], np.uint8)
    want_len = {int(k): int(v) for k, v in (p.split(":") for p in g["lengths"].split())}
    want_code = {int(k): int(v) for k, v in (p.split(":") for p in g["codes"].split())}
    h = oracle.histogram(seq)
    ln = oracle.huffman_lengths(h)
    assert {s: int(ln[s]) for s in range(256) if ln[s]} == want_len
    code = oracle.canonical_codes(ln)
    assert {s: int(code[s]) for s in want_code} == want_code
    stream, total = oracle.encode_bits(seq, ln, 4)
    assert total == int(g["total_bits"])
    assert stream[:2].tolist() == [int(x, 16) for x in g["packed"].split()]
    assert stream[2:].tolist() == [0, 0]
    dec, end = oracle.decode(stream, total, 0, seq.size, ln)
    assert end == total and np.array_equal(dec, seq)


# ----------------------------------------------------- optimality and limits

def _brute_min_cost(counts, max_len):
    """Minimum sum(count * length) over every prefix code (Kraft <= 1)."""
    k = len(counts)
    best = None
    c = np.array(counts, np.int64)
    for ls in itertools.product(range(1, max_len + 1), repeat=k):
        if sum(2.0 ** -l for l in ls) <= 1.0 + 1e-12:
            cost = int((c * np.array(ls)).sum())
            best = cost if best is None else min(best, cost)
    return best


@pytest.mark.parametrize("seed", range(12))
def test_huffman_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    k = int(rng.integers(2, 7))
    counts = rng.integers(1, 51, k)
    syms = rng.choice(256, k, replace=False)
    h = np.zeros(256, np.uint64)
    h[syms] = counts
    ln = oracle.huffman_lengths(h)
    cost = int((h * ln.astype(np.uint64)).sum())
    assert cost == _brute_min_cost(counts.tolist(), k - 1)
    assert _kraft_units(ln) == 1 << 40
    assert set(np.nonzero(ln)[0].tolist()) == set(syms.tolist())


@pytest.mark.parametrize("seed", range(8))
def test_length_limit_against_brute_force(seed):
    rng = np.random.default_rng(200 + seed)
    k = int(rng.integers(4, 7))
    counts = np.array([int(x) for x in rng.geometric(0.35, k) * rng.integers(1, 40, k)])
    counts = np.maximum(counts, 1)
    h = np.zeros(256, np.uint64)
    h[np.arange(k) * 7] = counts
    free = oracle.huffman_lengths(h)
    free_cost = int((h * free.astype(np.uint64)).sum())
    for L in range(max(2, math.ceil(math.log2(k))), k):
        ln, rounds = oracle.limited_lengths(h, L)
        cost = int((h * ln.astype(np.uint64)).sum())
        assert int(ln.max()) <= L
        assert _kraft_units(ln) == 1 << 40
        assert cost >= _brute_min_cost(counts.tolist(), L) >= free_cost
        if int(free.max()) <= L:
            assert rounds == 0 and np.array_equal(ln, free)


@pytest.mark.parametrize("seed", range(10))
def test_kraft_equality_and_entropy_bound(seed):
    rng = np.random.default_rng(300 + seed)
    k = int(rng.integers(2, 257))
    h = np.zeros(256, np.uint64)
    h[rng.choice(256, k, replace=False)] = rng.integers(1, 10 ** 6, k)
    ln = oracle.huffman_lengths(h)
    assert _kraft_units(ln, 300) == 1 << 300
    H = oracle.entropy_bits(h)
    avg = oracle.average_length(h, ln)
    assert H <= avg + 1e-12 and avg < H + 1.0


def test_fibonacci_closed_forms():
    fib = [1, 1]
    while len(fib) < 34:
        fib.append(fib[-1] + fib[-2])
    # F(1..33) on 33 symbols: a chain; the j-th most frequent gets j bits,
    # the two rarest 32 bits
    h = np.zeros(256, np.uint64)
    for i in range(33):
        h[10 + i] = fib[i]
    ln = oracle.huffman_lengths(h)
    got = [int(ln[10 + i]) for i in range(33)]
    assert got == [32, 32] + list(range(31, 0, -1))
    ln32, rounds = oracle.limited_lengths(h, 32)
    assert rounds == 0 and np.array_equal(ln32, ln)
    # F(1..34): the unlimited chain is 33 deep; the limit must cut it to 32
    h34 = np.zeros(256, np.uint64)
    for i in range(34):
        h34[10 + i] = fib[i]
    assert int(oracle.huffman_lengths(h34).max()) == 33
    lim, rounds = oracle.limited_lengths(h34, 32)
    assert int(lim.max()) <= 32 and rounds >= 1
    assert _kraft_units(lim) == 1 << 40


def test_uniform_and_single():
    h = np.full(256, 1000, np.uint64)
    assert (oracle.huffman_lengths(h) == 8).all()
    h1 = np.zeros(256, np.uint64)
    h1[0x7C] = 77
    ln = oracle.huffman_lengths(h1)
    assert ln[0x7C] == 1 and int(ln.sum()) == 1
    assert oracle.canonical_codes(ln)[0x7C] == 0


@pytest.mark.parametrize("seed", range(6))
def test_canonical_codes_prefix_free(seed):
    rng = np.random.default_rng(400 + seed)
    k = int(rng.integers(2, 60))
    h = np.zeros(256, np.uint64)
    h[rng.choice(256, k, replace=False)] = rng.geometric(0.2, k) ** 3
    ln = oracle.huffman_lengths(h)
    code = oracle.canonical_codes(ln)
    words = ["{:0{}b}".format(int(code[s]), int(ln[s])) for s in range(256) if ln[s]]
    for a in words:
        for b in words:
            if a is not b:
                assert not b.startswith(a)
    # codes of one length are consecutive values in symbol order
    for L in set(ln[ln > 0].tolist()):
        syms = [s for s in range(256) if ln[s] == L]
        assert [int(code[s]) for s in syms] == list(range(int(code[syms[0]]),
                                                         int(code[syms[0]]) + len(syms)))


# ------------------------------------------------ stream and auxiliary arrays

def _check_aux(enc, max_slices=4096, seed=0):
    """Gaps and block positions against the chunk-decode premise: a decoder
    started at slice s's gap yields exactly the codes that start inside slice s,
    and block_pos[b] counts the codes that start before block b.  Large tensors
    are checked on a sample of slices."""
    e, ln = enc.exponents, enc.lengths
    gaps, bp = enc.gaps, enc.block_pos
    assert int(gaps.max()) <= 31
    assert bp[0] == 0 and bp[-1] == enc.n and (np.diff(bp.astype(np.int64)) >= 0).all()
    starts = np.concatenate([[0], np.cumsum(ln[e].astype(np.int64))])[:-1]
    nslices = -(-enc.total_bits // 64)
    if nslices <= max_slices:
        sample = np.arange(nslices)
    else:
        rng = np.random.default_rng(seed)
        sample = np.unique(np.concatenate([[0, nslices - 1], np.arange(0, nslices, 64)[:64],
                                           rng.choice(nslices, max_slices, replace=False)]))
    total = 0
    for s in sample.tolist():
        got = oracle.decode_range(enc.stream, enc.total_bits, 64 * s + int(gaps[s]),
                                  min(64 * (s + 1), enc.total_bits), ln, 64)
        first = int(np.searchsorted(starts, 64 * s))
        assert np.array_equal(got, e[first:first + got.size])
        assert first + got.size == int(np.searchsorted(starts, 64 * (s + 1)))
        if s % 64 == 0:
            assert int(bp[s // 64]) == first
        total += got.size
    if nslices <= max_slices:
        assert total == enc.n
    assert (gaps[nslices:] == 0).all()


@pytest.mark.parametrize("kind,n", [("normal", 1), ("normal", 63), ("normal", 4097),
                                    ("normal", 20011), ("single", 5000), ("uniform", 3001),
                                    ("int8", 7777)])
def test_roundtrip_and_aux(kind, n):
    w = wl.random_small(n, 11 + n, kind)
    enc = oracle.encode(w)
    assert np.array_equal(oracle.decode_tensor(enc), w)
    _check_aux(enc)


def test_roundtrip_fibonacci_and_all_exponents():
    for w in (wl.fibonacci_exponents(33, 7, 1024, 16 * 1024).weights,
              wl.fibonacci_exponents(34, 8, 1024, 16 * 1024).weights,
              wl.all_exponents(9, 64, 1024).weights):
        enc = oracle.encode(w)
        assert int(enc.lengths.max()) <= 32
        assert np.array_equal(oracle.decode_tensor(enc), w)
        _check_aux(enc)


def test_exact_32_bit_codes_present():
    w = wl.fibonacci_exponents(33, 5002, 1024, 16384).weights
    enc = oracle.encode(w)
    assert int(enc.lengths.max()) == 32 and int((enc.lengths == 32).sum()) == 2


def test_pack_gaps_bit_layout():
    # fields 1, 31, 0, 17, 5 written LSB first, 5 bits each, laid out by hand:
    # bits 0-4 = 1,0,0,0,0   5-9 = 1,1,1,1,1   10-14 = 0,0,0,0,0
    # bits 15-19 = 1,0,0,0,1 20-24 = 1,0,1,0,0
    # byte0 = bits 0-7  = 1,0,0,0,0,1,1,1 -> 0xE1
    # byte1 = bits 8-15 = 1,1,0,0,0,0,0,1 -> 0x83
    # byte2 = bits 16-23 = 0,0,0,1,1,0,1,0 -> 0x58
    # byte3 = bit 24 = 0 -> 0x00
    gaps = np.array([1, 31, 0, 17, 5], np.uint32)
    packed = oracle.pack_gaps(gaps, 4)
    assert packed.tolist() == [0xE1, 0x83, 0x58, 0x00]


def test_bits_per_weight_band_linear_4096():
    """The pages' 10.8-11.1 bits/weight band on an 8-bit-exponent N(0, 0.02) matrix."""
    w = wl.linear_4096().weights
    e, _ = oracle.split_bf16(w)
    h = oracle.histogram(e)
    ln, _ = oracle.limited_lengths(h, 32)
    total = int((h * ln.astype(np.uint64)).sum())
    nb = -(-total // 4096)
    aux_bits = 5 * (64 * nb + 1) + 32 * (nb + 1)
    bpw = 8 + (total + aux_bits) / w.size
    H = oracle.entropy_bits(h)
    assert 2.4 < H < 2.7
    assert 10.6 < bpw < 11.1
