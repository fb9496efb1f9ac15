"""A CPU model of the decode kernel's per-wave algorithm, run on small inputs.

It mirrors the kernel step for step -- the multi-code count and decode tables
derived from the 8-bit table image, phase 1 with the bits after a lane's last
code forced to one, phase 2 with four-slot stores that leave stray bytes, the head rewrites, and
the BF16 join -- and checks the result against the original words.  A logic
error in the kernel's scheme shows up here without a GPU.
"""
import numpy as np
import pytest

import huffman_decode_amd as hd
from huffman_decode_amd import workloads as wl

COUNT_BITS = 11
DECODE_BITS = 11
MAX_SYMS = 4
STRAY = 0xEE  # value of the unfilled slots of a decode entry in this model


def _lookup8(lut, w, n_tables):
    e = int(lut[w & 0xFF])
    for lvl in range(1, 4):
        if not e & 0x8000:
            break
        t = e & 63
        t = t if t < n_tables else 0
        e = int(lut[t * 256 + ((w >> (8 * lvl)) & 0xFF)])
    return e


def _leaf_len(e):
    return ((e >> 8) & 31) + 1


def _tables(lut, n_tables, max_len):
    count_w = min(max_len - 1, COUNT_BITS)
    span = max(COUNT_BITS, DECODE_BITS)
    count_t = np.zeros(1 << COUNT_BITS, np.uint32)
    dec_t = []
    for i in range(1 << span):
        pos = k = cpos = ck = dpos = dk = 0
        syms = []
        for _ in range(span):
            e = _lookup8(lut, i >> pos, n_tables)
            ln = _leaf_len(e)
            if pos + ln > span:
                break
            if pos + ln <= count_w:
                cpos, ck = pos + ln, k + 1
            if pos + ln <= DECODE_BITS and k < MAX_SYMS:
                syms.append(e & 0xFF)
                dpos, dk = pos + ln, k + 1
            pos += ln
            k += 1
        if i < (1 << COUNT_BITS):
            count_t[i] = cpos | (ck << 16)
        if i < (1 << DECODE_BITS):
            dec_t.append((dpos, dk, syms + [STRAY] * (MAX_SYMS - len(syms))))
    return count_t, dec_t


def _window(bits, p, width=32):
    v = 0
    for j in range(width):
        if p + j < bits.size:
            v |= int(bits[p + j]) << j
    return v


def _model_block(enc, b, count_t, dec_t, lut):
    s = enc.sizes
    n_tables, max_len = enc.codebook.n_tables, enc.codebook.max_len
    bits = np.unpackbits(enc.stream, bitorder="little")
    gbits = np.unpackbits(enc.gaps, bitorder="little")
    stop_bit, total = int(s.last_start) + 1, int(s.total_bits)
    p0, p1 = int(enc.block_pos[b]), int(enc.block_pos[b + 1])
    base = p0 & ~7
    lanes = []
    for lane in range(64):
        g = 64 * b + lane
        gw = sum(int(gbits[5 * g + j]) << j for j in range(10))
        gap, gap_next = gw & 31, (gw >> 5) & 31
        rel = stop_bit - 64 * g
        lim = 0 if rel <= 0 else min(64, rel)
        end = total - 64 * g if 0 < rel <= 64 else 64 + gap_next
        # phase 1 on padded bits: ones from `end` on
        slice_bits = bits[64 * g: 64 * g + 96].copy()
        padded = slice_bits.copy()
        padded[max(0, end):] = 1
        cnt = 0
        if lim:
            pos = gap
            for half_stop in (min(end, 32), end):
                while pos < half_stop:
                    x = int(count_t[_window(padded, pos, COUNT_BITS)])
                    if x < 0x10000:
                        x = _leaf_len(_lookup8(lut, _window(slice_bits, pos), n_tables)) | 0x10000
                    pos += x & 0xFFFF
                    cnt += x >> 16
        lanes.append(dict(gap=gap, lim=lim, cnt=cnt, bits=slice_bits))
    counts = [ln["cnt"] for ln in lanes]
    assert sum(counts) == p1 - p0
    excl = np.concatenate([[0], np.cumsum(counts)])[:-1]
    tile = np.full(4096 + 64, 0x77, np.int32)

    # phase 2: each lane steps through its own codes while below its stop
    # (first to bit 32, then to its stop) and stores the four slots of every
    # entry; a code longer than the window stores the entry's slots, then its
    # symbol over slot 0.  Lanes run from last to first, so a lane's stray
    # bytes land after the next lane's own stores (the worst order).
    for lane in range(63, -1, -1):
        ln = lanes[lane]
        if not ln["lim"]:
            continue
        pos, at = ln["gap"], (p0 - base) + int(excl[lane])
        for half_stop in (min(ln["lim"], 32), ln["lim"]):
            while pos < half_stop:
                dpos, dk, syms = dec_t[_window(ln["bits"], pos, DECODE_BITS)]
                tile[at:at + 4] = syms
                if dk == 0:
                    e = _lookup8(lut, _window(ln["bits"], pos), n_tables)
                    tile[at] = e & 0xFF
                    dpos, dk = _leaf_len(e), 1
                pos += dpos
                at += dk

    def rewrite(ln, pos, cnt, at):
        need, done = min(3, cnt), 0
        while done < need:
            dpos, dk, syms = dec_t[_window(ln["bits"], pos, DECODE_BITS)]
            if dk == 0:
                e = _lookup8(lut, _window(ln["bits"], pos), n_tables)
                syms, dk, dpos = [e & 0xFF], 1, _leaf_len(e)
            for j in range(min(dk, 3)):
                if done + j < need:
                    tile[at + done + j] = syms[j]
            done += dk
            pos += dpos

    for lane, ln in enumerate(lanes):          # then every head rewrite
        if not ln["lim"]:
            continue
        rewrite(ln, ln["gap"], ln["cnt"], (p0 - base) + int(excl[lane]))
    ex = tile[p0 - base: p1 - base].astype(np.uint16)
    sm = enc.signmant[p0:p1].astype(np.uint16)
    return ((sm & 0x80) << 8) | (ex << 7) | (sm & 0x7F)


def _check(w, blocks=None):
    enc = hd.encode(w)
    lut = enc.luts.view(np.uint16)
    count_t, dec_t = _tables(lut, enc.codebook.n_tables, enc.codebook.max_len)
    nb = int(enc.sizes.n_blocks)
    for b in (range(nb) if blocks is None else blocks):
        p0, p1 = int(enc.block_pos[b]), int(enc.block_pos[b + 1])
        got = _model_block(enc, b, count_t, dec_t, lut)
        assert np.array_equal(got, w[p0:p1]), f"block {b}"


@pytest.mark.parametrize("kind,n,seed", [("normal", 9000, 1), ("normal", 4097, 7),
                                          ("uniform", 2000, 2), ("int8", 5000, 3),
                                          ("single", 700, 4)])
def test_model_small(kind, n, seed):
    _check(wl.random_small(n, seed, kind))


def test_model_all_exponents():
    _check(wl.all_exponents(5, 16, 512).weights, blocks=range(3))


def test_model_longest_codes():
    w = wl.fibonacci_exponents(33, 44, 1024, 16384).weights
    enc = hd.encode(w)
    e = (w >> 7) & 0xFF
    ln = enc.codebook.lengths
    starts = np.concatenate([[0], np.cumsum(ln[e].astype(np.int64))])
    idx = np.nonzero(ln[e] >= 30)[0][:3]
    _check(w, blocks=sorted({int(starts[i]) // 4096 for i in idx}))
