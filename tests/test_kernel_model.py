"""A CPU model of the decode kernel's per-wave algorithm, run on small inputs.

It mirrors the kernel step for step and checks the joined BF16 words against
the originals, so a logic error in the kernel's scheme shows up without a GPU:

* the multi-code decode table derived from the 8-bit table image (window
  narrower than the longest code, at most four symbols per entry);
* phase 1 on the slice bits with everything after the lane's last code forced
  to one: every step stores four symbol bytes into the lane's private staging
  slot (stray bytes included), and the step count gives the exact code count;
* the wave scan and, when every lane holds 3 to 32 codes (56 in the wide
  geometry for streams of short codes) or is past the block's last code, the
  placement: each lane writes the aligned tile dwords that end inside its own
  output bytes, the first one completed with the previous lane's last bytes,
  the lane holding the block's last code also its final partial dword; every
  tile dword is written exactly once;
* otherwise the fallback: phase 2 decodes the real bits again straight into
  the tile, then every lane's first symbols are decoded and stored again.
"""
import numpy as np
import pytest

import huffman_decode_amd as hd
from huffman_decode_amd import workloads as wl

DECODE_BITS = 11
MAX_SYMS = 4
STAGE_BASE = 4         # lane t's slot starts at byte 4 + stride t of the region
MIN_CODES = 3          # fewer (before the block's last code) also does
# staging geometries: codes a lane may stage (more sends the wave to the
# fallback), bytes of staging per lane, LDS bytes per wave (staging and tile
# share them), exponent bytes one tile holds.  The kernel stages 32 codes per
# lane, and 56 for streams whose codes average under 2.51 bits.
NARROW = dict(codes=32, stride=40, region=2600, cap=2560)
WIDE = dict(codes=56, stride=60, region=3856, cap=3816)
TILE_CAP = NARROW["cap"]
STRAY = 0xEE           # value of the unfilled slots of a decode entry in this model


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


def _table(lut, n_tables, max_len):
    width = min(max_len - 1, DECODE_BITS)
    dec_t = []
    for i in range(1 << DECODE_BITS):
        pos = k = 0
        syms = []
        while k < MAX_SYMS:
            e = _lookup8(lut, i >> pos, n_tables)
            ln = _leaf_len(e)
            if pos + ln > width:
                break
            syms.append(e & 0xFF)
            pos += ln
            k += 1
        dec_t.append((pos, k, syms + [STRAY] * (MAX_SYMS - len(syms))))
    return dec_t


def _window(bits, p, width=32):
    v = 0
    for j in range(width):
        if p + j < bits.size:
            v |= int(bits[p + j]) << j
    return v


def _walk(ln, bits, dec_t, lut, n_tables, mem, at):
    """Step through the lane's codes starting below its limit, storing four
    bytes per table step at mem[at...]; returns the number of codes."""
    pos, k = ln["gap"], 0
    for half_stop in (min(ln["lim"], 32), ln["lim"]):
        while pos < half_stop:
            dpos, dk, syms = dec_t[_window(bits, pos, DECODE_BITS)]
            mem[at + k:at + k + 4] = syms
            if dk == 0:  # longer than the window: the 8-bit tables, real bits
                e = _lookup8(lut, _window(ln["bits"], pos), n_tables)
                mem[at + k] = e & 0xFF
                dpos, dk = _leaf_len(e), 1
            pos += dpos
            k += dk
    return k


def _model_block(enc, b, dec_t, lut, geo=NARROW):
    s = enc.sizes
    n_tables = enc.codebook.n_tables
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
        slice_bits = bits[64 * g: 64 * g + 96].copy()
        padded = slice_bits.copy()
        padded[max(0, end):] = 1
        lanes.append(dict(gap=gap, lim=lim, bits=slice_bits, padded=padded))

    # the wave's LDS region; garbage to start with
    mem = np.full(geo["region"] + 8, 0x77, np.int32)
    # phase 1 in lane order 63..0 so that overflowing lanes' stores land last
    for lane in range(63, -1, -1):
        ln = lanes[lane]
        slot = STAGE_BASE + geo["stride"] * lane
        ln["cnt"] = _walk(ln, ln["padded"], dec_t, lut, n_tables, mem, slot) if ln["lim"] else 0
    counts = [ln["cnt"] for ln in lanes]
    assert sum(counts) == p1 - p0
    incl = np.cumsum(counts)
    excl = incl - counts
    total = int(incl[-1])
    groups = (p1 - base + 7) >> 3
    bad = [c > geo["codes"] or (c < MIN_CODES and incl[l] != total) for l, c in enumerate(counts)]

    if not any(bad) and groups * 8 + 4 <= geo["cap"]:
        # every lane reads its codes / 4 staged dwords and the 4 bytes ending at its
        # last code (from its slot, before anything is written)
        staged, tail4 = [], []
        for lane in range(64):
            slot = STAGE_BASE + geo["stride"] * lane
            staged.append([int(x) for x in mem[slot: slot + geo["codes"]]] + [0, 0, 0, 0])
            b = counts[lane] - 4
            tail4.append([int(x) for x in mem[slot + b: slot + b + 4]])
        written = np.zeros(mem.size, bool)
        for lane in range(64):
            cnt = counts[lane]
            e = (p0 - base) + int(excl[lane])
            sft, a0 = e & 3, e & ~3
            prev = tail4[(lane - 1) % 64]
            ext = prev + staged[lane]                   # byte -4.. of the lane's sequence
            j_full = ((sft + cnt) >> 2) - 1
            if cnt == 0:
                last = -1                              # past the block's last code
            elif incl[lane] == total:
                last = (sft + cnt - 1) >> 2            # holds the last code: partial dword too
            else:
                last = j_full
            for j in range(0, last + 1):
                for t in range(4):
                    at = a0 + 4 * j + t
                    assert not written[at], "tile byte written twice"
                    written[at] = True
                    mem[at] = ext[4 + 4 * j + t - sft]
    else:
        # fallback: decode the real bits again into the tile, then restore heads
        for lane in range(63, -1, -1):
            ln = lanes[lane]
            if ln["lim"]:
                _walk(ln, ln["bits"], dec_t, lut, n_tables, mem, (p0 - base) + int(excl[lane]))
        for lane in range(64):
            ln = lanes[lane]
            if not ln["lim"]:
                continue
            head = np.zeros(64 + 8, np.int32)
            _walk(ln, ln["bits"], dec_t, lut, n_tables, head, 0)
            at = (p0 - base) + int(excl[lane])
            for j in range(min(3, counts[lane])):
                mem[at + j] = head[j]
    ex = mem[p0 - base: p1 - base].astype(np.uint16)
    sm = enc.signmant[p0:p1].astype(np.uint16)
    return ((sm & 0x80) << 8) | (ex << 7) | (sm & 0x7F), any(bad)


def _check(w, blocks=None, geo=NARROW):
    enc = hd.encode(w)
    lut = enc.luts.view(np.uint16)
    dec_t = _table(lut, enc.codebook.n_tables, enc.codebook.max_len)
    nb = int(enc.sizes.n_blocks)
    fallbacks = 0
    for b in (range(nb) if blocks is None else blocks):
        p0, p1 = int(enc.block_pos[b]), int(enc.block_pos[b + 1])
        if p1 - p0 > geo["cap"] - 16:
            continue  # multi-pass blocks: checked on the GPU only
        got, fell_back = _model_block(enc, b, dec_t, lut, geo)
        fallbacks += fell_back
        assert np.array_equal(got, w[p0:p1]), f"block {b}"
    return fallbacks


@pytest.mark.parametrize("kind,n,seed", [("normal", 9000, 1), ("normal", 4097, 7),
                                          ("uniform", 2000, 2), ("int8", 5000, 3)])
def test_model_small(kind, n, seed):
    assert _check(wl.random_small(n, seed, kind)) == 0


def test_model_fallback_on_short_codes():
    # two symbols, one far more frequent: 1- and 2-bit codes overflow the staging
    rng = np.random.default_rng(11)
    e = np.where(rng.random(6000) < 0.9, 126, 125).astype(np.uint16)
    low = rng.integers(0, 256, e.size, dtype=np.uint16)
    w = (((low & 0x80) << 8) | (e << 7) | (low & 0x7F)).astype(np.uint16)
    assert _check(w) > 0


@pytest.mark.parametrize("kind,n,seed", [("geometric", 30_000, 21), ("geometric_steep", 30_000, 22),
                                          ("normal", 9000, 23)])
def test_model_wide_slots(kind, n, seed):
    """The 56-code slots: streams of 1.4-2 bit codes (30-45 codes per slice)
    stage every block that the 32-code slots send to the fallback, and
    ordinary weights decode the same way in either geometry."""
    w = wl.random_small(n, seed, kind)
    wide = _check(w, geo=WIDE)
    if kind == "geometric":
        assert _check(w) > 0 and wide == 0
    if kind == "normal":
        assert wide == 0


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


@pytest.mark.parametrize("kind", ["normal", "uniform", "single", "fibonacci_33"])
def test_host_decode_table_matches_model(kind):
    """The table image ends with the multi-code decode table that the kernel
    copies to LDS (built by the host library).  Every entry must be the
    model's: total length | code count << 16, then the symbols, each rotated
    right by one bit (the form the kernel joins), unused bytes 0.
    The cases cover short codes, a flat code, the one-symbol code (no code
    fits the window, every entry is empty) and codes up to 32 bits."""
    if kind == "fibonacci_33":
        w = wl.fibonacci_exponents(33, 5002, 1024, 16384).weights
    else:
        w = wl.random_small({"normal": 100_000, "uniform": 50_000, "single": 4096}[kind], 3, kind)
    enc = hd.encode(w)
    n_tables = enc.codebook.n_tables
    lut = enc.luts.view(np.uint16)
    tail = enc.luts[n_tables * 512:].view(np.uint32)
    assert tail.size == 2 * (1 << DECODE_BITS)
    rotr8 = lambda e: ((e >> 1) | (e << 7)) & 0xFF  # the kernel's form of an exponent byte
    for i, (pos, k, syms) in enumerate(_table(lut, n_tables, enc.codebook.max_len)):
        packed = sum(rotr8(int(s)) << (8 * j) for j, s in enumerate(syms[:k]))
        assert int(tail[2 * i]) == pos | (k << 16), (kind, i)
        assert int(tail[2 * i + 1]) == packed, (kind, i)


def _pad_ones(d, end, base):
    keep = end - base
    if keep >= 32:
        return d
    if keep <= 0:
        return 0xFFFFFFFF
    return (d | (0xFFFFFFFF << keep)) & 0xFFFFFFFF


@pytest.mark.parametrize("stop_at", [4097, 4096 + 4095, 1 << 30])
def test_block_before_stop_needs_only_third_dword_padded(stop_at):
    """The kernel's shortcut for a block wholly before the stop bit (every lane
    lim = 64, end = 64 + next gap) equals the per-lane limits and padding."""
    rng = np.random.default_rng(stop_at & 0xFFFF)
    for lane in range(64):
        rel = stop_at - 64 * lane
        for gap_next in range(32):
            d = [int(v) for v in rng.integers(0, 1 << 32, 3, dtype=np.uint64)]
            assert rel > 64  # so the per-lane rule takes end = 64 + gap_next
            lim, end = min(64, rel), 64 + gap_next
            general = (lim, _pad_ones(d[0], end, 0), _pad_ones(d[1], end, 32),
                       _pad_ones(d[2], end, 64))
            shortcut = (64, d[0], d[1], (d[2] | (0xFFFFFFFF << gap_next)) & 0xFFFFFFFF)
            assert general == shortcut
