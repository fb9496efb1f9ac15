"""CPU oracle for the DFloat11 (DF11) exponent codec.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the product package ``huffman_decode_amd`` and never imports it.

The arithmetic lives in ``df11_oracle.c`` (bit-at-a-time C, built with gcc into
``libdf11_oracle.so``).  This module marshals numpy arrays into it and adds the
few statistics that are plain numpy: Shannon entropy and average code length.

Page followed throughout: "DFloat11: lossless BFloat16 compression"
(ai-infrastructure.net), sections "What it is", "Architecture" and
"How it works: the core algorithm".  The packed layout of the encoded arrays
(bit order, slice and block sizes, 5-bit gap fields) is a reading of that page,
stated in ``df11_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "df11_oracle.c")
_SO = os.path.join(_HERE, "libdf11_oracle.so")

SLICE_BITS = 64          # one 8-byte slice per lane
BLOCK_SLICES = 64        # slices per block
BLOCK_BITS = SLICE_BITS * BLOCK_SLICES
STREAM_GUARD = 16        # zero bytes after the last block

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C11, no GPU code)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared",
                               "-fPIC", "-o", tmp, _SRC])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        U64 = ctypes.c_uint64
        U32 = ctypes.c_uint32
        lib.orc_split.argtypes = [P, U64, P, P]
        lib.orc_join.argtypes = [P, P, U64, P]
        lib.orc_histogram.argtypes = [P, U64, P]
        lib.orc_huffman_lengths.argtypes = [P, P]
        lib.orc_limited_lengths.argtypes = [P, U32, P, P]
        lib.orc_canonical_codes.argtypes = [P, P]
        lib.orc_encode.argtypes = [P, U64, P, P, U64]
        lib.orc_encode.restype = ctypes.c_int64
        lib.orc_decode.argtypes = [P, U64, U64, U64, P, P, P]
        lib.orc_decode_range.argtypes = [P, U64, U64, U64, P, P, U64]
        lib.orc_decode_range.restype = ctypes.c_int64
        lib.orc_aux.argtypes = [P, U64, P, P, U64, P, U64]
        lib.orc_pack_gaps.argtypes = [P, U64, P, U64]
        lib.orc_count_subtables.argtypes = [P, U32]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _check(status: int, what: str) -> int:
    if status < 0:
        raise RuntimeError(f"oracle {what} failed with status {status}")
    return status


# ----------------------------------------------------------------- fields

def split_bf16(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """BF16 bit patterns -> (exponent bytes, sign|mantissa bytes)."""
    w = np.ascontiguousarray(w, dtype=np.uint16)
    e = np.empty(w.size, np.uint8)
    sm = np.empty(w.size, np.uint8)
    _check(_load().orc_split(_ptr(w), w.size, _ptr(e), _ptr(sm)), "split")
    return e, sm


def join_bf16(e: np.ndarray, sm: np.ndarray) -> np.ndarray:
    e = np.ascontiguousarray(e, dtype=np.uint8)
    sm = np.ascontiguousarray(sm, dtype=np.uint8)
    assert e.size == sm.size
    w = np.empty(e.size, np.uint16)
    _check(_load().orc_join(_ptr(e), _ptr(sm), e.size, _ptr(w)), "join")
    return w


def histogram(e: np.ndarray) -> np.ndarray:
    e = np.ascontiguousarray(e, dtype=np.uint8)
    h = np.zeros(256, np.uint64)
    _check(_load().orc_histogram(_ptr(e), e.size, _ptr(h)), "histogram")
    return h


# ------------------------------------------------------------- statistics

def entropy_bits(counts: np.ndarray) -> float:
    """Shannon entropy in bits of a histogram (zero bins contribute nothing)."""
    c = np.asarray(counts, dtype=np.float64)
    p = c[c > 0] / c.sum()
    return float(-(p * np.log2(p)).sum())


def average_length(counts: np.ndarray, lengths: np.ndarray) -> float:
    c = np.asarray(counts, dtype=np.float64)
    return float((c * np.asarray(lengths, dtype=np.float64)).sum() / c.sum())


# ---------------------------------------------------------------- lengths

def huffman_lengths(hist: np.ndarray) -> np.ndarray:
    """Unlimited Huffman code lengths (0 = symbol absent)."""
    h = np.ascontiguousarray(hist, dtype=np.uint64)
    assert h.size == 256
    ln = np.zeros(256, np.uint8)
    _check(_load().orc_huffman_lengths(_ptr(h), _ptr(ln)), "huffman")
    return ln


def limited_lengths(hist: np.ndarray, max_len: int = 32) -> tuple[np.ndarray, int]:
    """Huffman lengths with the count-halving length limit; returns (lengths, rounds)."""
    h = np.ascontiguousarray(hist, dtype=np.uint64)
    ln = np.zeros(256, np.uint8)
    rounds = ctypes.c_uint32(0)
    _check(_load().orc_limited_lengths(_ptr(h), max_len, _ptr(ln), ctypes.addressof(rounds)),
           "limited lengths")
    return ln, int(rounds.value)


def canonical_codes(lengths: np.ndarray) -> np.ndarray:
    ln = np.ascontiguousarray(lengths, dtype=np.uint8)
    code = np.zeros(256, np.uint32)
    _check(_load().orc_canonical_codes(_ptr(ln), _ptr(code)), "canonical codes")
    return code


def count_subtables(lengths: np.ndarray, chunk: int = 8) -> int:
    ln = np.ascontiguousarray(lengths, dtype=np.uint8)
    return _check(_load().orc_count_subtables(_ptr(ln), chunk), "subtables")


# ------------------------------------------------------- encode / decode

def encode_bits(e: np.ndarray, lengths: np.ndarray, cap_bytes: int | None = None
                ) -> tuple[np.ndarray, int]:
    """Packed stream (zero-filled to cap_bytes) and its length in bits."""
    e = np.ascontiguousarray(e, dtype=np.uint8)
    ln = np.ascontiguousarray(lengths, dtype=np.uint8)
    if cap_bytes is None:
        total = int((histogram(e).astype(np.uint64) * ln.astype(np.uint64)).sum())
        cap_bytes = (total + 7) // 8 + 8
    stream = np.zeros(cap_bytes, np.uint8)
    bits = _load().orc_encode(_ptr(e), e.size, _ptr(ln), _ptr(stream), cap_bytes)
    _check(bits, "encode")
    return stream, int(bits)


def decode(stream: np.ndarray, avail_bits: int, start_bit: int, count: int,
           lengths: np.ndarray) -> tuple[np.ndarray, int]:
    """Exactly `count` symbols from start_bit (bits past avail_bits read as 0)."""
    stream = np.ascontiguousarray(stream, dtype=np.uint8)
    ln = np.ascontiguousarray(lengths, dtype=np.uint8)
    out = np.zeros(max(count, 1), np.uint8)
    end = ctypes.c_uint64(0)
    _check(_load().orc_decode(_ptr(stream), avail_bits, start_bit, count, _ptr(ln), _ptr(out),
                              ctypes.addressof(end)), "decode")
    return out[:count], int(end.value)


def decode_range(stream: np.ndarray, avail_bits: int, start_bit: int, stop_bit: int,
                 lengths: np.ndarray, cap: int) -> np.ndarray:
    """Symbols of every code starting in [start_bit, stop_bit)."""
    stream = np.ascontiguousarray(stream, dtype=np.uint8)
    ln = np.ascontiguousarray(lengths, dtype=np.uint8)
    out = np.zeros(max(cap, 1), np.uint8)
    k = _load().orc_decode_range(_ptr(stream), avail_bits, start_bit, stop_bit, _ptr(ln),
                                 _ptr(out), cap)
    _check(k, "decode range")
    return out[:k]


def aux(e: np.ndarray, lengths: np.ndarray, n_gaps: int, n_bp: int
        ) -> tuple[np.ndarray, np.ndarray]:
    """(gaps, block_pos) by definition; gaps unpacked, one uint32 per slice."""
    e = np.ascontiguousarray(e, dtype=np.uint8)
    ln = np.ascontiguousarray(lengths, dtype=np.uint8)
    gaps = np.zeros(n_gaps, np.uint32)
    bp = np.zeros(n_bp, np.uint32)
    _check(_load().orc_aux(_ptr(e), e.size, _ptr(ln), _ptr(gaps), n_gaps, _ptr(bp), n_bp), "aux")
    return gaps, bp


def pack_gaps(gaps: np.ndarray, cap: int) -> np.ndarray:
    g = np.ascontiguousarray(gaps, dtype=np.uint32)
    out = np.zeros(cap, np.uint8)
    _check(_load().orc_pack_gaps(_ptr(g), g.size, _ptr(out), cap), "pack gaps")
    return out


@dataclass
class Encoded:
    """Every array of the DF11 format for one BF16 tensor, computed by the oracle."""
    n: int
    lengths: np.ndarray      # uint8[256]
    total_bits: int
    n_blocks: int
    stream: np.ndarray       # uint8, n_blocks*512 + guard bytes, zero padded
    gaps: np.ndarray         # uint32, one per slice plus one (unpacked)
    block_pos: np.ndarray    # uint32[n_blocks + 1]
    signmant: np.ndarray     # uint8[n]
    exponents: np.ndarray    # uint8[n]


def encode(w: np.ndarray, max_len: int = 32) -> Encoded:
    """Full DF11 encoding of a flat BF16 tensor (bit patterns as uint16)."""
    e, sm = split_bf16(w)
    hist = histogram(e)
    lengths, _ = limited_lengths(hist, max_len)
    total = int((hist * lengths.astype(np.uint64)).sum())
    n_blocks = max(1, -(-total // BLOCK_BITS))
    stream, bits = encode_bits(e, lengths, n_blocks * BLOCK_BITS // 8 + STREAM_GUARD)
    assert bits == total
    gaps, bp = aux(e, lengths, n_blocks * BLOCK_SLICES + 1, n_blocks + 1)
    return Encoded(n=int(w.size), lengths=lengths, total_bits=total, n_blocks=n_blocks,
                   stream=stream, gaps=gaps, block_pos=bp, signmant=sm, exponents=e)


def decode_tensor(enc: Encoded) -> np.ndarray:
    """Serial bit-by-bit decode of the whole stream, joined back to BF16."""
    ex, end = decode(enc.stream, enc.total_bits, 0, enc.n, enc.lengths)
    if end != enc.total_bits:
        raise RuntimeError("decode did not end on the stream's last bit")
    return join_bf16(ex, enc.signmant)
