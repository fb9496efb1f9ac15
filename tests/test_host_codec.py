"""Host codec and C-ABI checks that need no GPU.

The host encoder (libdf11) must produce exactly the arrays the oracle computes
from the format's definitions; its device table image must decode the stream
when walked the way the kernel walks it (a Python model of one wave, below).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import huffman_decode_amd as hd
from huffman_decode_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _built():
    if not os.path.exists(hd.LIB_PATH):
        from huffman_decode_amd.build import build_library
        build_library()
    oracle.build()


def test_library_exports_every_declared_symbol():
    text = open(os.path.join(ROOT, "include", "df11.h")).read()
    declared = set(re.findall(r"\b(df11_\w+)\s*\(", text))
    assert {"df11_decode", "df11_encode", "df11_build_codebook", "df11_histogram",
            "df11_encoded_sizes", "df11_build_luts", "df11_status_string"} <= declared
    lib = ctypes.CDLL(hd.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def _inputs():
    yield "normal_small", wl.random_small(5000, 1, "normal")
    yield "normal_ragged", wl.random_small(77_777, 2, "normal")
    yield "single", wl.random_small(3000, 3, "single")
    yield "uniform", wl.random_small(50_000, 4, "uniform")
    yield "int8", wl.random_small(40_000, 5, "int8")
    yield "one", wl.random_small(1, 6, "normal")
    yield "all_exponents", wl.all_exponents(7, 64, 512).weights
    yield "flux_small", wl.flux_block(8, scale=1 / 256).weights


@pytest.mark.parametrize("name,w", list(_inputs()))
def test_encode_matches_oracle(name, w):
    enc = hd.encode(w)
    ref = oracle.encode(w)
    cb = enc.codebook
    assert np.array_equal(cb.lengths, ref.lengths)
    assert np.array_equal(cb.codes, oracle.canonical_codes(ref.lengths))
    assert cb.n_tables == oracle.count_subtables(ref.lengths, 8)
    sz = enc.sizes
    assert sz.total_bits == ref.total_bits and sz.n_blocks == ref.n_blocks
    assert np.array_equal(enc.stream, ref.stream)
    assert np.array_equal(enc.block_pos, ref.block_pos)
    gaps_ref = oracle.pack_gaps(ref.gaps, enc.gaps.size)
    assert np.array_equal(enc.gaps, gaps_ref)
    assert np.array_equal(enc.signmant[:ref.n], ref.signmant)
    assert not enc.signmant[ref.n:].any()
    last_len = int(ref.lengths[ref.exponents[-1]])
    assert sz.last_start == ref.total_bits - last_len
    # the oracle decodes the product's stream back to the original words
    ex, end = oracle.decode(enc.stream, int(sz.total_bits), 0, ref.n, cb.lengths)
    assert end == sz.total_bits
    assert np.array_equal(oracle.join_bf16(ex, enc.signmant[:ref.n]), w)


def test_length_limit_agrees_with_oracle():
    for k, seed in ((33, 11), (34, 12)):
        w = wl.fibonacci_exponents(k, seed, 1024, 16384).weights
        hist = hd.df11_histogram(w)
        cb = hd.df11_build_codebook(hist, 32)
        ref, rounds = oracle.limited_lengths(hist, 32)
        assert np.array_equal(cb.lengths, ref) and cb.limit_rounds == rounds
        # 33 Fibonacci counts reach exactly 32 bits unlimited; 34 need one halving
        assert (cb.max_len, cb.limit_rounds) == ((32, 0) if k == 33 else (int(ref.max()), 1))


@pytest.mark.parametrize("limit", [8, 10, 12, 16])
def test_tighter_limits_agree_with_oracle(limit):
    w = wl.flux_block(21, scale=1 / 128).weights
    hist = hd.df11_histogram(w)
    cb = hd.df11_build_codebook(hist, limit)
    ref, rounds = oracle.limited_lengths(hist, limit)
    assert np.array_equal(cb.lengths, ref) and cb.limit_rounds == rounds


def test_thread_count_does_not_change_output():
    w = wl.random_small(1_500_001, 9, "normal")
    a = hd.encode(w, n_threads=1)
    b = hd.encode(w, n_threads=7)
    c = hd.encode(w, n_threads=64)
    for x in (b, c):
        assert np.array_equal(a.stream, x.stream)
        assert np.array_equal(a.gaps, x.gaps)
        assert np.array_equal(a.block_pos, x.block_pos)
        assert np.array_equal(a.signmant, x.signmant)


def test_error_codes():
    lib = hd.library()
    hist = np.zeros(256, np.uint64)
    cb = hd.Codebook()
    assert lib.df11_build_codebook(hist.ctypes.data, 32, ctypes.byref(cb)) == -1  # empty
    hist[:] = 1
    assert lib.df11_build_codebook(hist.ctypes.data, 7, ctypes.byref(cb)) == -3  # 256 syms in 7 bits
    assert lib.df11_build_codebook(hist.ctypes.data, 33, ctypes.byref(cb)) == -3
    assert lib.df11_build_codebook(hist.ctypes.data, 8, ctypes.byref(cb)) == 0
    sz = hd.Sizes()
    assert lib.df11_encoded_sizes(hist.ctypes.data, 255, ctypes.byref(cb), ctypes.byref(sz)) == -5
    assert lib.df11_encoded_sizes(hist.ctypes.data, 0, ctypes.byref(cb), ctypes.byref(sz)) == -1
    # a weight whose exponent has no code
    w = wl.random_small(1000, 1, "single")
    cb1 = hd.df11_build_codebook(hd.df11_histogram(w))
    with pytest.raises(hd.Df11Error):
        hd.df11_encode(wl.random_small(1000, 2, "normal"), cb1,
                       hist=hd.df11_histogram(w))
    # too-small buffers
    w = wl.random_small(10_000, 3, "normal")
    h = hd.df11_histogram(w)
    cb = hd.df11_build_codebook(h)
    sz = hd.df11_encoded_sizes(h, w.size, cb)
    buf = np.zeros(sz.stream_bytes, np.uint8)
    g = np.zeros(sz.gaps_bytes, np.uint8)
    bp = np.zeros(sz.block_pos_count, np.uint32)
    sm = np.zeros(sz.signmant_bytes, np.uint8)
    out = hd.Sizes()
    st = lib.df11_encode(w.ctypes.data, w.size, ctypes.byref(cb), buf.ctypes.data, buf.size - 1,
                         g.ctypes.data, g.size, bp.ctypes.data, bp.size, sm.ctypes.data, sm.size,
                         ctypes.byref(out), 0)
    assert st == -2
    # decode descriptor checks happen before any device call
    d = hd.DeviceStream()
    assert lib.df11_decode(ctypes.byref(d), None, None) == -1
    assert lib.df11_decode(None, None, None) == -1


def test_decode_rejects_inconsistent_descriptor_on_host():
    lib = hd.library()
    w = wl.random_small(10_000, 3, "normal")
    enc = hd.encode(w)
    sz = enc.sizes
    d = hd.DeviceStream()
    fake = 1 << 20  # aligned non-null addresses; the checks fail before any use
    d.stream = d.gaps = d.block_pos = d.signmant = d.luts = fake
    d.stream_bytes, d.gaps_bytes = sz.stream_bytes, sz.gaps_bytes
    d.block_pos_count, d.signmant_bytes, d.lut_bytes = sz.block_pos_count, sz.signmant_bytes, \
        sz.lut_bytes
    d.n, d.total_bits, d.last_start = sz.n, sz.total_bits, sz.last_start
    d.n_blocks, d.n_tables, d.max_len = sz.n_blocks, enc.codebook.n_tables, enc.codebook.max_len
    for field, value, want in (("max_len", 0, -5), ("max_len", 33, -5), ("n_blocks", sz.n_blocks + 1, -5), ("total_bits", sz.n - 1, -5),
                               ("last_start", sz.total_bits, -5), ("stream_bytes", 100, -2),
                               ("gaps_bytes", 8, -2), ("n_tables", 0, -4),
                               ("n_tables", 65, -4), ("n", 0, -1)):
        saved = getattr(d, field)
        setattr(d, field, value)
        assert lib.df11_decode(ctypes.byref(d), fake, None) == want, field
        setattr(d, field, saved)
    assert lib.df11_decode(ctypes.byref(d), fake + 2, None) == -1  # misaligned output


# ---------------------------------------------------------------------------
# A Python model of one wave of the decode kernel: per lane, codes that start
# in [gap, min(64, stop - 64g)) of its slice, read from LSB-first windows via
# the table image; wave prefix sum; merge into BF16.  It checks the table
# image and the slice/limit arithmetic the kernel relies on.

@pytest.mark.parametrize("name,w", [
    ("normal", wl.random_small(9000, 31, "normal")),
    ("single", wl.random_small(700, 32, "single")),
    ("uniform", wl.random_small(1500, 33, "uniform")),
])
def test_kernel_model_decodes_table_image(name, w):
    enc = hd.encode(w)
    got = _model_blocks(enc, range(int(enc.sizes.n_blocks)))
    assert np.array_equal(np.concatenate([got[b] for b in sorted(got)]), w)


@pytest.mark.parametrize("k", [33, 34])
def test_kernel_model_on_longest_codes(k):
    """Blocks holding the longest codes (32 bits for 33 Fibonacci counts)."""
    w = wl.fibonacci_exponents(k, 40 + k, 1024, 16384).weights
    enc = hd.encode(w)
    e, _ = oracle.split_bf16(w)
    ln = enc.codebook.lengths
    idx = np.nonzero(ln[e] == ln.max())[0][:4]
    starts = np.concatenate([[0], np.cumsum(ln[e].astype(np.int64))])
    blocks = sorted({int(starts[i]) // 4096 for i in idx} | {int(enc.sizes.n_blocks) - 1})
    got = _model_blocks(enc, blocks)
    for b, vals in got.items():
        p0, p1 = int(enc.block_pos[b]), int(enc.block_pos[b + 1])
        assert np.array_equal(vals, w[p0:p1])


def _model_blocks(enc, blocks):
    s = enc.sizes
    lut = enc.luts.view(np.uint16)
    bits = np.unpackbits(enc.stream, bitorder="little")
    gaps_bits = np.unpackbits(enc.gaps, bitorder="little")
    stop = int(s.last_start) + 1
    res = {}
    for b in blocks:
        syms = []
        for lane in range(64):
            g = 64 * b + lane
            gap = int(sum(int(gaps_bits[5 * g + j]) << j for j in range(5)))
            lim = max(0, min(64, stop - 64 * g))
            pos = gap
            while pos < lim:
                p = 64 * g + pos
                w = int(sum(int(bits[p + j]) << j for j in range(32)))
                e = int(lut[w & 0xFF])
                lvl = 1
                while e & 0x8000 and lvl < 4:
                    e = int(lut[(e & 63) * 256 + ((w >> (8 * lvl)) & 0xFF)])
                    lvl += 1
                syms.append(e & 0xFF)
                pos += ((e >> 8) & 31) + 1
        p0, p1 = int(enc.block_pos[b]), int(enc.block_pos[b + 1])
        assert len(syms) == p1 - p0
        ex = np.array(syms, np.uint16)
        smb = enc.signmant[p0:p1].astype(np.uint16)
        res[b] = ((smb & 0x80) << 8) | (ex << 7) | (smb & 0x7F)
    return res


def test_decode_gemv_rejects_bad_matrix_lists_on_host():
    """The fused GEMV checks its matrix list before any device call."""
    lib = hd.library()
    w = wl.random_small(3 * 4096 * 8, 5, "normal")
    enc = hd.encode(w)
    sz = enc.sizes
    d = hd.DeviceStream()
    fake = 1 << 20
    d.stream = d.gaps = d.block_pos = d.signmant = d.luts = fake
    d.stream_bytes, d.gaps_bytes = sz.stream_bytes, sz.gaps_bytes
    d.block_pos_count, d.signmant_bytes, d.lut_bytes = sz.block_pos_count, sz.signmant_bytes, \
        sz.lut_bytes
    d.n, d.total_bits, d.last_start = sz.n, sz.total_bits, sz.last_start
    d.n_blocks, d.n_tables, d.max_len = sz.n_blocks, enc.codebook.n_tables, enc.codebook.max_len
    # per block 16 bytes of partial sums, then one word per possible row
    # (rows hold at least 2048 weights) and one more
    rows_words = 4 * (sz.n // 2048 + 1)
    assert lib.df11_gemv_workspace_bytes(ctypes.byref(d)) == 16 * sz.n_blocks + rows_words
    ws = 16 * sz.n_blocks + rows_words

    def call(shapes, x=fake, wsb=ws, mats=None):
        mats = mats if mats is not None else hd.gemv_matrices(shapes)[0]
        arr = (hd.GemvMatrix * len(mats))(*mats)
        return lib.df11_decode_gemv(ctypes.byref(d), arr, len(mats), x, fake, fake, wsb, None)

    assert call([(24, 4096)], wsb=ws - 16) == -2          # workspace too small
    assert call([(24, 4096)], x=fake + 4) == -1           # x not 16-byte aligned
    assert call([(48, 2048), (1, 0)]) == -1                # empty matrix
    assert call([(96, 1024)]) == -1                        # rows shorter than 2048
    assert call([(23, 4096)]) == -1                        # does not cover all weights
    assert call([(12, 4100), (12, 4092)]) == -1            # cols not a multiple of 8
    mats, _, _ = hd.gemv_matrices([(12, 4096), (12, 4096)])
    mats[1].offset += 8
    assert call(None, mats=mats) == -1                     # gap between matrices
    mats, _, _ = hd.gemv_matrices([(12, 4096), (12, 4096)])
    mats[1].x_offset += 4
    assert call(None, mats=mats) == -1                     # x slice not 8-aligned
    assert call([(1, 4096)] * 17 + [(7, 4096)]) == -1      # more than 16 matrices

    # several input vectors: batch range, strides, workspace per batch capacity
    shapes = [(24, 4096)]
    mats = hd.gemv_matrices(shapes)[0]
    arr = (hd.GemvMatrix * 1)(*mats)
    for batch, floats in ((1, 4), (2, 8), (3, 16), (4, 16), (5, 28), (8, 28)):
        assert lib.df11_gemm_workspace_bytes(ctypes.byref(d), batch) == \
            4 * floats * sz.n_blocks + rows_words
    assert lib.df11_gemm_workspace_bytes(ctypes.byref(d), 0) == 0
    assert lib.df11_gemm_workspace_bytes(ctypes.byref(d), 9) == 0

    def gemm(batch, xs=4096, ys=24, wsb=None):
        wsb = lib.df11_gemm_workspace_bytes(ctypes.byref(d), batch) if wsb is None else wsb
        return lib.df11_decode_gemm(ctypes.byref(d), arr, 1, fake, batch, xs, fake, ys, fake, wsb,
                                    None)

    assert gemm(0) == -1 and gemm(9) == -1                 # batch outside 1..8
    assert gemm(4, xs=4100) == -1                          # x stride not a multiple of 8
    assert gemm(4, xs=4088) == -1                          # x rows would overlap
    assert gemm(4, ys=23) == -1                            # y rows would overlap
    assert gemm(4, xs=1 << 32) == -1                       # stride beyond 32 bits
    assert gemm(4, wsb=lib.df11_gemm_workspace_bytes(ctypes.byref(d), 2)) == -2  # workspace


def test_checksum_detects_a_flipped_bit_and_offload_refuses_it():
    """One flipped stream bit desynchronises the decoder (the pages' failure
    mode), so artifacts carry a CRC-32 of their arrays; the offload runner
    checks it before using a block."""
    from huffman_decode_amd.pipeline import OffloadRunner
    enc = hd.encode(wl.random_small(50_000, 17, "normal"))
    good = enc.checksum()
    assert good == enc.checksum()
    for name in ("stream", "gaps", "block_pos", "signmant", "luts"):
        arr = getattr(enc, name)
        b = arr.view(np.uint8)
        b[b.size // 3] ^= 0x10
        assert enc.checksum() != good, name
        b[b.size // 3] ^= 0x10
    assert enc.checksum() == good
    enc.stream[100] ^= 1
    with pytest.raises(ValueError, match="checksum mismatch"):
        OffloadRunner([enc], [good])


def test_bench_reports_traffic_only_for_the_profiled_workload():
    """bench.py takes roofline.traffic from the committed counter profile only
    when that profile was taken on the current kernel (the hash of its machine
    code that the build records) and on the workload being measured (same
    algorithmic bytes per launch)."""
    import importlib.util
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(root, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    text = open(bench.TRAFFIC_FILE).read()
    alg = int(re.search(r"^algorithmic_bytes_per_launch: (\d+)", text, re.M).group(1))
    assert bench.measured_traffic(alg + 1) is None
    got = bench.measured_traffic(alg)
    if re.search(r"^kernel_isa_sha16: (\w+)", text, re.M).group(1) == bench.kernel_hash():
        assert got is not None and 0.95 * alg < got < 1.10 * alg
    else:
        assert got is None


def test_fused_wrappers_check_x_and_y_before_any_launch():
    """The C calls of the fused product receive no sizes for x and y, so the
    binding checks them: x and y must reach every matrix's inputs and
    results, and every tensor must sit on the encoded tensor's device.  All
    of it fails before anything is launched (CPU tensors stand in here)."""
    import torch
    shapes = [(8, 2048), (4, 4096)]
    w = wl.random_small(sum(r * c for r, c in shapes), 9, "normal")
    dev = hd.to_device(hd.encode(w), "cpu")
    mats, nx, ny = hd.gemv_matrices(shapes)
    ws = torch.empty(hd.df11_gemv_workspace_bytes(dev), dtype=torch.uint8)
    x = torch.zeros(nx, dtype=torch.bfloat16)
    y = torch.zeros(ny, dtype=torch.float32)
    with pytest.raises(ValueError, match="need"):
        hd.df11_decode_gemv(dev, mats, x[: nx - 8], y, ws)
    with pytest.raises(ValueError, match="need"):
        hd.df11_decode_gemv(dev, mats, x, y[: ny - 1], ws)
    with pytest.raises(ValueError, match="device"):
        hd.df11_decode_gemv(dev, mats, x.to("meta"), y, ws)
    with pytest.raises(ValueError, match="device"):
        hd.df11_decode_gemv(dev, mats, x, y, ws.to("meta"))
    xb = torch.zeros(3, nx, dtype=torch.bfloat16)
    yb = torch.zeros(3, ny, dtype=torch.float32)
    ws3 = torch.empty(hd.df11_gemm_workspace_bytes(dev, 3), dtype=torch.uint8)
    with pytest.raises(ValueError, match="need"):
        hd.df11_decode_gemm(dev, mats, xb[:, : nx - 8], yb, ws3)
    with pytest.raises(ValueError, match="need"):
        hd.df11_decode_gemm(dev, mats, xb, yb[:, : ny - 1], ws3)
    with pytest.raises(ValueError, match="device"):
        hd.df11_decode_gemm(dev, mats, xb, yb.to("meta"), ws3)


def test_noalloc_product_refuses_a_workspace_beyond_its_array():
    """df11_decode_gemm_noalloc serves the workspace from a static device array
    of NOALLOC_SCRATCH_BYTES; a stream and batch that need more are refused
    with BUFSIZE before any device call (this runs without a GPU)."""
    lib = hd.library()
    d = hd.DeviceStream()
    fake = 1 << 20
    d.stream = d.gaps = d.block_pos = d.signmant = d.luts = fake
    d.n = 855_638_016           # the 70B-shaped block
    d.n_blocks = 540_000
    mats = (hd.GemvMatrix * 1)(hd.GemvMatrix(0, 8192, d.n // 8192, 0, 0))
    for batch in (4, 8):
        need = lib.df11_gemm_workspace_bytes(ctypes.byref(d), batch)
        assert need > hd.NOALLOC_SCRATCH_BYTES
        assert lib.df11_decode_gemm_noalloc(ctypes.byref(d), mats, 1, fake, batch, 1 << 20,
                                            fake, 8192, None) == -2
    assert lib.df11_decode_gemm_noalloc(ctypes.byref(d), mats, 1, fake, 9, 1 << 20, fake, 8192,
                                        None) == -1


def test_tile_order_follows_its_definition():
    """df11_tile_order puts each word of a 16-row, 32-column operand tile where
    the definition puts it: tile (rt, ks) of a matrix at 512 (rt * cols / 32 +
    ks), group L at 8 L, word j: W[16 rt + L % 16][32 ks + 8 (L / 16) + j]."""
    shapes = [(32, 64), (16, 96), (48, 32)]
    n = sum(r * c for r, c in shapes)
    w = np.arange(n, dtype=np.uint16)
    mats, _, _ = hd.gemv_matrices(shapes)
    t = hd.df11_tile_order(w, mats)
    off = 0
    for (r, c) in shapes:
        W = w[off: off + r * c].reshape(r, c)
        for rt in range(r // 16):
            for ks in range(c // 32):
                for L in range(64):
                    at = off + ((rt * (c // 32) + ks) * 64 + L) * 8
                    col = 32 * ks + 8 * (L // 16)
                    assert np.array_equal(t[at: at + 8], W[16 * rt + L % 16, col: col + 8])
        off += r * c
    assert np.array_equal(np.sort(t), w)
    # refused: rows not a multiple of 16, cols not a multiple of 32, not covering n
    for bad in ([(24, 64)], [(16, 48)]):
        m2, _, _ = hd.gemv_matrices(bad)
        with pytest.raises(hd.Df11Error):
            hd.df11_tile_order(np.zeros(sum(r * c for r, c in bad), np.uint16), m2)
    with pytest.raises(hd.Df11Error):
        hd.df11_tile_order(np.zeros(n + 8, np.uint16), mats)


def test_tile_segments_match_a_search_of_block_pos():
    """Each segment's entry is the block holding its first weight (the last
    block whose first code index is at most that weight), and the final entry
    the block of the last weight; checked on a real encoding with a linear
    search."""
    shapes = [(64, 4096), (32, 2048), (16, 8192)]
    w = wl.random_small(sum(r * c for r, c in shapes), 3, "normal")
    te = hd.encode_tiled(w, shapes)
    bp = te.enc.block_pos.astype(np.int64)
    nb = bp.size - 1
    starts = [m.offset + rt * 16 * m.cols for m in te.mats for rt in range(m.rows // 16)]
    holder = lambda q: max(b for b in range(nb) if bp[b] <= q)
    want = [holder(q) for q in starts] + [holder(int(bp[nb]) - 1)]
    assert te.seg_blk.tolist() == want
    assert hd.library().df11_tile_segment_count(hd._mat_array(te.mats), len(te.mats)) == len(starts)


def test_tiled_workspace_size_and_refusal():
    """The tiled product's workspace holds the inputs rewritten k-step-major
    from 12 vectors on: 2 bytes x 16 per group of 16 vectors x the columns of
    the distinct input ranges; a shorter workspace is refused before any
    device call."""
    lib = hd.library()
    shapes = [(64, 4096), (32, 2048)]
    mats, _, _ = hd.gemv_matrices(shapes)
    assert hd.df11_tiled_workspace_bytes(mats, 1) == 0
    assert hd.df11_tiled_workspace_bytes(mats, 11) == 0
    assert hd.df11_tiled_workspace_bytes(mats, 12) == 2 * 16 * (4096 + 2048)
    assert hd.df11_tiled_workspace_bytes(mats, 33) == 2 * 64 * (4096 + 2048)
    assert hd.df11_tiled_workspace_bytes(mats, 65) == 0
    shared = [hd.GemvMatrix(0, 64, 4096, 0, 0), hd.GemvMatrix(64 * 4096, 32, 4096, 0, 64)]
    assert hd.df11_tiled_workspace_bytes(shared, 20) == 2 * 32 * 4096
    n = sum(r * c for r, c in shapes)
    te = hd.encode_tiled(wl.random_small(n, 4, "normal"), shapes)
    sz = te.enc.sizes
    d = hd.DeviceStream()
    fake = 1 << 20
    d.stream = d.gaps = d.block_pos = d.signmant = d.luts = fake
    d.stream_bytes, d.gaps_bytes = sz.stream_bytes, sz.gaps_bytes
    d.block_pos_count, d.signmant_bytes, d.lut_bytes = sz.block_pos_count, sz.signmant_bytes, \
        sz.lut_bytes
    d.n, d.total_bits, d.last_start = sz.n, sz.total_bits, sz.last_start
    d.n_blocks, d.n_tables, d.max_len = sz.n_blocks, te.enc.codebook.n_tables, \
        te.enc.codebook.max_len
    arr = hd._mat_array(mats)
    need = hd.df11_tiled_workspace_bytes(mats, 16)
    assert lib.df11_decode_gemm_tiled(ctypes.byref(d), arr, 2, fake, fake, 16, 6144, fake, 96,
                                      fake, need - 16, None) == -2
    assert lib.df11_decode_gemm_tiled(ctypes.byref(d), arr, 2, fake, fake, 65, 6144, fake, 96,
                                      fake, need, None) == -1
    bad = hd._mat_array(hd.gemv_matrices([(24, 4096), (40, 2048)])[0])
    assert lib.df11_decode_gemm_tiled(ctypes.byref(d), bad, 2, fake, fake, 2, 6144, fake, 96,
                                      fake, need, None) == -1


def test_plain_streams_refuse_bad_arguments_before_any_device_call():
    """The measurement-aid streams check sizes and alignment on the host."""
    lib = hd.library()
    ok, odd = 1 << 20, (1 << 20) + 8
    assert lib.df11_stream_copy(ok, odd, 1024, 0, None) == -1      # misaligned dst
    assert lib.df11_stream_copy(ok, ok, 1000, 0, None) == -1       # not a multiple of 16
    assert lib.df11_stream_copy(ok, ok, 0, 0, None) == -1
    assert lib.df11_stream_write(odd, 1024, 0, 0, None) == -1
    assert lib.df11_stream_write(0, 1024, 0, 0, None) == -1
    assert lib.df11_stream_read(ok, 1024, 0, 0, 0, None) == -1     # no out
    assert lib.df11_stream_read(odd, 1024, ok, 1 << 20, 0, None) == -1
    assert lib.df11_stream_read_slots(1000, 4) == 0
    assert lib.df11_stream_read_slots(1 << 20, 4) == 4 * 256        # the grid given, 256 threads each
    assert lib.df11_stream_read_slots(16, 4) == 256                 # never more than the bytes need


def test_decode_tiled_refuses_bad_matrix_lists_before_any_device_call():
    """The tile-order decode takes 1..16 matrices laid end to end from 0 over
    all n words, rows a multiple of 16 and cols of 32; anything else, or a
    misaligned output, is refused on the host."""
    lib = hd.library()
    shapes = [(64, 4096), (32, 2048)]
    n = sum(r * c for r, c in shapes)
    te = hd.encode_tiled(wl.random_small(n, 4, "normal"), shapes)
    sz = te.enc.sizes
    d = hd.DeviceStream()
    fake = 1 << 20
    d.stream = d.gaps = d.block_pos = d.signmant = d.luts = fake
    d.stream_bytes, d.gaps_bytes = sz.stream_bytes, sz.gaps_bytes
    d.block_pos_count, d.signmant_bytes, d.lut_bytes = sz.block_pos_count, sz.signmant_bytes, \
        sz.lut_bytes
    d.n, d.total_bits, d.last_start = sz.n, sz.total_bits, sz.last_start
    d.n_blocks, d.n_tables, d.max_len = sz.n_blocks, te.enc.codebook.n_tables, \
        te.enc.codebook.max_len
    call = lambda mats, count, out=fake: lib.df11_decode_tiled(
        ctypes.byref(d), hd._mat_array(mats), count, out, None)
    mats = te.mats
    assert call(mats, 0) == -1                                   # no matrices
    assert call(mats, 1) == -1                                   # does not cover n
    assert call(mats, 2, fake + 8) == -1                         # output not 16-byte aligned
    assert call(hd.gemv_matrices([(24, 4096), (40, 2048)])[0], 2) == -1   # rows % 16
    assert call(hd.gemv_matrices([(64, 4080), (32, 2064)])[0], 2) == -1   # cols % 32
    gap = [hd.GemvMatrix(0, 64, 4096, 0, 0), hd.GemvMatrix(64 * 4096 + 512, 32, 2048, 0, 64)]
    assert call(gap, 2) == -1                                    # not end to end
    many = hd.gemv_matrices([(16, 32)] * 17)[0]
    assert call(many, 17) == -1                                  # more than 16


def test_largest_n_is_accepted_and_one_more_is_refused():
    """n up to 2^32 - 64 passes the size and descriptor checks; 2^32 - 63 is
    refused by both (the kernels' 32-bit positions need a group of headroom)."""
    lib = hd.library()
    top = (1 << 32) - 64
    for n, want in ((top, 0), (top + 1, -1)):
        hist = np.zeros(256, np.uint64)
        hist[127] = n
        cb = hd.Codebook()
        assert lib.df11_build_codebook(hist.ctypes.data, 32, ctypes.byref(cb)) == 0
        sz = hd.Sizes()
        assert lib.df11_encoded_sizes(hist.ctypes.data, n, ctypes.byref(cb), ctypes.byref(sz)) == want
    d = hd.DeviceStream()
    fake = 1 << 20
    d.stream = d.gaps = d.block_pos = d.signmant = d.luts = fake
    d.n = top + 1
    assert lib.df11_decode(ctypes.byref(d), fake, None) == -1


def test_constructed_stream_hits_every_gap_value_and_32_bit_codes():
    """The Fibonacci histogram (codes up to 32 bits) laid out so that codes end
    at every offset 1..31 of some slice: the host encoder's gap fields then take
    all 32 values, and its arrays equal the oracle's, which decodes the stream
    back to the words."""
    import gap_streams as gs
    hist = gs.fibonacci_hist()
    lengths, _ = oracle.limited_lengths(hist, 32)
    w = gs.every_gap_stream(lengths, hist)
    enc = hd.encode(w)
    assert enc.codebook.max_len == 32 and np.array_equal(enc.codebook.lengths, lengths)
    nb, n, total = int(enc.sizes.n_blocks), int(enc.sizes.n), int(enc.sizes.total_bits)
    g = gs.gap_values(enc.gaps, 64 * nb + 1)
    assert set(g.tolist()) == set(range(32))
    oe = oracle.encode(w)
    nbytes = (total + 7) // 8
    assert oe.total_bits == total and np.array_equal(oe.stream[:nbytes], enc.stream[:nbytes])
    assert np.array_equal(oe.gaps, g) and np.array_equal(oe.block_pos, enc.block_pos[: nb + 1])
    ex, end = oracle.decode(enc.stream, total, 0, n, lengths)
    assert end == total and np.array_equal(oracle.join_bf16(ex, enc.signmant[:n]), w)
