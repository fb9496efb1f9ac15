"""GPU parity: df11_decode (through the C ABI) against the oracle and the originals.

DF11 is lossless (page "DFloat11: lossless BFloat16 compression", section
"What it is"), so the decode result is defined as the original BF16 words.
Every case checks bit-exact equality with them and, where the oracle finishes
in seconds, element-by-element equality with the oracle's own decode of the
same seeded input.  Each output buffer is pre-filled with two different
sentinels on two runs, so an element left unwritten, or written outside the
tensor, shows up.
"""
import sys

import numpy as np
import pytest

import oracle
import huffman_decode_amd as hd
from huffman_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu

GUARD = 64  # extra output elements past n that must keep their sentinel


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _gpu_decode(torch, enc, label):
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    dev = hd.to_device(enc, status=st)
    outs = []
    for fill in (0x5555, -0x5556):  # 0x5555 and 0xAAAA
        out = torch.full((enc.n + GUARD,), fill, dtype=torch.int16, device="cuda")
        _say(f"[gpu] df11_decode {label} n={enc.n} blocks={enc.sizes.n_blocks} "
             f"tables={enc.codebook.n_tables} max_len={enc.codebook.max_len} fill={fill & 0xFFFF:#x}")
        hd.df11_decode(dev, out)
        torch.cuda.synchronize()
        host = out.cpu().numpy().view(np.uint16)
        assert (host[enc.n:] == (fill & 0xFFFF)).all(), "write past the end of the tensor"
        outs.append(host[:enc.n])
    assert int(st.item()) == 0, "blocks with a count mismatch"
    assert np.array_equal(outs[0], outs[1])
    return outs[0]


SMALL = [
    ("n1", lambda: wl.random_small(1, 1, "normal")),
    ("n2", lambda: wl.random_small(2, 2, "normal")),
    ("n7", lambda: wl.random_small(7, 3, "normal")),
    ("n63", lambda: wl.random_small(63, 4, "normal")),
    ("n64", lambda: wl.random_small(64, 5, "normal")),
    ("n65", lambda: wl.random_small(65, 6, "normal")),
    ("n4097", lambda: wl.random_small(4097, 7, "normal")),
    ("ragged_100003", lambda: wl.random_small(100_003, 8, "normal")),
    ("ragged_1234567", lambda: wl.random_small(1_234_567, 9, "normal")),
    ("single_5000", lambda: wl.random_small(5000, 10, "single")),
    ("single_full_tiles", lambda: wl.random_small(4096 * 70 + 3, 11, "single")),
    ("uniform_300001", lambda: wl.random_small(300_001, 12, "uniform")),
    # codes of 1.4-2 bits: the 56-code staging slots, staged and fallback blocks
    ("geometric_1000003", lambda: wl.random_small(1_000_003, 16, "geometric")),
    ("geometric_steep_700001", lambda: wl.random_small(700_001, 17, "geometric_steep")),
    ("geometric_4097", lambda: wl.random_small(4097, 18, "geometric")),
    ("int8_200000", lambda: wl.random_small(200_000, 13, "int8")),
    ("all_exponents_small", lambda: wl.all_exponents(14, 256, 1024).weights),
    ("flux_small", lambda: wl.flux_block(15, scale=1 / 64).weights),
]


@pytest.mark.parametrize("name,make", SMALL, ids=[s[0] for s in SMALL])
def test_small_cases_match_oracle(torch, name, make):
    w = make()
    enc = hd.encode(w)
    got = _gpu_decode(torch, enc, name)
    ref = oracle.encode(w)
    assert np.array_equal(oracle.decode_tensor(ref), got)  # the oracle's own decode
    assert np.array_equal(got, w)


FULL = ["linear_4096", "fibonacci_33", "fibonacci_34", "all_exponents", "flux_block",
        "llama8b_block", "llama70b_block"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_configs(torch, name):
    wlx = wl.CONFIGS[name]()
    w = wlx.weights
    enc = hd.encode(w)
    got = _gpu_decode(torch, enc, name)
    assert np.array_equal(got, w)
    # the oracle decodes sampled blocks of the same stream independently
    rng = np.random.default_rng(99)
    nb = int(enc.sizes.n_blocks)
    blocks = np.unique(np.concatenate([[0, nb - 1], rng.choice(nb, min(nb, 48), replace=False)]))
    _oracle_blocks(enc, lambda p0, p1: got[p0:p1], blocks.tolist())


@pytest.mark.parametrize("kind,n,seed", [("normal", 300_000, 31), ("single", 4096 * 40, 32),
                                          ("uniform", 200_000, 33), ("geometric", 400_000, 34),
                                          ("geometric_steep", 300_000, 35)])
def test_flipped_stream_bits_stay_in_their_blocks(torch, kind, n, seed):
    """A flipped stream bit desynchronises the codes of its slice (the pages'
    failure mode).  A lane also reads 32 bits into the next slice, so a flip
    can reach the block before its own; every other block must still decode
    bit-exact.  A block whose code count no longer matches block_pos is
    counted in the status word and left unwritten."""
    import dataclasses
    w = wl.random_small(n, seed, kind)
    enc = hd.encode(w)
    nb = int(enc.sizes.n_blocks)
    rng = np.random.default_rng(seed)
    stream = enc.stream.copy()
    hit = set()
    for b in sorted(set(rng.choice(nb, min(nb, 6), replace=False).tolist())):
        bit = 4096 * b + int(rng.integers(0, 4096))
        if bit < int(enc.sizes.total_bits):
            stream[bit >> 3] ^= np.uint8(1 << (bit & 7))
            hit |= {b, b - 1}
    bad = dataclasses.replace(enc, stream=stream)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    dev = hd.to_device(bad, status=st)
    out = torch.full((enc.n + GUARD,), 0x5555, dtype=torch.int16, device="cuda")
    _say(f"[gpu] df11_decode flipped bits {kind} n={enc.n} blocks={nb} hit={sorted(hit)}")
    hd.df11_decode(dev, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    assert (got[enc.n:] == 0x5555).all(), "write past the end of the tensor"
    bp = enc.block_pos.astype(np.int64)
    for b in range(nb):
        if b not in hit:
            assert np.array_equal(got[bp[b]:bp[b + 1]], w[bp[b]:bp[b + 1]]), f"block {b}"
    assert 0 <= int(st.item()) <= len(hit)


def _corrupt(enc, seed, n_flips=3, bad_pos=True):
    """Flip stream bits in a few blocks and, optionally, overwrite one interior
    block_pos entry with a position past the end.  Returns the corrupted
    arrays and the blocks whose output may be wrong: a flip reaches its own
    block and the one before (a lane reads 32 bits into the next slice), and a
    bad entry makes both blocks that share it fail the host's range check."""
    import dataclasses
    nb = int(enc.sizes.n_blocks)
    rng = np.random.default_rng(seed)
    stream = enc.stream.copy()
    hit = set()
    for b in sorted(set(rng.choice(nb, min(nb, n_flips), replace=False).tolist())):
        bit = 4096 * b + int(rng.integers(0, 4096))
        if bit < int(enc.sizes.total_bits):
            stream[bit >> 3] ^= np.uint8(1 << (bit & 7))
            hit |= {b, b - 1}
    block_pos = enc.block_pos.copy()
    if bad_pos and nb > 4:
        b = int(rng.integers(2, nb - 1))
        block_pos[b] = np.uint32(enc.n + 12345)
        hit |= {b - 1, b}
    return dataclasses.replace(enc, stream=stream, block_pos=block_pos), hit


@pytest.mark.parametrize("seed", [11, 12])
def test_corrupt_block_pos_leaves_other_blocks_exact(torch, seed):
    """A block_pos entry past the end fails the range check of the two blocks
    that share it: both are counted and left unwritten, with no access outside
    the arrays, and every other block (flipped stream bits aside) decodes
    bit-exact."""
    w = wl.random_small(40 * 4096, seed, "normal")
    enc = hd.encode(w)
    bad, hit = _corrupt(enc, seed)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    dev = hd.to_device(bad, status=st)
    out = torch.full((enc.n + GUARD,), 0x5555, dtype=torch.int16, device="cuda")
    _say(f"[gpu] df11_decode corrupt block_pos seed={seed} hit={sorted(hit)}")
    hd.df11_decode(dev, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    assert (got[enc.n:] == 0x5555).all(), "write past the end of the tensor"
    bp = enc.block_pos.astype(np.int64)
    for b in range(int(enc.sizes.n_blocks)):
        if b not in hit:
            assert np.array_equal(got[bp[b]:bp[b + 1]], w[bp[b]:bp[b + 1]]), f"block {b}"
    assert 2 <= int(st.item()) <= len(hit)


def test_fused_gemv_with_corrupt_blocks(torch):
    """The fused product on a corrupted stream: blocks that fail their checks
    leave stale partial sums and row-table entries in a workspace full of
    garbage; the reduce keeps every read inside the workspace, and each row
    whose words all lie in intact blocks still gets its exact-within-bound
    sum."""
    shapes = [(24, 4096), (8, 8192)]
    n = sum(r * c for r, c in shapes)
    w = wl.random_small(n, 21, "normal")
    enc = hd.encode(w)
    bad, hit = _corrupt(enc, 21)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    dev = hd.to_device(bad, status=st)
    mats, nx, ny = hd.gemv_matrices(shapes)
    rng = np.random.default_rng(22)
    x_bits = wl.to_bf16(rng.standard_normal(nx).astype(np.float32))
    x = torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    ws = torch.full((hd.df11_gemv_workspace_bytes(dev),), 0xFF, dtype=torch.uint8, device="cuda")
    y = torch.full((ny + 5,), 2.5, dtype=torch.float32, device="cuda")
    _say(f"[gpu] df11_decode_gemv corrupt blocks hit={sorted(hit)}")
    hd.df11_decode_gemv(dev, mats, x, y, ws)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    assert np.all(got[ny:] == 2.5), "wrote past the results"
    assert int(st.item()) >= 2
    bp = enc.block_pos.astype(np.int64)
    block_of = lambda pos: int(np.searchsorted(bp, pos, side="right") - 1)
    xv_all = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    wf = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).float().numpy().astype(np.float64)
    off, checked = 0, 0
    for m, (r, c) in zip(mats, shapes):
        for row in range(r):
            rs, re = off + row * c, off + (row + 1) * c
            touched = set(range(block_of(rs), block_of(re - 1) + 1))
            # the row's range also comes from the next row's table entry
            if re < n:
                touched.add(block_of(re))
            if touched & hit:
                continue
            W = wf[rs:re]
            xv = xv_all[m.x_offset: m.x_offset + c].astype(np.float64)
            ref = W @ xv
            k = 30 + block_of(re - 1) - block_of(rs) + 1
            bound = np.abs(W) @ np.abs(xv) * k * 2.0 ** -24 + 1e-30
            assert abs(got[m.y_offset + row] - ref) <= bound, (m.rows, row)
            checked += 1
        off += r * c
    assert checked > 0


def test_gemm_bit_exact_after_decode(torch):
    """The consumer GEMM sees identical weights: Y = X W^T matches bit for bit."""
    wlx = wl.linear_4096()
    enc = hd.encode(wlx.weights)
    dev = hd.to_device(enc)
    _say("[gpu] df11_decode linear_4096 for GEMM check")
    w_dec = hd.decode(dev).view(4096, 4096)
    w_orig = torch.from_numpy(wlx.weights.view(np.int16)).to("cuda").view(torch.bfloat16)
    w_orig = w_orig.view(4096, 4096)
    gen = torch.Generator(device="cuda").manual_seed(3999)
    for batch in (1, 64):
        x = torch.randn(batch, 4096, generator=gen, device="cuda").to(torch.bfloat16)
        y0 = torch.matmul(x, w_orig.t())
        y0b = torch.matmul(x, w_orig.t())
        assert torch.equal(y0, y0b), "GEMM itself is not deterministic"
        y1 = torch.matmul(x, w_dec.t())
        torch.cuda.synchronize()
        assert torch.equal(y0, y1)


def test_stack_pipeline_overlapped_matches_bf16_gemms(torch):
    """Decode-then-GEMM over a small stack: serial and overlapped schedules
    give, block by block, the same GEMM outputs as the GEMMs on the original
    BF16 weights (same matmuls on bit-identical inputs)."""
    from huffman_decode_amd.pipeline import StackBlock, StackRunner
    blocks, originals = [], []
    for layer in range(4):
        w = wl.llama8b_block(seed=(3001, layer), scale=1 / 64)
        enc = hd.encode(w.weights)
        blocks.append(StackBlock(hd.to_device(enc), [(m.rows, m.cols) for m in w.matrices]))
        originals.append(torch.from_numpy(w.weights.view(np.int16)).cuda().view(torch.bfloat16))
    runner = StackRunner(blocks)
    for batch in (1, 64):
        acts, ref = runner.activations(batch, per_block=True)
        runner.run_gemms_only(acts, ref, originals)
        for mode in ("serial", "overlapped"):
            _say(f"[gpu] stack pipeline {mode} batch={batch}")
            _, outs = runner.activations(batch, per_block=True)
            getattr(runner, f"run_{mode}")(acts, outs)
            torch.cuda.synchronize()
            for i in range(len(blocks)):
                for sh in ref[i]:
                    assert torch.equal(outs[i][sh], ref[i][sh]), (mode, batch, i, sh)


def _oracle_blocks(enc, fetch, blocks):
    """The oracle decodes the given blocks of enc's stream on its own, from
    each block's gap offset; each must equal the GPU output there
    (fetch(p0, p1): the GPU's words p0..p1 as uint16)."""
    stop = int(enc.sizes.last_start) + 1
    gbits = np.unpackbits(enc.gaps, bitorder="little")
    for b in blocks:
        p0, p1 = int(enc.block_pos[b]), int(enc.block_pos[b + 1])
        gap = int(sum(int(gbits[5 * 64 * b + j]) << j for j in range(5)))
        ex = oracle.decode_range(enc.stream, int(enc.sizes.total_bits), 4096 * b + gap,
                                 min(4096 * (b + 1), stop), enc.codebook.lengths, 4096)
        assert ex.size == p1 - p0, f"block {b}"
        assert np.array_equal(fetch(p0, p1), oracle.join_bf16(ex, enc.signmant[p0:p1])), f"block {b}"


def test_every_gap_value_and_32_bit_codes(torch):
    """A stream whose gap fields take all 32 values and whose code book has
    32-bit codes (the Fibonacci histogram laid out so that codes end at every
    offset 1..31 of a slice; 9.2 M words): bit-exact, and the blocks holding
    the constructed codes decoded by the oracle on their own."""
    import gap_streams as gs
    hist = gs.fibonacci_hist()
    lengths, _ = oracle.limited_lengths(hist, 32)
    w = gs.every_gap_stream(lengths, hist)
    enc = hd.encode(w)
    nb = int(enc.sizes.n_blocks)
    assert enc.codebook.max_len == 32
    assert set(gs.gap_values(enc.gaps, 64 * nb + 1).tolist()) == set(range(32))
    got = _gpu_decode(torch, enc, "every gap value")
    assert np.array_equal(got, w)
    _oracle_blocks(enc, lambda p0, p1: got[p0:p1], [0, 1, 2, nb - 1])


def _skewed_stream(k, seed, total=1 << 21):
    """Exponent j < k with count total / 2^(j+1), every other exponent 1-3
    times, shuffled, random sign|mantissa: short codes for the common
    exponents (about 2 bits on average) and many long ones under different
    8-bit prefixes, so the code book needs many lookup tables."""
    rng = np.random.default_rng(seed)
    h = np.zeros(256, np.int64)
    for j in range(k):
        h[j] = max(1, total >> (j + 1))
    h[k:] = rng.integers(1, 4, 256 - k)
    e = np.repeat(np.arange(256, dtype=np.uint16), h)
    np.random.default_rng(seed + 1000).shuffle(e)
    low = np.random.default_rng(seed + 2000).integers(0, 256, e.size).astype(np.uint16)
    return (((low & 0x80) << 8) | (e << 7) | (low & 0x7F)).astype(np.uint16)


@pytest.mark.parametrize("k,seed,tables", [(4, 0, 17), (8, 4, 38), (8, 156, 53)])
def test_many_lookup_tables(torch, k, seed, tables):
    """Code books of 17, 38 and 53 8-bit tables (up to 27 KB of them in LDS
    beside the decode table and the staging regions; the codes average under
    2.51 bits, so the wide-slot kernel runs): bit-exact, and sampled blocks
    decoded by the oracle on their own."""
    w = _skewed_stream(k, seed)
    enc = hd.encode(w)
    assert enc.codebook.n_tables == tables
    got = _gpu_decode(torch, enc, f"tables={tables}")
    assert np.array_equal(got, w)
    nb = int(enc.sizes.n_blocks)
    _oracle_blocks(enc, lambda p0, p1: got[p0:p1], sorted({0, nb // 2, nb - 1}))


def test_decode_at_the_largest_n(torch):
    """The largest stream the format's 32-bit output positions allow, to the
    nearest multiple of 64: n = 2^32 - 64 words (8.6 GB of BF16, 64 copies of
    one 2^26 - 1-word N(0, 0.02) draw, seed 77).  Every output position, block
    index and stream offset of the kernel is then at its widest.  The decode
    must give the original words bit for bit, leave the guard past n alone and
    report no block; the oracle decodes the first and the last two blocks on
    its own."""
    chunk = wl.random_small((1 << 26) - 1, 77, "normal")
    n = 64 * chunk.size
    assert n == (1 << 32) - 64
    _say(f"[gpu] df11_decode largest n={n}: encoding")
    w = np.tile(chunk, 64)
    enc = hd.encode(w)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    dev = hd.to_device(enc, status=st)
    out = torch.full((n + GUARD,), 0x5555, dtype=torch.int16, device="cuda")
    _say(f"[gpu] df11_decode largest n={n} blocks={enc.sizes.n_blocks} "
         f"total_bits={enc.sizes.total_bits}: decoding")
    hd.df11_decode(dev, out)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert bool((out[n:] == 0x5555).all()), "write past the end of the tensor"
    ref = torch.from_numpy(w.view(np.int16)).cuda()
    assert torch.equal(out[:n], ref), "decoded words differ from the originals"
    del ref
    nb = int(enc.sizes.n_blocks)
    stop = int(enc.sizes.last_start) + 1
    for b in (0, nb - 2, nb - 1):
        p0, p1 = int(enc.block_pos[b]), int(enc.block_pos[b + 1])
        gap = int(enc.gaps[40 * b]) & 31  # block b's first 5-bit field starts at byte 40 b
        ex = oracle.decode_range(enc.stream, int(enc.sizes.total_bits), 4096 * b + gap,
                                 min(4096 * (b + 1), stop), enc.codebook.lengths, 4096)
        got = out[p0:p1].cpu().numpy().view(np.uint16)
        assert np.array_equal(got, oracle.join_bf16(ex, enc.signmant[p0:p1])), f"block {b}"


def test_fused_products_at_the_largest_n(torch):
    """The row-major fused products on one 262,080 x 16,384 matrix (n within
    2^20 of the format's 32-bit limit; 64 rows of one seeded draw repeated,
    |w| in [2^-8, 2^-5) or 0) with inputs in {-1, 0, 1}: every partial sum is
    a multiple of 2^-15 below 2^9, exact in fp32 in any order, so df11_decode_gemv
    and df11_decode_gemm (8 vectors) must equal numpy's fp64 product bit for
    bit on sampled rows, and write nothing past the results."""
    rows, cols = 262_080, 16_384
    chunk = wl.random_small(64 * cols, 94, "normal").copy()
    e = (chunk >> 7) & 0xFF
    chunk[e < 127 - 8] = 0
    chunk[e >= 127 - 5] = (chunk[e >= 127 - 5] & 0x807F) | np.uint16((127 - 6) << 7)
    w = np.tile(chunk, rows // 64)
    n = w.size
    _say(f"[gpu] fused products largest n={n}: encoding")
    enc = hd.encode(w)
    dev = hd.to_device(enc)
    mats, nx, ny = hd.gemv_matrices([(rows, cols)])
    wc = torch.from_numpy(chunk.view(np.int16)).view(torch.bfloat16).double().numpy().reshape(64, cols)
    sample = np.unique(np.concatenate([np.arange(64), rows - 64 + np.arange(64),
                                       np.random.default_rng(95).integers(0, rows, 256)]))
    for batch in (1, 8):
        x_bits = np.array([0xBF80, 0, 0x3F80], np.uint16)[
            np.random.default_rng(96 + batch).integers(0, 3, (batch, nx))]
        x = torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)
        y = torch.full((batch, ny + 5), -7.0, dtype=torch.float32, device="cuda")
        _say(f"[gpu] fused products largest n={n} batch={batch}")
        if batch == 1:
            ws = torch.empty(hd.df11_gemv_workspace_bytes(dev), dtype=torch.uint8, device="cuda")
            hd.df11_decode_gemv(dev, mats, x[0], y[0], ws)
        else:
            ws = torch.empty(hd.df11_gemm_workspace_bytes(dev, batch), dtype=torch.uint8,
                             device="cuda")
            hd.df11_decode_gemm(dev, mats, x, y[:, :ny], ws)
        torch.cuda.synchronize()
        h = y.cpu().numpy()
        assert np.all(h[:, ny:] == -7.0), "wrote past the results"
        xf = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).double().numpy()
        assert (np.abs(xf) @ np.abs(wc).T).max() < 2.0 ** 9
        ref = (xf @ wc.T)[:, sample % 64]
        assert np.array_equal(h[:, sample].astype(np.float64), ref), f"batch {batch}"
        del ws


@pytest.mark.parametrize("layer", list(range(32)))
def test_stack_block_full_size(torch, layer):
    """The 32-block Llama-3.1-8B-shaped stack at full size, one block at a
    time (218,103,808 weights each, seeds (3001, layer)): generate, encode,
    decode, compare bit for bit with the originals on the GPU, and decode
    sampled blocks with the oracle.  On the first and the last block the
    consumer GEMMs (batch 1 and 64) on the decoded weights must equal those on
    the originals, matrix by matrix."""
    wlx = wl.llama8b_stack_block(layer)
    enc = hd.encode(wlx.weights)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    dev = hd.to_device(enc, status=st)
    out = torch.full((enc.n + GUARD,), 0x5555, dtype=torch.int16, device="cuda")
    _say(f"[gpu] df11_decode stack layer {layer} n={enc.n} blocks={enc.sizes.n_blocks}")
    hd.df11_decode(dev, out)
    orig = torch.from_numpy(wlx.weights.view(np.int16)).cuda()
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert bool((out[enc.n:] == 0x5555).all()), "write past the end of the tensor"
    assert torch.equal(out[:enc.n], orig), f"layer {layer} differs from the original weights"
    nb = int(enc.sizes.n_blocks)
    rng = np.random.default_rng(layer)
    sample = sorted(set([0, nb - 1] + rng.choice(nb, 6, replace=False).tolist()))
    _oracle_blocks(enc, lambda p0, p1: out[p0:p1].cpu().numpy().view(np.uint16), sample)
    if layer in (0, 31):
        dec = out[:enc.n].view(torch.bfloat16)
        ref = orig.view(torch.bfloat16)
        gen = torch.Generator(device="cuda").manual_seed(3999)
        off = 0
        for m in wlx.matrices:
            wd = dec[off: off + m.rows * m.cols].view(m.rows, m.cols)
            wo = ref[off: off + m.rows * m.cols].view(m.rows, m.cols)
            for batch in (1, 64):
                x = torch.randn(batch, m.cols, generator=gen, device="cuda").to(torch.bfloat16)
                _say(f"[gpu] stack layer {layer} GEMM {m.name} batch={batch}")
                y0 = torch.matmul(x, wo.t())
                y1 = torch.matmul(x, wd.t())
                assert torch.equal(y0, y1), (layer, m.name, batch)
            off += m.rows * m.cols
    del out, orig, dev, enc


@pytest.fixture(scope="module")
def small_stack(torch):
    from huffman_decode_amd.pipeline import StackBlock
    blocks, originals = [], []
    for layer in range(4):
        w = wl.llama8b_block(seed=(3001, layer), scale=1 / 16)
        enc = hd.encode(w.weights)
        blocks.append(StackBlock(hd.to_device(enc), [(m.rows, m.cols) for m in w.matrices]))
        originals.append(torch.from_numpy(w.weights.view(np.int16)).cuda().view(torch.bfloat16))
    return blocks, originals


@pytest.mark.parametrize("groups", [8, 256, 384, 512])
def test_capped_decode_grid(torch, small_stack, groups):
    """A decode grid capped at `groups` workgroups (df11_device_stream.max_groups,
    what the overlapped schedule uses to leave compute units to the GEMMs)
    decodes bit-exact, and the overlapped schedule with that cap gives the same
    GEMM outputs as the GEMMs on the original weights."""
    from huffman_decode_amd.pipeline import StackRunner
    blocks, originals = small_stack
    for i, (blk, orig) in enumerate(zip(blocks, originals)):
        out = torch.full((blk.dev.n + GUARD,), 0x5555, dtype=torch.int16, device="cuda")
        blk.dev.desc.max_groups = groups
        _say(f"[gpu] df11_decode capped at {groups} groups, block {i}")
        try:
            hd.df11_decode(blk.dev, out)
        finally:
            blk.dev.desc.max_groups = 0
        torch.cuda.synchronize()
        assert torch.equal(out[:blk.dev.n], orig.view(torch.int16)), (groups, i)
        assert bool((out[blk.dev.n:] == 0x5555).all())
    runner = StackRunner(blocks)
    for batch in (1, 64):
        acts, ref = runner.activations(batch, per_block=True)
        runner.run_gemms_only(acts, ref, originals)
        _, outs = runner.activations(batch, per_block=True)
        _say(f"[gpu] stack pipeline overlapped, decode capped at {groups}, batch={batch}")
        runner.run_overlapped(acts, outs, groups)
        torch.cuda.synchronize()
        for i in range(len(blocks)):
            for sh in ref[i]:
                assert torch.equal(outs[i][sh], ref[i][sh]), (groups, batch, i, sh)


# ---------------------------------------------------------------------------
# Fused decode + GEMV.  Reference: the plain product of the original BF16
# weights with the BF16 x, both as float64, by numpy.  BF16 x BF16 products
# are exact in fp32.  A row's sum is formed with: per 8-word group, four packed
# dot instructions (each counted as 2 roundings, and at twice the unit
# roundoff in case it truncates: 16 units); the group added to the lane's sum
# (at most 8 groups per lane per block: 8); the wave's 64-lane sum (6); and
# one addition per block that holds words of the row.  So |y - ref| <=
# (30 + B_row) 2^-24 sum |w x|, with B_row the blocks the row touches, taken
# from block_pos.  (For rows of 28672 words in 512-word blocks, B_row is 57.)

def _row_bounds(enc, mats, shapes):
    """Per matrix, the rounding count 30 + B_row of each row."""
    bp = enc.block_pos.astype(np.int64)
    out = []
    for m, (r, c) in zip(mats, shapes):
        rs = m.offset + c * np.arange(r, dtype=np.int64)
        first = np.searchsorted(bp, rs, side="right") - 1
        last = np.searchsorted(bp, rs + c - 1, side="right") - 1
        out.append(30 + (last - first + 1))
    return out


def _gemv_check(torch, w, shapes, label, seed=7):
    enc = hd.encode(w)
    dev = hd.to_device(enc)
    mats, nx, ny = hd.gemv_matrices(shapes)
    rng = np.random.default_rng(seed)
    x_bits = wl.to_bf16(rng.standard_normal(nx).astype(np.float32))
    x = torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    x_host = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    ws = torch.empty(hd.df11_gemv_workspace_bytes(dev), dtype=torch.uint8, device="cuda")
    ys = []
    for fill in (1.0e30, -7.0):
        y = torch.full((ny,), fill, dtype=torch.float32, device="cuda")
        _say(f"[gpu] df11_decode_gemv {label} n={enc.n} mats={len(mats)} fill={fill}")
        hd.df11_decode_gemv(dev, mats, x, y, ws)
        torch.cuda.synchronize()
        ys.append(y.cpu().numpy())
    assert np.array_equal(ys[0].view(np.uint32), ys[1].view(np.uint32)), "not deterministic"
    wf = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).float().numpy().astype(np.float64)
    off = 0
    for m, (r, c), k in zip(mats, shapes, _row_bounds(enc, mats, shapes)):
        W = wf[off: off + r * c].reshape(r, c)
        xv = x_host[m.x_offset: m.x_offset + c].astype(np.float64)
        ref = W @ xv
        bound = np.abs(W) @ np.abs(xv) * k * 2.0 ** -24 + 1e-30
        got = ys[0][m.y_offset: m.y_offset + r].astype(np.float64)
        bad = np.abs(got - ref) > bound
        assert not bad.any(), (label, m.rows, m.cols, int(bad.sum()))
        off += r * c


@pytest.mark.parametrize("name,make,scale", [
    ("llama8b_1_64", lambda: wl.llama8b_block(seed=11, scale=1 / 64), None),
    ("flux_1_64", lambda: wl.flux_block(12, scale=1 / 64), None),
    ("ragged_rows", lambda: wl.normal_block("r", [("a", 37, 2048), ("b", 5, 6144), ("c", 129, 2056)],
                                            13, 0.02), None),
])
def test_fused_gemv_small(torch, name, make, scale):
    wlx = make()
    _gemv_check(torch, wlx.weights, [(m.rows, m.cols) for m in wlx.matrices], name)


def test_fused_gemv_single_exponent_fallback(torch):
    """A one-exponent tensor has 1-bit codes: every block takes the re-decode
    route and several tile passes."""
    w = wl.random_small(64 * 4096, 21, "single")
    _gemv_check(torch, w, [(64, 4096)], "single")


def test_fused_gemv_llama8b_block(torch):
    wlx = wl.llama8b_block()
    _gemv_check(torch, wlx.weights, [(m.rows, m.cols) for m in wlx.matrices], "llama8b_block")


def _flat_exponents(n, seed):
    """Words whose exponents are spread evenly over 127 values (7-bit codes,
    about 580 words per block), all finite: sign and mantissa random."""
    rng = np.random.default_rng(seed)
    e = rng.integers(64, 191, n).astype(np.uint16)
    return (rng.integers(0, 1 << 16, n).astype(np.uint16) & 0x807F) | (e << 7)


@pytest.mark.parametrize("kind", ["normal", "flat"])
def test_fused_gemv_70b_down_rows(torch, kind):
    """Rows of the 70B-shaped down matrix (28672 columns): with flat exponents
    a row spans about 50 blocks, beyond what a fixed bound of 46 roundings
    would cover; the per-row bound follows the stream."""
    shapes = [(8, 28672)]
    n = 8 * 28672
    w = wl.random_small(n, 51, "normal") if kind == "normal" else _flat_exponents(n, 52)
    _gemv_check(torch, w, shapes, f"70b_down_{kind}")
    _gemm_check(torch, w, shapes, f"70b_down_{kind}", 3)


# Fused decode + product with several input vectors: each vector's result is
# checked like the batch-1 one, and must equal, bit for bit, what the batch-1
# call gives for that vector alone (the same sums in the same order).

def _gemm_check(torch, w, shapes, label, batch, seed=17, x_pad=24, y_pad=5):
    enc = hd.encode(w)
    dev = hd.to_device(enc)
    mats, nx, ny = hd.gemv_matrices(shapes)
    rng = np.random.default_rng(seed)
    x_bits = wl.to_bf16(rng.standard_normal((batch, nx + x_pad)).astype(np.float32))
    x = torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    x_host = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    ws = torch.empty(hd.df11_gemm_workspace_bytes(dev, batch), dtype=torch.uint8, device="cuda")
    ys = []
    for fill in (1.0e30, -7.0):
        y = torch.full((batch, ny + y_pad), fill, dtype=torch.float32, device="cuda")
        _say(f"[gpu] df11_decode_gemm {label} n={enc.n} batch={batch} fill={fill}")
        hd.df11_decode_gemm(dev, mats, x, y, ws)
        torch.cuda.synchronize()
        ys.append(y.cpu().numpy())
    assert np.array_equal(ys[0][:, :ny].view(np.uint32), ys[1][:, :ny].view(np.uint32)), \
        "not deterministic"
    assert np.all(ys[0][:, ny:] == 1.0e30) and np.all(ys[1][:, ny:] == -7.0), "wrote past the results"
    wf = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).float().numpy().astype(np.float64)
    ws1 = torch.empty(hd.df11_gemv_workspace_bytes(dev), dtype=torch.uint8, device="cuda")
    ks = _row_bounds(enc, mats, shapes)
    for b in range(batch):
        off = 0
        for m, (r, c), k in zip(mats, shapes, ks):
            W = wf[off: off + r * c].reshape(r, c)
            xv = x_host[b, m.x_offset: m.x_offset + c].astype(np.float64)
            ref = W @ xv
            bound = np.abs(W) @ np.abs(xv) * k * 2.0 ** -24 + 1e-30
            got = ys[0][b, m.y_offset: m.y_offset + r].astype(np.float64)
            bad = np.abs(got - ref) > bound
            assert not bad.any(), (label, b, m.rows, m.cols, int(bad.sum()))
            off += r * c
        y1 = torch.full((ny,), 3.0, dtype=torch.float32, device="cuda")
        hd.df11_decode_gemv(dev, mats, x[b, :nx].contiguous(), y1, ws1)
        torch.cuda.synchronize()
        assert np.array_equal(y1.cpu().numpy().view(np.uint32), ys[0][b, :ny].view(np.uint32)), \
            (label, b, "differs from the batch-1 result")


@pytest.mark.parametrize("batch", [2, 3, 5, 8])
def test_fused_gemm_batches(torch, batch):
    wlx = wl.llama8b_block(seed=11, scale=1 / 64)
    _gemm_check(torch, wlx.weights, [(m.rows, m.cols) for m in wlx.matrices], "llama8b_1_64", batch)


def test_fused_gemm_ragged_rows_and_fallback(torch):
    wlx = wl.normal_block("r", [("a", 37, 2048), ("b", 5, 6144), ("c", 129, 2056)], 13, 0.02)
    _gemm_check(torch, wlx.weights, [(m.rows, m.cols) for m in wlx.matrices], "ragged_rows", 4)
    w = wl.random_small(64 * 4096, 21, "single")
    _gemm_check(torch, w, [(64, 4096)], "single", 2)


def test_fused_gemm_llama8b_block_batch4(torch):
    wlx = wl.llama8b_block()
    _gemm_check(torch, wlx.weights, [(m.rows, m.cols) for m in wlx.matrices], "llama8b_block", 4)


def test_offload_runner_decodes_blocks_from_pinned_host_memory(torch):
    """CPU offload: blocks copied from pinned host memory per decode, two
    staging slots reused in turn; every block bit-exact."""
    from huffman_decode_amd.pipeline import OffloadRunner
    ws = [wl.llama8b_block(seed=(3001, layer), scale=1 / 64).weights for layer in range(5)]
    encs = [hd.encode(w) for w in ws]
    runner = OffloadRunner(encs, [e.checksum() for e in encs])
    seen = {}

    def keep(i, out):
        seen[i] = out.view(torch.int16).clone()

    _say("[gpu] offload runner, 5 blocks")
    runner.run(keep)
    torch.cuda.synchronize()
    for i, w in enumerate(ws):
        assert np.array_equal(seen[i].cpu().numpy().view(np.uint16), w), i
