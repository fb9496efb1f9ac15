"""GPU parity of the tiled fused product (df11_decode_gemm_tiled) through the C ABI.

y_b = W x_b for 1-64 input vectors, computed on the matrix cores straight from
a DF11 stream whose weights are in operand-tile order.  The reference is the
plain product of the original row-major BF16 weights with the BF16 inputs in
float64 (numpy), which knows nothing of the tile order.

Two kinds of check:
  * exact: weights of magnitude below 2^-8 set to zero and inputs in
    {-1, 0, 1}.  Every product is then a multiple of 2^-15 and every partial
    sum a multiple of 2^-15 below 2^9 in magnitude (the tests assert it), so
    it is exact in fp32 whatever the order or grouping of the additions, and
    the result must equal the float64 product bit for bit.  A weight paired
    with the wrong input, counted twice or left out shows up here.
  * bounded: ordinary N(0, sigma) data.  Each result is formed by the matrix
    instructions of each wave (32 products each, added to the running sum),
    then 8 wave sums added in order.  Counting every one of the 32 additions
    of an instruction as a separate fp32 rounding (2^-23 each, which also
    covers truncation), a result whose wave took at most k instructions has
    |y - ref| <= (32 k + 8) 2^-23 sum |w x|; k <= cols / 256 + 3 (its share of
    the row tile's cols / 32 operand tiles, plus the tiles at the edges of
    its blocks).
The result must also be the same, bit for bit, on two runs, and nothing may be
written past the results.
"""
import sys

import numpy as np
import pytest

import huffman_decode_amd as hd
from huffman_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _bf16_to_f64(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).float().numpy().astype(np.float64)


def _run_tiled(torch, te, x_bits, batch, label, y_pad=5, status=None):
    td = hd.tiled_to_device(te, status=status)
    nx = x_bits.shape[1]
    ny = sum(m.rows for m in te.mats)
    x = torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    need = hd.df11_tiled_workspace_bytes(te.mats, batch)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda") if need else None
    ys = []
    for fill in (1.0e30, -7.0):
        y = torch.full((batch, ny + y_pad), fill, dtype=torch.float32, device="cuda")
        _say(f"[gpu] df11_decode_gemm_tiled {label} n={te.enc.n} batch={batch} "
             f"blocks={te.enc.sizes.n_blocks} segments={te.seg_blk.size - 1} fill={fill}")
        hd.df11_decode_gemm_tiled(td, x[:, :nx], y[:, :ny], ws)
        torch.cuda.synchronize()
        h = y.cpu().numpy()
        assert np.all(h[:, ny:] == fill), "wrote past the results"
        ys.append(h[:, :ny])
    return ys


def _reference(torch, w_bits, shapes, mats, x_bits):
    """float64 W x of the original row-major weights, per vector, and sum |w x|."""
    wf = _bf16_to_f64(torch, w_bits)
    xf = _bf16_to_f64(torch, x_bits)
    refs, mags, off = [], [], 0
    for m, (r, c) in zip(mats, shapes):
        W = wf[off: off + r * c].reshape(r, c)
        X = xf[:, m.x_offset: m.x_offset + c]
        refs.append(X @ W.T)
        mags.append(np.abs(X) @ np.abs(W).T)
        off += r * c
    return refs, mags


def _check(torch, w_bits, shapes, batch, label, exact, seed=5, shared_x=False):
    te = hd.encode_tiled(w_bits, shapes)
    if shared_x:  # every matrix reads the same inputs (as q, k and v do)
        for m in te.mats:
            m.x_offset = 0
    mats = te.mats
    nx = max(m.x_offset + m.cols for m in mats)
    rng = np.random.default_rng(seed)
    if exact:
        x_bits = np.array([0xBF80, 0, 0x3F80], np.uint16)[rng.integers(0, 3, (batch, nx))]
    else:
        x_bits = wl.to_bf16(rng.standard_normal((batch, nx)).astype(np.float32))
    ys = _run_tiled(torch, te, x_bits, batch, label)
    assert np.array_equal(ys[0].view(np.uint32), ys[1].view(np.uint32)), "not deterministic"
    refs, mags = _reference(torch, w_bits, shapes, mats, x_bits)
    for m, (r, c), ref, mag in zip(mats, shapes, refs, mags):
        got = ys[0][:, m.y_offset: m.y_offset + r].astype(np.float64)
        if exact:
            assert mag.max() < 2.0 ** 9, "the exact case needs sums below 2^9"
            bad = got != ref
        else:
            k = c // 256 + 3
            bad = np.abs(got - ref) > (32 * k + 8) * 2.0 ** -23 * mag + 1e-30
        assert not bad.any(), (label, batch, r, c, int(bad.sum()))


def _exact_weights(n, seed, kind="normal"):
    """BF16 words with every nonzero magnitude at least 2^-8 (smaller ones
    set to +0), so that products with inputs in {-1, 0, 1} are multiples of
    2^-15."""
    w = wl.random_small(n, seed, kind).copy()
    w[((w >> 7) & 0xFF) < 127 - 8] = 0
    return w


EXACT_SHAPES = {
    "mixed": [(64, 4096), (32, 2048), (16, 4096), (48, 1024)],
    # cols, and the power of two each |w| is held below (cols * 2^-c = 448)
    "down": ([(32, 14336)], 5),
    "down70b": ([(32, 28672)], 6),
}


@pytest.mark.parametrize("batch", [1, 2, 9, 16, 17, 33, 64])
def test_tiled_exact_batches(torch, batch):
    shapes = EXACT_SHAPES["mixed"]
    w = _exact_weights(sum(r * c for r, c in shapes), 100 + batch)
    _check(torch, w, shapes, batch, "exact_mixed", exact=True)


@pytest.mark.parametrize("batch", [8, 12, 64])
def test_tiled_exact_shared_inputs(torch, batch):
    """Matrices that read the same input range: the inputs are rewritten once
    for all of them."""
    shapes = [(64, 4096), (32, 4096), (16, 4096)]
    w = _exact_weights(sum(r * c for r, c in shapes), 40 + batch)
    _check(torch, w, shapes, batch, "exact_shared_x", exact=True, shared_x=True)


@pytest.mark.parametrize("name", ["down", "down70b"])
def test_tiled_exact_wide_rows(torch, name):
    shapes, c = EXACT_SHAPES[name]
    n = sum(r * cols for r, cols in shapes)
    w = _exact_weights(n, 7)
    # keep |w| < 2^-c so that a row's sum of |w| stays below 2^9
    big = ((w >> 7) & 0xFF) >= 127 - c
    w[big] = (w[big] & 0x807F) | np.uint16((127 - c - 1) << 7)
    for batch in (1, 64):
        _check(torch, w, shapes, batch, f"exact_{name}", exact=True)


def test_tiled_exact_one_bit_codes(torch):
    """One exponent only: 1-bit codes, 4096 words per block, so every block
    decodes again in tile-sized passes and operand tiles straddle passes."""
    shapes = [(32, 4096), (16, 8192)]
    n = sum(r * c for r, c in shapes)
    w = wl.random_small(n, 8, "single")
    w = (w & 0x807F) | np.uint16((127 - 6) << 7)  # one exponent, 2^-6 .. 2^-5
    for batch in (1, 20, 64):
        _check(torch, w, shapes, batch, "exact_single", exact=True)


def test_tiled_exact_flat_codes(torch):
    """Uniform random words (8-bit codes, about 512 words per block) with
    their exponents folded into [2^-8, 2^-5)."""
    shapes = [(48, 4096)]
    n = sum(r * c for r, c in shapes)
    w = wl.random_small(n, 9, "uniform")
    e = ((w >> 7) & 0xFF) % 3 + (127 - 8)
    w = (w & 0x807F) | (e.astype(np.uint16) << 7)
    for batch in (1, 3, 64):
        _check(torch, w, shapes, batch, "exact_flat", exact=True)


@pytest.mark.parametrize("batch", [1, 16, 64])
def test_tiled_llama8b_shapes(torch, batch):
    wlx = wl.llama8b_block(seed=31, scale=1 / 16)
    _check(torch, wlx.weights, [(m.rows, m.cols) for m in wlx.matrices], batch, "llama8b_1_16",
           exact=False)


def test_tiled_flux_and_70b_down(torch):
    wlx = wl.flux_block(33, scale=1 / 32)
    _check(torch, wlx.weights, [(m.rows, m.cols) for m in wlx.matrices], 40, "flux_1_32",
           exact=False)
    shapes = [(64, 28672)]
    w = wl.random_small(64 * 28672, 34, "normal")
    _check(torch, w, shapes, 64, "70b_down_rows", exact=False)


@pytest.mark.parametrize("batch", [1, 64])
def test_tiled_llama8b_block_full(torch, batch):
    """The full 8B-shaped block at the batches the benchmark times first and
    last (1: the one-vector kernel; 64: four groups of 16)."""
    wlx = wl.llama8b_block()
    _check(torch, wlx.weights, [(m.rows, m.cols) for m in wlx.matrices], batch, "llama8b_block",
           exact=False)


def test_tiled_paths_at_the_largest_n(torch):
    """One 262,080 x 16,384 matrix: n = 4,293,918,720 words, within 2^20 of
    the format's 32-bit limit, and 8,386,560 operand tiles (the tile-order
    decode divides tile indices by a float reciprocal, exact below 2^23).
    The weights repeat one seeded draw of 64 rows (|w| in [2^-8, 2^-5) or 0,
    so each row's sum of |w| stays below 2^9).  The tiled product at one and
    at 64 vectors in {-1, 0, 1} must equal numpy's fp64 product bit for bit
    on sampled rows (every 64-row period, first and last rows included), and
    the tile-order decode must give back every word."""
    rows, cols = 262_080, 16_384
    chunk = _exact_weights(64 * cols, 91)
    big = ((chunk >> 7) & 0xFF) >= 127 - 5
    chunk[big] = (chunk[big] & 0x807F) | np.uint16((127 - 6) << 7)
    w = np.tile(chunk, rows // 64)
    n = w.size
    assert n == rows * cols and (1 << 32) - n <= (1 << 20)
    _say(f"[gpu] tiled paths largest n={n}: encoding")
    te = hd.encode_tiled(w, [(rows, cols)])
    td = hd.tiled_to_device(te)
    wc = _bf16_to_f64(torch, chunk).reshape(64, cols)
    sample = np.unique(np.concatenate([np.arange(64), rows - 64 + np.arange(64),
                                       np.random.default_rng(92).integers(0, rows, 256)]))
    for batch in (1, 64):
        x_bits = np.array([0xBF80, 0, 0x3F80], np.uint16)[
            np.random.default_rng(93 + batch).integers(0, 3, (batch, cols))]
        x = torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)
        need = hd.df11_tiled_workspace_bytes(te.mats, batch)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
        y = torch.full((batch, rows + 5), -7.0, dtype=torch.float32, device="cuda")
        _say(f"[gpu] df11_decode_gemm_tiled largest n={n} batch={batch}")
        hd.df11_decode_gemm_tiled(td, x, y[:, :rows], ws)
        torch.cuda.synchronize()
        h = y.cpu().numpy()
        assert np.all(h[:, rows:] == -7.0), "wrote past the results"
        xf = _bf16_to_f64(torch, x_bits)
        ref = xf @ wc.T  # [batch, 64]: row r of the matrix is chunk row r % 64
        assert (np.abs(xf) @ np.abs(wc).T).max() < 2.0 ** 9
        got = h[:, sample].astype(np.float64)
        assert np.array_equal(got, ref[:, sample % 64]), f"batch {batch}"
    out = torch.full((n + 40,), 0x5555, dtype=torch.int16, device="cuda")
    _say(f"[gpu] df11_decode_tiled largest n={n}")
    hd.df11_decode_tiled(td, out)
    torch.cuda.synchronize()
    assert bool((out[n:] == 0x5555).all()), "write past the end of the tensor"
    assert torch.equal(out[:n], torch.from_numpy(w.view(np.int16)).cuda())


@pytest.mark.parametrize("batch", [1, 8])
def test_tiled_corrupt_blocks_stay_contained(torch, batch):
    """Flipped stream bits: the blocks whose counts no longer match are
    counted in the status word and left out; nothing is written outside y,
    and every segment whose blocks are all intact is still exact (one vector
    runs its own kernel, with the inputs gathered across the wave)."""
    import dataclasses
    shapes = [(64, 4096), (32, 8192)]
    w = _exact_weights(sum(r * c for r, c in shapes), 61)
    te = hd.encode_tiled(w, shapes)
    nb = int(te.enc.sizes.n_blocks)
    rng = np.random.default_rng(62)
    stream = te.enc.stream.copy()
    hit = set()
    for b in sorted(set(rng.choice(nb, 4, replace=False).tolist())):
        bit = 4096 * b + int(rng.integers(0, 4096))
        if bit < int(te.enc.sizes.total_bits):
            stream[bit >> 3] ^= np.uint8(1 << (bit & 7))
            hit |= {b, b - 1}
    bad = hd.TiledEncoded(dataclasses.replace(te.enc, stream=stream), te.mats, te.seg_blk)
    nx = max(m.x_offset + m.cols for m in te.mats)
    x_bits = np.array([0xBF80, 0, 0x3F80], np.uint16)[rng.integers(0, 3, (batch, nx))]
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ys = _run_tiled(torch, bad, x_bits, batch, "corrupt", status=st)
    assert int(st.item()) >= 1
    refs, _ = _reference(torch, w, shapes, te.mats, x_bits)
    seg, checked = 0, 0
    for m, (r, c), ref in zip(te.mats, shapes, refs):
        for rt in range(r // 16):
            blocks = set(range(int(te.seg_blk[seg]), int(te.seg_blk[seg + 1]) + 1))
            if not blocks & hit:
                got = ys[0][:, m.y_offset + 16 * rt: m.y_offset + 16 * rt + 16].astype(np.float64)
                assert np.array_equal(got, ref[:, 16 * rt: 16 * rt + 16]), (r, c, rt)
                checked += 1
            seg += 1
    assert checked > 0


def test_stack_runner_fused_tiled(torch):
    """The stack schedule of the tiled product: every block writes the same y
    (one activation buffer), so after a pass y holds the last block's result,
    which must equal a direct call on that block bit for bit."""
    from huffman_decode_amd.pipeline import StackBlock, StackRunner
    blocks = []
    for layer in range(3):
        w = wl.llama8b_block(seed=(3001, layer), scale=1 / 64)
        shapes = [(m.rows, m.cols) for m in w.matrices]
        te = hd.encode_tiled(w.weights, shapes)
        blocks.append(StackBlock(hd.to_device(hd.encode(w.weights)), shapes, hd.tiled_to_device(te)))
    runner = StackRunner(blocks)
    for batch in (4, 24):
        x, y, ws = runner.tiled_inputs(batch)
        _say(f"[gpu] stack runner fused tiled batch={batch}")
        runner.run_fused_tiled(x, y, ws)
        y_ref = torch.empty_like(y)
        hd.df11_decode_gemm_tiled(blocks[-1].tiled, x, y_ref, ws)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32))


def test_stream_ceiling_reads_every_byte(torch):
    """The traffic-only kernel the decode is measured against.  A wave takes
    tiles of 128 consecutive 8-word groups, lane l groups l and l + 64 of the
    tile; tile t's share of b is its 16-byte units [t U / T, (t + 1) U / T),
    lane l XORing units l, l + 64, ... of that share into both its groups.
    Each output word is its sign|mantissa byte widened to 16 bits, XORed with
    the lane's share."""
    n, b_bytes = 8 * 3001, 16 * 257
    rng = np.random.default_rng(71)
    a = rng.integers(0, 256, n).astype(np.uint8)
    b = rng.integers(0, 256, b_bytes).astype(np.uint8)
    out = torch.full((n + 8,), 0x1234, dtype=torch.int16, device="cuda")
    _say("[gpu] df11_stream_ceiling")
    hd.df11_stream_ceiling(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(), out, n)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    assert np.all(got[n:] == 0x1234), "wrote past the output"
    groups, units = n // 8, b_bytes // 16
    tiles = -(-groups // 128)
    want = a.astype(np.uint16).reshape(groups, 8).copy()
    bw = b.view(np.uint16).reshape(units, 8)
    for t in range(tiles):
        u0, u1 = t * units // tiles, (t + 1) * units // tiles
        for lane in range(64):
            extra = np.zeros(8, np.uint16)
            for u in range(u0 + lane, u1, 64):
                extra ^= bw[u]
            for g in (128 * t + lane, 128 * t + 64 + lane):
                if g < groups:
                    want[g] ^= extra
    assert np.array_equal(got[:n].reshape(groups, 8), want)


@pytest.mark.parametrize("nbytes,grid", [(16, 0), ((1 << 20) + 48, 0), ((5 << 20) + 4096, 7)])
def test_plain_streams_do_what_they_say(torch, nbytes, grid):
    """The read-only, write-only and copy streams (measurement aids): the copy
    copies, the write writes its records, the read's per-thread XORs fold to
    the XOR of everything read."""
    n32 = nbytes // 4
    src = torch.randint(-(1 << 31), (1 << 31) - 1, (n32 + 8,), dtype=torch.int32, device="cuda")
    dst = torch.full((n32 + 8,), 7, dtype=torch.int32, device="cuda")
    _say(f"[gpu] plain streams bytes={nbytes} grid={grid}")
    hd.df11_stream_copy(src, dst, nbytes, grid)
    torch.cuda.synchronize()
    assert torch.equal(dst[:n32], src[:n32]) and bool((dst[n32:] == 7).all())
    hd.df11_stream_write(dst, nbytes, 0x01020304, grid)
    torch.cuda.synchronize()
    rec = dst[:n32].view(-1, 4).cpu().numpy().astype(np.uint32)
    assert (rec[:, :3] == 0x01020304).all()
    assert (rec[:, 3] == np.arange(rec.shape[0], dtype=np.uint32)).all()
    assert bool((dst[n32:] == 7).all())
    slots = torch.full((hd.df11_stream_read_slots(nbytes, grid),), 5, dtype=torch.int32,
                       device="cuda")
    hd.df11_stream_read(src, slots, nbytes, grid)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(src[:n32].cpu().numpy().view(np.uint32))
    assert np.bitwise_xor.reduce(slots.cpu().numpy().view(np.uint32)) == want
