"""GPU parity of the decode of a tile-order stream (df11_decode_tiled) through
the C ABI: the stream holds the weights in operand-tile order, and the decode
must give back the original row-major BF16 words bit for bit (the same
Huffman decode and sign|mantissa join as the plain decode, with the tile-order
positions mapped back to rows and columns), with nothing written past n and
the same result on every run."""
import sys

import numpy as np
import pytest

import huffman_decode_amd as hd
from huffman_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu

GUARD = 40


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _decode_tiled(torch, te, label, status=None):
    td = hd.tiled_to_device(te, status=status)
    n = te.enc.n
    outs = []
    for fill in (0x5555, -0x5556):  # 0x5555 and 0xAAAA
        out = torch.full((n + GUARD,), fill, dtype=torch.int16, device="cuda")
        _say(f"[gpu] df11_decode_tiled {label} n={n} mats={len(te.mats)} "
             f"blocks={te.enc.sizes.n_blocks} max_len={te.enc.codebook.max_len} fill={fill & 0xFFFF:#x}")
        hd.df11_decode_tiled(td, out)
        torch.cuda.synchronize()
        host = out.cpu().numpy().view(np.uint16)
        assert (host[n:] == (fill & 0xFFFF)).all(), "write past the end of the tensor"
        outs.append(host[:n])
    assert np.array_equal(outs[0], outs[1]), "not deterministic (or words left unwritten)"
    return outs[0]


def _words(n, seed, kind):
    if kind == "flat":  # uniform words: 8-bit codes, about 512 words per block
        return wl.random_small(n, seed, "uniform")
    if kind == "one_exponent":  # 1-bit codes, 4096 words per block: blocks decode in passes
        w = wl.random_small(n, seed, "single")
        return (w & 0x807F) | np.uint16(120 << 7)
    return wl.random_small(n, seed, kind)


SHAPES = [
    ("one_tile", [(16, 32)]),
    ("sixteen_tiny", [(16, 32)] * 16),  # many matrices inside one block
    ("mixed", [(48, 96), (16, 4096), (64, 32), (32, 160)]),
    ("narrow_tall", [(1024, 32), (16, 64)]),
    ("wide", [(32, 14336), (16, 4096)]),
]


@pytest.mark.parametrize("kind", ["normal", "flat", "one_exponent"])
@pytest.mark.parametrize("label,shapes", SHAPES, ids=[s[0] for s in SHAPES])
def test_decode_tiled_gives_back_the_row_major_words(torch, label, shapes, kind):
    n = sum(r * c for r, c in shapes)
    w = _words(n, 31 + len(label), kind)
    te = hd.encode_tiled(w, shapes)
    got = _decode_tiled(torch, te, f"{label}_{kind}")
    assert np.array_equal(got, w)


def test_decode_tiled_llama8b_block_full(torch):
    """The seven matrices of a Llama-3.1-8B transformer block (218M words)."""
    wlx = wl.llama8b_block()
    w = wlx.weights
    te = hd.encode_tiled(w, [(m.rows, m.cols) for m in wlx.matrices])
    got = _decode_tiled(torch, te, "llama8b_block")
    assert np.array_equal(got, w)


def test_decode_tiled_corrupt_blocks_stay_contained(torch):
    """Flipped code bits and an impossible block position: the blocks that
    fail their count check are reported and left unwritten, and every word
    of every other block lands, exact, at its row-major place."""
    from test_gpu_parity import _corrupt
    shapes = [(64, 4096), (32, 1024), (16, 32)]
    n = sum(r * c for r, c in shapes)
    w = wl.random_small(n, 43, "normal")
    te = hd.encode_tiled(w, shapes)
    bad, hit = _corrupt(te.enc, 43)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    td = hd.tiled_to_device(hd.TiledEncoded(bad, te.mats, te.seg_blk), status=st)
    out = torch.full((n + GUARD,), 0x5555, dtype=torch.int16, device="cuda")
    _say(f"[gpu] df11_decode_tiled corrupt hit={sorted(hit)}")
    hd.df11_decode_tiled(td, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    assert (got[n:] == 0x5555).all(), "write past the end of the tensor"
    assert 2 <= int(st.item()) <= len(hit)
    # where each tile-order word lives in row-major order: the tile order of
    # the indices themselves, in two 16-bit halves
    idx = np.arange(n, dtype=np.uint32)
    lo = hd.df11_tile_order((idx & 0xFFFF).astype(np.uint16), te.mats)
    hi = hd.df11_tile_order((idx >> 16).astype(np.uint16), te.mats)
    where = lo.astype(np.int64) | (hi.astype(np.int64) << 16)
    bp = te.enc.block_pos.astype(np.int64)
    checked = 0
    for b in range(int(te.enc.sizes.n_blocks)):
        if b in hit:
            continue
        rows = where[bp[b]:bp[b + 1]]
        assert np.array_equal(got[rows], w[rows]), f"block {b}"
        checked += rows.size
    assert checked > n // 2
