"""Every device entry point captured in a HIP graph (torch.cuda.CUDAGraph)
and replayed: the calls enqueue kernels only (no allocation, no memset, no
copy), so a replay must give exactly what the eager call gives.  Before each
of several replays the outputs are overwritten with a byte pattern, and eager
launches of the same entry point into other buffers, plus other torch work,
run between the replays."""
import sys

import numpy as np
import pytest

import huffman_decode_amd as hd
from huffman_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _replays_match(torch, label, launch, outputs, eager_outputs):
    """launch() enqueues into `outputs`; eager_outputs are other buffers of
    the same shapes for the eager launches between replays."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch(outputs)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    expect = [t.clone() for t in outputs]
    graph = torch.cuda.CUDAGraph()
    _say(f"[gpu] capture {label}")
    with torch.cuda.graph(graph):
        launch(outputs)
    busy = torch.randn(512, 512, device="cuda")
    for r in range(REPLAYS):
        for t in outputs:
            t.view(torch.uint8).fill_(0xA5)
        _say(f"[gpu] replay {label} #{r}")
        graph.replay()
        torch.cuda.synchronize()
        for a, e in zip(outputs, expect):
            assert torch.equal(a, e), f"{label}: replay {r} differs from the eager result"
        # the program's own work between replays: eager launches of the same
        # call into other buffers, and a matrix product
        launch(eager_outputs)
        busy = busy @ busy.T / 512.0
        torch.cuda.synchronize()
        for a, e in zip(eager_outputs, expect):
            assert torch.equal(a, e), f"{label}: eager call after replay {r} differs"
    del graph


def test_graph_decode(torch):
    w = wl.random_small(300_001, 61, "normal")
    enc = hd.encode(w)
    dev = hd.to_device(enc)
    bufs = [torch.empty(enc.n, dtype=torch.int16, device="cuda") for _ in range(2)]
    _replays_match(torch, "df11_decode", lambda o: hd.df11_decode(dev, o[0]), bufs[:1], bufs[1:])
    assert np.array_equal(bufs[0].cpu().numpy().view(np.uint16), w)


SHAPES = [(256, 4096), (64, 2048)]


def _inputs(torch, batch, nx, seed):
    rng = np.random.default_rng(seed)
    x = wl.to_bf16(rng.standard_normal((batch, nx)).astype(np.float32))
    return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)


@pytest.mark.parametrize("batch", [1, 4])
def test_graph_row_major_products(torch, batch):
    n = sum(r * c for r, c in SHAPES)
    enc = hd.encode(wl.random_small(n, 62, "normal"))
    dev = hd.to_device(enc)
    mats, nx, ny = hd.gemv_matrices(SHAPES)
    x = _inputs(torch, batch, nx, 63)
    ws = torch.empty(hd.df11_gemm_workspace_bytes(dev, batch), dtype=torch.uint8, device="cuda")
    ys = [torch.empty(batch, ny, dtype=torch.float32, device="cuda") for _ in range(2)]
    _replays_match(torch, f"df11_decode_gemm batch={batch}",
                   lambda o: hd.df11_decode_gemm(dev, mats, x, o[0], ws), ys[:1], ys[1:])
    zs = [torch.empty(batch, ny, dtype=torch.float32, device="cuda") for _ in range(2)]
    _replays_match(torch, f"df11_decode_gemm_noalloc batch={batch}",
                   lambda o: hd.df11_decode_gemm_noalloc(dev, mats, x, o[0]), zs[:1], zs[1:])
    assert torch.equal(ys[0], zs[0])


@pytest.mark.parametrize("batch", [1, 16, 64])
def test_graph_tiled_product(torch, batch):
    """Batch 1 takes the one-vector kernel, 16 and 64 the input rewrite into
    the workspace first (two kernels per call)."""
    n = sum(r * c for r, c in SHAPES)
    te = hd.encode_tiled(wl.random_small(n, 64, "normal"), SHAPES)
    td = hd.tiled_to_device(te)
    nx = max(m.x_offset + m.cols for m in te.mats)
    ny = sum(m.rows for m in te.mats)
    x = _inputs(torch, batch, nx, 65)
    need = hd.df11_tiled_workspace_bytes(te.mats, batch)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
    ys = [torch.empty(batch, ny, dtype=torch.float32, device="cuda") for _ in range(2)]
    _replays_match(torch, f"df11_decode_gemm_tiled batch={batch}",
                   lambda o: hd.df11_decode_gemm_tiled(td, x, o[0], ws), ys[:1], ys[1:])


def test_graph_tile_order_decode(torch):
    n = sum(r * c for r, c in SHAPES)
    w = wl.random_small(n, 66, "normal")
    te = hd.encode_tiled(w, SHAPES)
    td = hd.tiled_to_device(te)
    bufs = [torch.empty(n, dtype=torch.int16, device="cuda") for _ in range(2)]
    _replays_match(torch, "df11_decode_tiled", lambda o: hd.df11_decode_tiled(td, o[0]),
                   bufs[:1], bufs[1:])
    assert np.array_equal(bufs[0].cpu().numpy().view(np.uint16), w)
