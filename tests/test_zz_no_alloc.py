"""df11_decode_gemm_noalloc against df11_decode_gemm, through the C ABI.

The entry point without allocation uses the library's static device array as
the fused product's workspace.  Its results must equal, bit for bit, those of
df11_decode_gemm with a caller-owned workspace (the same kernels and the same
summation order), on two calls in a row, the second with a smaller input, so
that whatever the first call left in the array is in place for the second.
Both are also checked against the plain fp64 product of the original weights
within the fused product's error bound.
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


def _case(torch, wlx, batch, seed):
    shapes = [(m.rows, m.cols) for m in wlx.matrices]
    enc = hd.encode(wlx.weights)
    dev = hd.to_device(enc)
    mats, nx, ny = hd.gemv_matrices(shapes)
    rng = np.random.default_rng(seed)
    x_bits = wl.to_bf16(rng.standard_normal((batch, nx)).astype(np.float32))
    x = torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    need = hd.df11_gemm_workspace_bytes(dev, batch)
    assert need <= hd.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y_ref = torch.full((batch, ny + 3), 7.0, dtype=torch.float32, device="cuda")
    y = torch.full((batch, ny + 3), -3.0, dtype=torch.float32, device="cuda")
    print(f"[gpu] df11_decode_gemm_noalloc {wlx.name} n={enc.n} batch={batch}",
          file=sys.stderr, flush=True)
    hd.df11_decode_gemm(dev, mats, x[:, :nx], y_ref[:, :ny], ws)
    hd.df11_decode_gemm_noalloc(dev, mats, x[:, :nx], y[:, :ny])
    torch.cuda.synchronize()
    got, ref = y.cpu().numpy(), y_ref.cpu().numpy()
    assert np.all(got[:, ny:] == -3.0), "wrote past the results"
    assert np.array_equal(got[:, :ny].view(np.uint32), ref[:, :ny].view(np.uint32))
    # and within the fused product's bound against fp64: (30 + B_row) 2^-24
    # sum |w x|, B_row the blocks the row touches (see test_gpu_parity.py)
    wf = torch.from_numpy(wlx.weights.view(np.int16)).view(torch.bfloat16).float().numpy()
    xf = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    bp = enc.block_pos.astype(np.int64)
    off = 0
    for m, (r, c) in zip(mats, shapes):
        W = wf[off: off + r * c].reshape(r, c).astype(np.float64)
        rs = off + c * np.arange(r, dtype=np.int64)
        k = 31 + np.searchsorted(bp, rs + c - 1, side="right") - np.searchsorted(bp, rs, side="right")
        for b in range(batch):
            xv = xf[b, m.x_offset: m.x_offset + c].astype(np.float64)
            bound = np.abs(W) @ np.abs(xv) * k * 2.0 ** -24 + 1e-30
            assert np.all(np.abs(got[b, m.y_offset: m.y_offset + r] - W @ xv) <= bound)
        off += r * c


def test_noalloc_matches_workspace_entry_point_twice(torch):
    _case(torch, wl.llama8b_block(seed=41, scale=1 / 8), 4, 1)
    _case(torch, wl.llama8b_block(seed=42, scale=1 / 64), 2, 2)
