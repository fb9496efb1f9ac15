"""Decode-then-GEMM scheduling over a stack of DF11 transformer blocks.

The DF11 pages describe inference that decompresses each transformer block's
weights just before its matrix products and discards them afterwards (page
"DFloat11: lossless BFloat16 compression", section "Architecture").  This
module runs that pattern on one GPU, with the decode and the consumer GEMMs
(``y = x W^T`` for each matrix of a block, torch bf16 matmuls) either on one
stream (serial) or overlapped: block i+1 is decoded on a second stream into
the other half of a double buffer while block i's GEMMs run.  Device memory
holds the compressed blocks plus two BF16 buffers of the largest block.

Only stream/event ordering lives here; every decode is a ``df11_decode``
launch of the native library.
"""
from __future__ import annotations

from dataclasses import dataclass

from . import (DeviceEncoded, TiledDevice, df11_decode, df11_decode_gemm, df11_decode_gemm_tiled,
               df11_gemm_workspace_bytes, df11_tiled_workspace_bytes, gemv_matrices)


@dataclass
class StackBlock:
    """One encoded transformer block and the (rows, cols) of its matrices in
    storage order (row-major, concatenated); optionally the same block
    encoded in operand-tile order for the tiled product."""
    dev: DeviceEncoded
    shapes: list[tuple[int, int]]
    tiled: TiledDevice | None = None


class StackRunner:
    """Runs ``decode(block i) -> GEMMs(block i)`` for a list of blocks."""

    def __init__(self, blocks: list[StackBlock], device="cuda"):
        import torch
        if not blocks:
            raise ValueError("no blocks")
        self.blocks = blocks
        self.device = torch.device(device)
        n_max = max(b.dev.n for b in blocks)
        for b in blocks:
            if sum(r * c for r, c in b.shapes) != b.dev.n:
                raise ValueError("matrix shapes do not cover the block's weights")
        # two decode targets: block i uses buffer i % 2
        self.buffers = [torch.empty(n_max, dtype=torch.bfloat16, device=self.device)
                        for _ in range(2)]
        self.decode_stream = torch.cuda.Stream(device=self.device)

    @property
    def compute_stream(self):
        """torch's current stream on the device, read at each call (so that
        a schedule run under a HIP graph capture is captured)."""
        import torch
        return torch.cuda.current_stream(self.device)

    @staticmethod
    def _views(buf, shapes):
        out, off = [], 0
        for r, c in shapes:
            out.append(buf[off: off + r * c].view(r, c))
            off += r * c
        return out

    def _gemms(self, i, buf, acts, outs):
        """Block i's GEMMs on the weights in buf.  ``outs`` is one dict of
        outputs by matrix shape shared by all blocks, or a list of such dicts,
        one per block."""
        import torch
        shapes = self.blocks[i].shapes
        o = outs[i] if isinstance(outs, list) else outs
        for w, sh in zip(self._views(buf, shapes), shapes):
            torch.matmul(acts[sh], w.t(), out=o[sh])

    def activations(self, batch: int, seed: int = 3999, per_block: bool = False):
        """One bf16 activation [batch, cols] per matrix shape (N(0,1) from a
        seeded generator) and outputs [batch, rows]: one dict by shape, or with
        per_block a list of such dicts, one per block."""
        import torch
        g = torch.Generator(device=self.device).manual_seed(seed)
        shapes = sorted({s for b in self.blocks for s in b.shapes})
        acts = {(r, c): torch.randn(batch, c, generator=g, device=self.device).to(torch.bfloat16)
                for r, c in shapes}

        def new_outs():
            return {(r, c): torch.empty(batch, r, dtype=torch.bfloat16, device=self.device)
                    for r, c in shapes}
        return acts, ([new_outs() for _ in self.blocks] if per_block else new_outs())

    def run_serial(self, acts, outs):
        """Decode and GEMMs of every block in order on the compute stream."""
        s = self.compute_stream
        for i, blk in enumerate(self.blocks):
            buf = self.buffers[i % 2]
            df11_decode(blk.dev, buf, s)
            self._gemms(i, buf, acts, outs)

    def run_overlapped(self, acts, outs, decode_groups: int = 0):
        """Decode of block i+1 (decode stream) overlaps the GEMMs of block i
        (compute stream).  Buffer i % 2 is reused by block i + 2 only after
        block i's GEMMs are done.  Work is enqueued in block order, so every
        event is recorded before a stream is told to wait for it (a wait on
        an event not yet recorded would not wait at all).  ``decode_groups``
        (0 = all that fit) caps the decode's workgroups, leaving compute units
        to the GEMMs."""
        import torch
        ds, cs = self.decode_stream, self.compute_stream
        n = len(self.blocks)
        decoded = [torch.cuda.Event() for _ in range(n)]
        consumed = [torch.cuda.Event() for _ in range(n)]
        for blk in self.blocks:
            blk.dev.desc.max_groups = decode_groups
        ds.wait_stream(cs)  # inputs prepared on the compute stream
        df11_decode(self.blocks[0].dev, self.buffers[0], ds)
        decoded[0].record(ds)
        for i, blk in enumerate(self.blocks):
            if i + 1 < n:
                if i >= 1:
                    ds.wait_event(consumed[i - 1])  # block i+1 reuses block i-1's buffer
                df11_decode(self.blocks[i + 1].dev, self.buffers[(i + 1) % 2], ds)
                decoded[i + 1].record(ds)
            cs.wait_event(decoded[i])
            self._gemms(i, self.buffers[i % 2], acts, outs)
            consumed[i].record(cs)
        cs.wait_stream(ds)
        for blk in self.blocks:
            blk.dev.desc.max_groups = 0

    def run_gemms_only(self, acts, outs, resident):
        """The BF16 reference: the same GEMMs on already resident BF16 weights
        (``resident[i]`` holds block i's decoded weights)."""
        for i, buf in enumerate(resident):
            self._gemms(i, buf, acts, outs)

    def run_decodes_only(self):
        s = self.compute_stream
        for i, blk in enumerate(self.blocks):
            df11_decode(blk.dev, self.buffers[i % 2], s)

    def fused_inputs(self, batch: int, seed: int = 4001):
        """Inputs and outputs for run_fused: x [batch, nx] bf16 (N(0,1) from a
        seeded generator), y [batch, ny] fp32 and a workspace, all sized for
        the largest block; the matrix list of every block."""
        import torch
        mats = [gemv_matrices(b.shapes) for b in self.blocks]
        nx = max(m[1] for m in mats)
        ny = max(m[2] for m in mats)
        g = torch.Generator(device=self.device).manual_seed(seed)
        x = torch.randn(batch, nx, generator=g, device=self.device).to(torch.bfloat16)
        y = torch.empty(batch, ny, dtype=torch.float32, device=self.device)
        ws = torch.empty(max(df11_gemm_workspace_bytes(b.dev, batch) for b in self.blocks),
                         dtype=torch.uint8, device=self.device)
        return [m[0] for m in mats], x, y, ws

    def run_fused(self, mats, x, y, ws):
        """y = W x for every block straight from its DF11 stream (no BF16
        weights anywhere): the fused product in place of decode-then-GEMM.
        Every block writes the same y, as a forward pass would overwrite one
        activation buffer."""
        s = self.compute_stream
        for i, blk in enumerate(self.blocks):
            df11_decode_gemm(blk.dev, mats[i], x, y, ws, s)


    def tiled_inputs(self, batch: int, seed: int = 4002):
        """Inputs, outputs and workspace for run_fused_tiled (every block must
        carry its tile-order encoding)."""
        import torch
        if any(b.tiled is None for b in self.blocks):
            raise ValueError("run_fused_tiled needs every block's tile-order encoding")
        nx = max(max(m.x_offset + m.cols for m in b.tiled.mats) for b in self.blocks)
        ny = max(sum(m.rows for m in b.tiled.mats) for b in self.blocks)
        g = torch.Generator(device=self.device).manual_seed(seed)
        x = torch.randn(batch, nx, generator=g, device=self.device).to(torch.bfloat16)
        y = torch.empty(batch, ny, dtype=torch.float32, device=self.device)
        need = max(df11_tiled_workspace_bytes(b.tiled.mats, batch) for b in self.blocks)
        ws = torch.empty(need, dtype=torch.uint8, device=self.device) if need else None
        return x, y, ws

    def run_fused_tiled(self, x, y, ws):
        """y = W x for every block on the matrix cores, straight from its
        tile-order stream (no BF16 weights anywhere)."""
        s = self.compute_stream
        for blk in self.blocks:
            df11_decode_gemm_tiled(blk.tiled, x, y, ws, s)


class OffloadRunner:
    """CPU offload: the encoded blocks stay in pinned host memory and each is
    copied to the GPU just before its decode (the DF11 pages' offload mode,
    which trades PCIe traffic for GPU memory).  Two device staging slots
    alternate: block i+1's arrays are copied on a copy stream while block i
    decodes.  Device memory holds two blocks' compressed arrays and two BF16
    buffers.  Every block's checksum is verified when it is placed in host
    memory."""

    _ARRAYS = ("stream", "gaps", "block_pos", "signmant", "luts")

    def __init__(self, encoded: list, checksums: list[int], device="cuda"):
        import numpy as np
        import torch
        from . import _descriptor, to_device
        if len(encoded) != len(checksums) or not encoded:
            raise ValueError("one checksum per encoded block")
        for i, (enc, want) in enumerate(zip(encoded, checksums)):
            got = enc.checksum()
            if got != want:
                raise ValueError(f"block {i}: checksum mismatch: stored {want:#010x}, "
                                 f"data {got:#010x}")
        self.device = torch.device(device)
        self.encoded = encoded
        self.host = []
        for enc in encoded:
            pinned = {}
            for name in self._ARRAYS:
                arr = getattr(enc, name)
                if name == "block_pos":
                    arr = arr.view(np.int32)
                t = torch.empty(arr.shape, dtype=torch.from_numpy(arr[:0]).dtype, pin_memory=True)
                t.copy_(torch.from_numpy(arr))
                pinned[name] = t
            self.host.append(pinned)
        # staging slots sized for the largest block
        self.slots = []
        for _ in range(2):
            t = {name: torch.empty(max(h[name].numel() for h in self.host),
                                   dtype=self.host[0][name].dtype, device=self.device)
                 for name in self._ARRAYS}
            self.slots.append(t)
        self._descriptor = _descriptor
        n_max = max(e.n for e in encoded)
        self.buffers = [torch.empty(n_max, dtype=torch.bfloat16, device=self.device)
                        for _ in range(2)]
        self.copy_stream = torch.cuda.Stream(device=self.device)

    @property
    def compute_stream(self):
        """torch's current stream on the device, read at each call (so that
        a schedule run under a HIP graph capture is captured)."""
        import torch
        return torch.cuda.current_stream(self.device)

    def _desc(self, i, slot):
        enc = self.encoded[i]
        views = {name: self.slots[slot][name][: self.host[i][name].numel()]
                 for name in self._ARRAYS}
        return self._descriptor(enc.sizes, enc.codebook, views)

    def run(self, consume=None):
        """Copy and decode every block in order; consume(i, bf16) (optional)
        is enqueued on the compute stream after block i's decode.  Returns the
        BF16 buffer of the last block."""
        import torch
        from . import df11_decode, DeviceEncoded
        cs, xs = self.compute_stream, self.copy_stream
        n = len(self.encoded)
        copied = [torch.cuda.Event() for _ in range(n)]
        used = [torch.cuda.Event() for _ in range(n)]
        xs.wait_stream(cs)

        def copy(i):
            slot = i % 2
            if i >= 2:
                xs.wait_event(used[i - 2])  # slot i % 2 was block i-2's
            with torch.cuda.stream(xs):
                for name in self._ARRAYS:
                    src = self.host[i][name]
                    self.slots[slot][name][: src.numel()].copy_(src, non_blocking=True)
            copied[i].record(xs)

        copy(0)
        for i in range(n):
            if i + 1 < n:
                copy(i + 1)
            cs.wait_event(copied[i])
            dev = DeviceEncoded(self._desc(i, i % 2), self.slots[i % 2], self.encoded[i].n)
            out = self.buffers[i % 2]
            df11_decode(dev, out, cs)
            if consume is not None:
                consume(i, out[: self.encoded[i].n])
            used[i].record(cs)
        cs.wait_stream(xs)
        return self.buffers[(n - 1) % 2][: self.encoded[-1].n]
