"""MI355X (gfx950) implementation of the DFloat11 (DF11) decode path.

A thin ctypes binding over ``libdf11.so`` whose C ABI is declared in
``include/df11.h``.  The functions named ``df11_*`` mirror the C entry points
one to one and only marshal arguments; every step of encoding runs in the
library's C++ host code and every step of decoding in its HIP kernel.  PyTorch
is used only for device memory and streams.

Convenience wrappers: :func:`encode` (host numpy -> :class:`Encoded`),
:func:`to_device` (-> :class:`DeviceEncoded`) and :func:`decode` (-> a torch
bfloat16 tensor on the GPU).

Loading fails loudly if the library has not been built
(``python -m huffman_decode_amd.build``); there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdf11.so")

DF11_OK = 0
MAX_CODE_LEN = 32
BLOCK_BYTES = 512
STREAM_GUARD = 16

_U8, _U32, _U64, _P = ctypes.c_uint8, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p


class Codebook(ctypes.Structure):
    _fields_ = [("code_len", _U8 * 256), ("code", _U32 * 256), ("max_len", _U32),
                ("n_symbols", _U32), ("n_tables", _U32), ("lut_bytes", _U32),
                ("limit_rounds", _U32), ("reserved", _U32)]

    @property
    def lengths(self) -> np.ndarray:
        return np.frombuffer(bytes(self.code_len), np.uint8).copy()

    @property
    def codes(self) -> np.ndarray:
        return np.array(self.code[:], np.uint32)


class Sizes(ctypes.Structure):
    _fields_ = [("n", _U64), ("total_bits", _U64), ("last_start", _U64), ("stream_bytes", _U64),
                ("gaps_bytes", _U64), ("block_pos_count", _U64), ("signmant_bytes", _U64),
                ("lut_bytes", _U64), ("n_blocks", _U32), ("reserved", _U32)]


class GemvMatrix(ctypes.Structure):
    _fields_ = [("offset", _U64), ("rows", _U32), ("cols", _U32), ("x_offset", _U32),
                ("y_offset", _U32)]


class DeviceStream(ctypes.Structure):
    _fields_ = [("stream", _P), ("gaps", _P), ("block_pos", _P), ("signmant", _P), ("luts", _P),
                ("stream_bytes", _U64), ("gaps_bytes", _U64), ("block_pos_count", _U64),
                ("signmant_bytes", _U64), ("lut_bytes", _U64), ("n", _U64),
                ("total_bits", _U64), ("last_start", _U64), ("n_blocks", _U32),
                ("n_tables", _U32), ("max_len", _U32), ("max_groups", _U32), ("status", _P)]


class Df11Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m huffman_decode_amd.build` (there is no fallback)")
        lib = ctypes.CDLL(LIB_PATH)
        lib.df11_status_string.argtypes = [ctypes.c_int]
        lib.df11_status_string.restype = ctypes.c_char_p
        lib.df11_histogram.argtypes = [_P, _U64, _P, _U32]
        lib.df11_build_codebook.argtypes = [_P, _U32, ctypes.POINTER(Codebook)]
        lib.df11_build_luts.argtypes = [ctypes.POINTER(Codebook), _P, _U64]
        lib.df11_encoded_sizes.argtypes = [_P, _U64, ctypes.POINTER(Codebook),
                                           ctypes.POINTER(Sizes)]
        lib.df11_encode.argtypes = [_P, _U64, ctypes.POINTER(Codebook), _P, _U64, _P, _U64, _P,
                                    _U64, _P, _U64, ctypes.POINTER(Sizes), _U32]
        lib.df11_decode.argtypes = [ctypes.POINTER(DeviceStream), _P, _P]
        for fn in ("df11_histogram", "df11_build_codebook", "df11_build_luts",
                   "df11_encoded_sizes", "df11_encode", "df11_decode"):
            getattr(lib, fn).restype = ctypes.c_int
        if hasattr(lib, "df11_decode_gemv"):
            lib.df11_gemv_workspace_bytes.argtypes = [ctypes.POINTER(DeviceStream)]
            lib.df11_gemv_workspace_bytes.restype = _U64
            lib.df11_decode_gemv.argtypes = [ctypes.POINTER(DeviceStream),
                                             ctypes.POINTER(GemvMatrix), _U32, _P, _P, _P, _U64, _P]
            lib.df11_decode_gemv.restype = ctypes.c_int
        if hasattr(lib, "df11_decode_gemm"):
            lib.df11_gemm_workspace_bytes.argtypes = [ctypes.POINTER(DeviceStream), _U32]
            lib.df11_gemm_workspace_bytes.restype = _U64
            lib.df11_decode_gemm.argtypes = [ctypes.POINTER(DeviceStream), ctypes.POINTER(GemvMatrix),
                                             _U32, _P, _U32, _U64, _P, _U64, _P, _U64, _P]
            lib.df11_decode_gemm.restype = ctypes.c_int
        lib.df11_decode_gemm_noalloc.argtypes = [ctypes.POINTER(DeviceStream),
                                                 ctypes.POINTER(GemvMatrix), _U32, _P, _U32,
                                                 _U64, _P, _U64, _P]
        lib.df11_decode_gemm_noalloc.restype = ctypes.c_int
        lib.df11_tile_order.argtypes = [_P, _U64, ctypes.POINTER(GemvMatrix), _U32, _P, _U32]
        lib.df11_tile_order.restype = ctypes.c_int
        lib.df11_tile_segment_count.argtypes = [ctypes.POINTER(GemvMatrix), _U32]
        lib.df11_tile_segment_count.restype = _U64
        lib.df11_tile_segments.argtypes = [_P, _U32, ctypes.POINTER(GemvMatrix), _U32, _P, _U64]
        lib.df11_tile_segments.restype = ctypes.c_int
        lib.df11_decode_gemm_tiled.argtypes = [ctypes.POINTER(DeviceStream),
                                               ctypes.POINTER(GemvMatrix), _U32, _P, _P, _U32,
                                               _U64, _P, _U64, _P, _U64, _P]
        lib.df11_decode_gemm_tiled.restype = ctypes.c_int
        lib.df11_decode_tiled.argtypes = [ctypes.POINTER(DeviceStream),
                                          ctypes.POINTER(GemvMatrix), _U32, _P, _P]
        lib.df11_decode_tiled.restype = ctypes.c_int
        lib.df11_tiled_workspace_bytes.argtypes = [ctypes.POINTER(GemvMatrix), _U32, _U32]
        lib.df11_tiled_workspace_bytes.restype = _U64
        lib.df11_stream_ceiling.argtypes = [_P, _P, _U64, _P, _U64, _U32, _P]
        lib.df11_stream_ceiling.restype = ctypes.c_int
        lib.df11_stream_read_slots.argtypes = [_U64, _U32]
        lib.df11_stream_read_slots.restype = _U32
        lib.df11_stream_read.argtypes = [_P, _U64, _P, _U64, _U32, _P]
        lib.df11_stream_read.restype = ctypes.c_int
        lib.df11_stream_write.argtypes = [_P, _U64, _U32, _U32, _P]
        lib.df11_stream_write.restype = ctypes.c_int
        lib.df11_stream_copy.argtypes = [_P, _P, _U64, _U32, _P]
        lib.df11_stream_copy.restype = ctypes.c_int
        _lib = lib
    return _lib


def library():
    """The loaded ctypes library (raises if it is not built)."""
    return _load()


def status_string(status: int) -> str:
    return _load().df11_status_string(status).decode()


def _check(fn: str, status: int) -> None:
    if status != DF11_OK:
        raise Df11Error(fn, status)


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ------------------------------------------------------------ host entry points

def df11_histogram(bf16: np.ndarray, hist: np.ndarray | None = None, n_threads: int = 0
                   ) -> np.ndarray:
    w = np.ascontiguousarray(bf16, dtype=np.uint16).reshape(-1)
    if hist is None:
        hist = np.zeros(256, np.uint64)
    assert hist.dtype == np.uint64 and hist.size == 256 and hist.flags["C_CONTIGUOUS"]
    _check("df11_histogram", _load().df11_histogram(_ptr(w), w.size, _ptr(hist), n_threads))
    return hist


def df11_build_codebook(hist: np.ndarray, max_code_len: int = MAX_CODE_LEN) -> Codebook:
    h = np.ascontiguousarray(hist, dtype=np.uint64)
    cb = Codebook()
    _check("df11_build_codebook", _load().df11_build_codebook(_ptr(h), max_code_len,
                                                              ctypes.byref(cb)))
    return cb


def df11_build_luts(cb: Codebook) -> np.ndarray:
    lut = np.zeros(cb.lut_bytes, np.uint8)
    _check("df11_build_luts", _load().df11_build_luts(ctypes.byref(cb), _ptr(lut), lut.size))
    return lut


def df11_encoded_sizes(hist: np.ndarray, n: int, cb: Codebook) -> Sizes:
    h = np.ascontiguousarray(hist, dtype=np.uint64)
    sz = Sizes()
    _check("df11_encoded_sizes", _load().df11_encoded_sizes(_ptr(h), n, ctypes.byref(cb),
                                                            ctypes.byref(sz)))
    return sz


@dataclass
class Encoded:
    """Host copy of every DF11 array for one BF16 tensor."""
    codebook: Codebook
    sizes: Sizes
    stream: np.ndarray      # uint8[stream_bytes]
    gaps: np.ndarray        # uint8[gaps_bytes], packed 5-bit fields
    block_pos: np.ndarray   # uint32[n_blocks + 1]
    signmant: np.ndarray    # uint8[signmant_bytes]
    luts: np.ndarray        # uint8[lut_bytes]

    @property
    def n(self) -> int:
        return int(self.sizes.n)

    def compressed_bytes(self) -> int:
        """Bytes the decoder reads: stream, gaps, block_pos, sign|mantissa, tables."""
        s = self.sizes
        return int(s.stream_bytes + s.gaps_bytes + 4 * s.block_pos_count + s.signmant_bytes
                   + s.lut_bytes)

    def checksum(self) -> int:
        """CRC-32 (zlib's) over the arrays the decoder reads, in the order
        stream, gaps, block_pos, sign|mantissa, tables.  The code stream is
        not self-synchronising (one flipped bit corrupts the rest of its
        block), so a stored artifact carries this value and is checked
        against it when loaded."""
        import zlib
        c = 0
        for arr in (self.stream, self.gaps, self.block_pos, self.signmant, self.luts):
            c = zlib.crc32(np.ascontiguousarray(arr).view(np.uint8), c)
        return c


def df11_encode(bf16: np.ndarray, cb: Codebook, hist: np.ndarray | None = None,
                n_threads: int = 0) -> Encoded:
    w = np.ascontiguousarray(bf16, dtype=np.uint16).reshape(-1)
    if hist is None:
        hist = df11_histogram(w, n_threads=n_threads)
    sz = df11_encoded_sizes(hist, w.size, cb)
    stream = np.empty(sz.stream_bytes, np.uint8)
    gaps = np.empty(sz.gaps_bytes, np.uint8)
    bp = np.empty(sz.block_pos_count, np.uint32)
    sm = np.empty(sz.signmant_bytes, np.uint8)
    out = Sizes()
    _check("df11_encode", _load().df11_encode(
        _ptr(w), w.size, ctypes.byref(cb), _ptr(stream), stream.size, _ptr(gaps), gaps.size,
        _ptr(bp), bp.size, _ptr(sm), sm.size, ctypes.byref(out), n_threads))
    return Encoded(cb, out, stream, gaps, bp, sm, df11_build_luts(cb))


def encode(bf16: np.ndarray, max_code_len: int = MAX_CODE_LEN, n_threads: int = 0) -> Encoded:
    """Histogram -> code book -> tables -> encoded arrays, all on the host."""
    w = np.ascontiguousarray(bf16, dtype=np.uint16).reshape(-1)
    hist = df11_histogram(w, n_threads=n_threads)
    cb = df11_build_codebook(hist, max_code_len)
    return df11_encode(w, cb, hist, n_threads)


# ------------------------------------------------------------ device side

@dataclass
class DeviceEncoded:
    """Device copies of an :class:`Encoded` tensor plus the C descriptor."""
    desc: DeviceStream
    tensors: dict
    n: int

    def compressed_bytes(self) -> int:
        d = self.desc
        return int(d.stream_bytes + d.gaps_bytes + 4 * d.block_pos_count + d.signmant_bytes
                   + d.lut_bytes)


def to_device(enc: Encoded, device="cuda", status=None) -> DeviceEncoded:
    """Copy the encoded arrays to the GPU (torch allocations) and fill a descriptor.

    ``status``: optional int32 device tensor of one element that counts blocks
    whose decoded symbol count disagrees with block_pos."""
    import torch
    t = {
        "stream": torch.from_numpy(enc.stream).to(device),
        "gaps": torch.from_numpy(enc.gaps).to(device),
        "block_pos": torch.from_numpy(enc.block_pos.view(np.int32)).to(device),
        "signmant": torch.from_numpy(enc.signmant).to(device),
        "luts": torch.from_numpy(enc.luts).to(device),
    }
    if status is not None:
        t["status"] = status
    return DeviceEncoded(_descriptor(enc.sizes, enc.codebook, t), t, enc.n)


def _descriptor(sz: Sizes, cb: Codebook, t: dict) -> DeviceStream:
    d = DeviceStream()
    d.stream, d.gaps, d.block_pos = t["stream"].data_ptr(), t["gaps"].data_ptr(), \
        t["block_pos"].data_ptr()
    d.signmant, d.luts = t["signmant"].data_ptr(), t["luts"].data_ptr()
    d.stream_bytes = t["stream"].numel()
    d.gaps_bytes = t["gaps"].numel()
    d.block_pos_count = t["block_pos"].numel()
    d.signmant_bytes = t["signmant"].numel()
    d.lut_bytes = t["luts"].numel()
    d.n, d.total_bits, d.last_start = sz.n, sz.total_bits, sz.last_start
    d.n_blocks, d.n_tables, d.max_len = sz.n_blocks, cb.n_tables, cb.max_len
    d.status = t["status"].data_ptr() if "status" in t else None
    return d


def df11_decode(dev: DeviceEncoded, out, stream=None) -> None:
    """Enqueue the decode of ``dev`` into ``out`` (a CUDA tensor of n bf16/int16
    elements, 16-byte aligned) on ``stream`` (default: torch's current stream)."""
    import torch
    if out.numel() < dev.n or out.element_size() != 2 or not out.is_contiguous():
        raise ValueError("out must be a contiguous 2-byte tensor with at least n elements")
    if stream is None:
        stream = torch.cuda.current_stream(out.device)
    _check("df11_decode", _load().df11_decode(ctypes.byref(dev.desc), out.data_ptr(),
                                              stream.cuda_stream))


def decode(dev: DeviceEncoded, out=None, stream=None):
    """Decode into ``out`` (allocated as bfloat16 if None) and return it."""
    import torch
    if out is None:
        out = torch.empty(dev.n, dtype=torch.bfloat16, device=dev.tensors["stream"].device)
    df11_decode(dev, out, stream)
    return out


# ------------------------------------------------------------ fused GEMV

GEMV_MAX_MATRICES = 16
GEMV_MIN_COLS = 2048


def gemv_matrices(shapes: list[tuple[int, int]]) -> tuple[list[GemvMatrix], int, int]:
    """Matrix list for row-major [rows, cols] matrices laid end to end, each
    with its own slice of x and y (x slices 8-aligned).  Returns (matrices,
    x length, y length)."""
    mats, off, xo, yo = [], 0, 0, 0
    for r, c in shapes:
        mats.append(GemvMatrix(off, r, c, xo, yo))
        off += r * c
        xo += (c + 7) // 8 * 8
        yo += r
    return mats, xo, yo


def df11_gemv_workspace_bytes(dev: DeviceEncoded) -> int:
    return int(_load().df11_gemv_workspace_bytes(ctypes.byref(dev.desc)))


def _matrix_ends(mats: list[GemvMatrix]) -> tuple[int, int]:
    """(elements of x, elements of y) that one vector's matrices reach."""
    x_end = max((int(m.x_offset) + int(m.cols) for m in mats), default=0)
    y_end = max((int(m.y_offset) + int(m.rows) for m in mats), default=0)
    return x_end, y_end


def _same_device(dev: DeviceEncoded, **tensors) -> None:
    where = dev.tensors["stream"].device
    for name, t in tensors.items():
        if t.device != where:
            raise ValueError(f"{name} is on device {t.device}, the encoded tensor on {where}")


def df11_decode_gemv(dev: DeviceEncoded, mats: list[GemvMatrix], x, y, workspace,
                     stream=None) -> None:
    """Enqueue y = W x for every matrix of ``dev`` (x a bfloat16 and y a float32
    CUDA tensor, workspace a CUDA tensor of at least df11_gemv_workspace_bytes
    bytes).  x and y must reach every matrix's inputs and results (the C call
    receives no sizes for them, so they are checked here)."""
    import torch
    if x.dtype != torch.bfloat16 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bfloat16 tensor")
    if y.dtype != torch.float32 or not y.is_contiguous():
        raise ValueError("y must be a contiguous float32 tensor")
    _same_device(dev, x=x, y=y, workspace=workspace)
    x_end, y_end = _matrix_ends(mats)
    if x.numel() < x_end or y.numel() < y_end:
        raise ValueError(f"x holds {x.numel()} and y {y.numel()} elements; the matrices "
                         f"need {x_end} and {y_end}")
    if stream is None:
        stream = torch.cuda.current_stream(y.device)
    arr = (GemvMatrix * len(mats))(*mats)
    nbytes = workspace.numel() * workspace.element_size()
    _check("df11_decode_gemv", _load().df11_decode_gemv(
        ctypes.byref(dev.desc), arr, len(mats), x.data_ptr(), y.data_ptr(),
        workspace.data_ptr(), nbytes, stream.cuda_stream))


def df11_gemm_workspace_bytes(dev: DeviceEncoded, batch: int) -> int:
    return int(_load().df11_gemm_workspace_bytes(ctypes.byref(dev.desc), batch))


def _check_gemm_xy(dev: DeviceEncoded, mats: list[GemvMatrix], x, y) -> None:
    """x [batch, nx] bf16 and y [batch, ny] fp32 with unit column stride, on
    the encoded tensor's device, reaching every matrix's inputs and results
    (the C calls receive no sizes for them)."""
    import torch
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a [batch, nx] bfloat16 tensor with unit column stride")
    if y.dtype != torch.float32 or y.dim() != 2 or y.stride(1) != 1:
        raise ValueError("y must be a [batch, ny] float32 tensor with unit column stride")
    if x.shape[0] != y.shape[0]:
        raise ValueError("x and y must hold the same number of vectors")
    _same_device(dev, x=x, y=y)
    x_end, y_end = _matrix_ends(mats)
    if x.shape[1] < x_end or y.shape[1] < y_end:
        raise ValueError(f"x rows hold {x.shape[1]} and y rows {y.shape[1]} elements; the "
                         f"matrices need {x_end} and {y_end}")


def df11_decode_gemm(dev: DeviceEncoded, mats: list[GemvMatrix], x, y, workspace,
                     stream=None) -> None:
    """Enqueue y[b] = W x[b] for every matrix of ``dev`` and every row b of x
    (x a [batch, nx] bfloat16 and y a [batch, ny] float32 CUDA tensor, batch
    1..8, rows strided by their row stride; workspace a CUDA tensor of at
    least df11_gemm_workspace_bytes(dev, batch) bytes)."""
    import torch
    _check_gemm_xy(dev, mats, x, y)
    _same_device(dev, workspace=workspace)
    if stream is None:
        stream = torch.cuda.current_stream(y.device)
    arr = (GemvMatrix * len(mats))(*mats)
    nbytes = workspace.numel() * workspace.element_size()
    _check("df11_decode_gemm", _load().df11_decode_gemm(
        ctypes.byref(dev.desc), arr, len(mats), x.data_ptr(), x.shape[0], x.stride(0),
        y.data_ptr(), y.stride(0), workspace.data_ptr(), nbytes, stream.cuda_stream))


NOALLOC_SCRATCH_BYTES = 32 << 20


def df11_decode_gemm_noalloc(dev: DeviceEncoded, mats: list[GemvMatrix], x, y,
                             stream=None) -> None:
    """df11_decode_gemm without a workspace argument: the library's static
    device array (NOALLOC_SCRATCH_BYTES per GPU) serves instead, and nothing
    is allocated.  Calls that overlap on one GPU share that array and race."""
    import torch
    _check_gemm_xy(dev, mats, x, y)
    if stream is None:
        stream = torch.cuda.current_stream(y.device)
    arr = (GemvMatrix * len(mats))(*mats)
    _check("df11_decode_gemm_noalloc", _load().df11_decode_gemm_noalloc(
        ctypes.byref(dev.desc), arr, len(mats), x.data_ptr(), x.shape[0], x.stride(0),
        y.data_ptr(), y.stride(0), stream.cuda_stream))


# ------------------------------------------------------------ tiled product

TILED_MAX_BATCH = 64


def _mat_array(mats):
    return (GemvMatrix * len(mats))(*mats)


def df11_tile_order(w: np.ndarray, mats: list[GemvMatrix], n_threads: int = 0) -> np.ndarray:
    """Row-major matrices laid end to end -> the same words in operand-tile
    order (see include/df11.h); host only."""
    w = np.ascontiguousarray(w, dtype=np.uint16).reshape(-1)
    out = np.empty_like(w)
    _check("df11_tile_order", _load().df11_tile_order(_ptr(w), w.size, _mat_array(mats), len(mats),
                                                      _ptr(out), n_threads))
    return out


def df11_tile_segments(block_pos: np.ndarray, mats: list[GemvMatrix]) -> np.ndarray:
    """First block of each 16-row segment, then the block of the last weight."""
    bp = np.ascontiguousarray(block_pos, dtype=np.uint32)
    arr = _mat_array(mats)
    count = int(_load().df11_tile_segment_count(arr, len(mats)))
    seg = np.zeros(count + 1, np.uint32)
    _check("df11_tile_segments", _load().df11_tile_segments(_ptr(bp), bp.size - 1, arr, len(mats),
                                                            _ptr(seg), seg.size))
    return seg


@dataclass
class TiledEncoded:
    """A block of matrices encoded in operand-tile order for the tiled
    product: the encoded arrays, the matrix list and the segment table."""
    enc: Encoded
    mats: list
    seg_blk: np.ndarray


def encode_tiled(bf16: np.ndarray, shapes: list[tuple[int, int]], max_code_len: int = MAX_CODE_LEN,
                 n_threads: int = 0) -> TiledEncoded:
    """Row-major [rows, cols] matrices laid end to end (rows multiples of 16,
    cols of 32) -> tile order -> DF11 arrays, plus the segment table."""
    mats, _, _ = gemv_matrices(shapes)
    tiled = df11_tile_order(bf16, mats, n_threads)
    enc = encode(tiled, max_code_len, n_threads)
    return TiledEncoded(enc, mats, df11_tile_segments(enc.block_pos, mats))


@dataclass
class TiledDevice:
    dev: DeviceEncoded
    mats: list
    seg_blk: object  # device tensor (int32 view of the uint32 table)


def tiled_to_device(te: TiledEncoded, device="cuda", status=None) -> TiledDevice:
    import torch
    dev = to_device(te.enc, device, status)
    seg = torch.from_numpy(te.seg_blk.view(np.int32)).to(device)
    return TiledDevice(dev, te.mats, seg)


def df11_tiled_workspace_bytes(mats: list[GemvMatrix], batch: int) -> int:
    return int(_load().df11_tiled_workspace_bytes(_mat_array(mats), len(mats), batch))


def df11_decode_gemm_tiled(td: TiledDevice, x, y, workspace=None, stream=None) -> None:
    """Enqueue y[b] = W x[b] for every matrix and every row b of x (batch
    1..64) from a tile-order stream, on the matrix cores (x [batch, nx]
    bfloat16, y [batch, ny] float32, unit column stride; workspace a CUDA
    tensor of at least df11_tiled_workspace_bytes bytes, None when that is 0)."""
    import torch
    _check_gemm_xy(td.dev, td.mats, x, y)
    _same_device(td.dev, seg_blk=td.seg_blk)
    need = df11_tiled_workspace_bytes(td.mats, x.shape[0])
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        _same_device(td.dev, workspace=workspace)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if ws_bytes < need:
        raise ValueError(f"the tiled product needs a workspace of {need} bytes")
    if stream is None:
        stream = torch.cuda.current_stream(y.device)
    _check("df11_decode_gemm_tiled", _load().df11_decode_gemm_tiled(
        ctypes.byref(td.dev.desc), _mat_array(td.mats), len(td.mats), td.seg_blk.data_ptr(),
        x.data_ptr(), x.shape[0], x.stride(0), y.data_ptr(), y.stride(0), ws_ptr, ws_bytes,
        stream.cuda_stream))


def df11_decode_tiled(td: TiledDevice, out, stream=None) -> None:
    """Enqueue the decode of a tile-order stream into ``out`` (a CUDA tensor of
    at least n 16-bit elements), in the row-major order the weights had
    before df11_tile_order."""
    import torch
    if out.element_size() != 2 or not out.is_contiguous() or out.numel() < td.dev.n:
        raise ValueError("out must be a contiguous 16-bit tensor of at least n elements")
    _same_device(td.dev, out=out)
    if stream is None:
        stream = torch.cuda.current_stream(out.device)
    _check("df11_decode_tiled", _load().df11_decode_tiled(
        ctypes.byref(td.dev.desc), _mat_array(td.mats), len(td.mats), out.data_ptr(),
        stream.cuda_stream))


# ------------------------------------------------------------ measurement aid

def df11_stream_ceiling(a, b, out, n: int, max_groups: int = 0, stream=None) -> None:
    """Enqueue the traffic-only kernel: reads a[0..n) bytes and all of b,
    writes n 16-bit words to out (see include/df11.h).  a, b, out are CUDA
    tensors (b may be None)."""
    import torch
    b_bytes = 0 if b is None else b.numel() * b.element_size()
    if a.numel() * a.element_size() < n or out.numel() * out.element_size() < 2 * n:
        raise ValueError("a or out is smaller than n")
    if stream is None:
        stream = torch.cuda.current_stream(out.device)
    _check("df11_stream_ceiling", _load().df11_stream_ceiling(
        a.data_ptr(), 0 if b is None else b.data_ptr(), b_bytes, out.data_ptr(), n, max_groups,
        stream.cuda_stream))


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def df11_stream_read_slots(nbytes: int, grid: int = 0) -> int:
    return int(_load().df11_stream_read_slots(nbytes, grid))


def df11_stream_read(src, out, nbytes: int, grid: int = 0, stream=None) -> None:
    """Enqueue the read-only stream over src[0..nbytes) (CUDA tensors; out an
    int32/uint32 tensor of at least df11_stream_read_slots(nbytes, grid)
    elements, receiving one XOR of 32-bit words per thread)."""
    import torch
    if _nbytes(src) < nbytes:
        raise ValueError("src is smaller than nbytes")
    if out.element_size() != 4:
        raise ValueError("out must hold 32-bit words")
    if stream is None:
        stream = torch.cuda.current_stream(src.device)
    _check("df11_stream_read", _load().df11_stream_read(
        src.data_ptr(), nbytes, out.data_ptr(), out.numel(), grid, stream.cuda_stream))


def df11_stream_write(dst, nbytes: int, value: int = 0, grid: int = 0, stream=None) -> None:
    """Enqueue the write-only stream over dst[0..nbytes) (a CUDA tensor)."""
    import torch
    if _nbytes(dst) < nbytes:
        raise ValueError("dst is smaller than nbytes")
    if stream is None:
        stream = torch.cuda.current_stream(dst.device)
    _check("df11_stream_write", _load().df11_stream_write(
        dst.data_ptr(), nbytes, value & 0xFFFFFFFF, grid, stream.cuda_stream))


def df11_stream_copy(src, dst, nbytes: int, grid: int = 0, stream=None) -> None:
    """Enqueue dst[0..nbytes) = src[0..nbytes) (CUDA tensors)."""
    import torch
    if _nbytes(src) < nbytes or _nbytes(dst) < nbytes:
        raise ValueError("src or dst is smaller than nbytes")
    if stream is None:
        stream = torch.cuda.current_stream(dst.device)
    _check("df11_stream_copy", _load().df11_stream_copy(
        src.data_ptr(), dst.data_ptr(), nbytes, grid, stream.cuda_stream))
