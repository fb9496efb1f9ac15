"""Seeded synthetic BF16 weight sets for the DF11 decode path.

This module only draws numbers and rounds them to BF16: it holds none of the
codec's arithmetic, so the product path, the oracle tests and the benchmark can
all share it.  Every generator is deterministic in its seed.

The shapes stand in for real checkpoints the DF11 pages measure (Llama 3.1 8B,
Llama 3.3 70B, FLUX.1; page "DFloat11: lossless BFloat16 compression", section
"What it is", compression table).  No checkpoint is read: values are drawn from
the distributions stated per workload below.

Recipes (numpy PCG64 ``default_rng``; float32 draws rounded to nearest-even BF16;
row-major ``[out, in]`` matrices concatenated in the listed order).  Each matrix
is drawn in chunks of 2**22 elements, chunk c of matrix m from
``default_rng([*seed, m, c])``, so generation runs on several threads and the
result does not depend on their number:

* ``linear_4096``: one 4096x4096 matrix, N(0, 0.02).
* ``llama8b_block``: q, k, v, o, gate, up, down of an 8B-class block
  (q/o 4096x4096, k/v 1024x4096, gate/up 14336x4096, down 4096x14336),
  N(0, sigma_m) with sigma_m = 0.02 * 2**U(-1, 1) drawn per matrix.
* ``llama70b_block``: same layout at hidden 8192, MLP 28672, k/v 1024x8192,
  N(0, 0.015).
* ``flux_block``: q, k, v, o 3072x3072, mlp_in 12288x3072, mlp_out
  3072x12288; 0.02 * Student-t(3) plus round(1e-4 * n) outliers of magnitude
  10**U(2, 4) with random sign at distinct random positions.
* ``fibonacci_exponents``: exponent bytes 121 - j with counts F(k - j)
  (Fibonacci, F(1) = F(2) = 1), the remainder of n added to exponent 121,
  uniformly random sign|mantissa, seeded shuffle.  k = 33 gives a 32-bit
  longest Huffman code, k = 34 a 33-bit one that the length limit must cut.
* ``all_exponents``: N(0, 0.02) with every one of the 256 exponent values
  planted (zeros, subnormals, infinities and NaN payloads included).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK = 1 << 22


def to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bit patterns (uint16), round to nearest, ties to even.

    NaNs map to a quiet NaN of the same sign (plain RNE on the bit pattern
    would carry a NaN's payload into the exponent or sign)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # only NaN patterns can wrap around 2**32 here; they are replaced below
    rounded = ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))))
               >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = ((u[nan] >> np.uint32(16)) & np.uint32(0x8000)).astype(np.uint16) | 0x7FC0
    return rounded


@dataclass
class Matrix:
    name: str
    rows: int
    cols: int
    offset: int  # first element in the flat block

    @property
    def numel(self) -> int:
        return self.rows * self.cols


@dataclass
class Workload:
    name: str
    weights: np.ndarray                     # flat uint16 BF16 bit patterns
    matrices: list[Matrix] = field(default_factory=list)

    @property
    def n(self) -> int:
        return int(self.weights.size)


def _layout(shapes: list[tuple[str, int, int]]) -> list[Matrix]:
    out, off = [], 0
    for name, r, c in shapes:
        out.append(Matrix(name, r, c, off))
        off += r * c
    return out


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _fill_chunks(out: np.ndarray, seed: list, draw) -> None:
    """out[c*CHUNK:(c+1)*CHUNK] = to_bf16(draw(default_rng(seed + [c]), size))."""
    n = out.size

    def one(c):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        out[lo:hi] = to_bf16(draw(np.random.default_rng(seed + [c]), hi - lo))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(-(-n // CHUNK))))


def _normal_bf16(seed: list, count: int, sigma: float, out: np.ndarray) -> None:
    s = np.float32(sigma)

    def draw(rng, size):
        x = rng.standard_normal(size, dtype=np.float32)
        x *= s
        return x

    _fill_chunks(out[:count], seed, draw)


LLAMA8B_SHAPES = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
                  ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336)]
LLAMA70B_SHAPES = [("q", 8192, 8192), ("k", 1024, 8192), ("v", 1024, 8192), ("o", 8192, 8192),
                   ("gate", 28672, 8192), ("up", 28672, 8192), ("down", 8192, 28672)]
FLUX_SHAPES = [("q", 3072, 3072), ("k", 3072, 3072), ("v", 3072, 3072), ("o", 3072, 3072),
               ("mlp_in", 12288, 3072), ("mlp_out", 3072, 12288)]


def normal_block(name: str, shapes: list[tuple[str, int, int]], seed, sigma: float = 0.02,
                 jitter: bool = False, scale: float = 1.0) -> Workload:
    """Matrices of N(0, sigma) weights; with jitter, sigma_m = sigma * 2**U(-1, 1) per matrix.

    ``scale`` < 1 shrinks every matrix's row count (for fast reduced tests)."""
    mats = _layout([(nm, max(1, int(r * scale)), c) for nm, r, c in shapes])
    total = sum(m.numel for m in mats)
    w = np.empty(total, np.uint16)
    seed = list(seed) if isinstance(seed, (tuple, list)) else [seed]
    for i, m in enumerate(mats):
        s = sigma
        if jitter:
            s = sigma * float(2.0 ** np.random.default_rng(seed + [i]).uniform(-1, 1))
        _normal_bf16(seed + [i], m.numel, s, w[m.offset:m.offset + m.numel])
    return Workload(name, w, mats)


def linear_4096(seed: int = 1001) -> Workload:
    return normal_block("linear_4096", [("w", 4096, 4096)], seed, 0.02)


def llama8b_block(seed=2001, scale: float = 1.0) -> Workload:
    return normal_block("llama8b_block", LLAMA8B_SHAPES, seed, 0.02, jitter=True, scale=scale)


def llama8b_stack_block(layer: int, seed: int = 3001) -> Workload:
    wl = normal_block("llama8b_block", LLAMA8B_SHAPES, (seed, layer), 0.02, jitter=True)
    wl.name = f"llama8b_stack_layer{layer}"
    return wl


def llama70b_block(seed: int = 4001, scale: float = 1.0) -> Workload:
    return normal_block("llama70b_block", LLAMA70B_SHAPES, seed, 0.015, scale=scale)


def flux_block(seed: int = 5001, scale: float = 1.0) -> Workload:
    """Heavy-tailed block: 0.02 * Student-t(3) plus 0.01 % large outliers."""
    mats = _layout([(nm, max(1, int(r * scale)), c) for nm, r, c in FLUX_SHAPES])
    total = sum(m.numel for m in mats)
    w = np.empty(total, np.uint16)
    _fill_chunks(w, [seed, 0],
                 lambda rng, size: rng.standard_t(3.0, size).astype(np.float32) * np.float32(0.02))
    rng = np.random.default_rng([seed, 1])
    n_out = int(round(1e-4 * total))
    pos = rng.choice(total, size=n_out, replace=False)
    mag = 10.0 ** rng.uniform(2.0, 4.0, n_out)
    sign = np.where(rng.integers(0, 2, n_out) == 1, -1.0, 1.0)
    w[pos] = to_bf16((mag * sign).astype(np.float32))
    return Workload("flux_block", w, mats)


def fibonacci_exponents(k: int = 33, seed: int = 5002, rows: int = 4096, cols: int = 4096
                        ) -> Workload:
    """Exponent counts F(1..k) on exponents 121-(k-1) .. 121, remainder on 121."""
    n = rows * cols
    fib = [1, 1]
    while len(fib) < k:
        fib.append(fib[-1] + fib[-2])
    # exponent 121 - j gets F(k - j): j = 0 is the most frequent
    counts = {121 - j: fib[k - 1 - j] for j in range(k)}
    used = sum(counts.values())
    if used > n:
        raise ValueError("tensor too small for this many Fibonacci counts")
    counts[121] += n - used
    rng = np.random.default_rng(seed)
    expo = np.concatenate([np.full(c, e, np.uint16) for e, c in sorted(counts.items())])
    rng.shuffle(expo)
    low = rng.integers(0, 256, n, dtype=np.uint16)        # sign|mantissa byte
    w = ((low & 0x80) << 8) | (expo << 7) | (low & 0x7F)
    return Workload(f"fibonacci_{k}", w.astype(np.uint16), _layout([("w", rows, cols)]))


SPECIAL_PATTERNS = [0x0000, 0x8000, 0x0001, 0x807F, 0x007F, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1,
                    0x7F81, 0x7FFF, 0xFFFF, 0x0080, 0x8080, 0x7F7F, 0xFF7F]


def all_exponents(seed: int = 5004, rows: int = 4096, cols: int = 4096) -> Workload:
    """N(0, 0.02) with all 256 exponent values planted at random positions."""
    n = rows * cols
    w = np.empty(n, np.uint16)
    _normal_bf16([seed, 0], n, 0.02, w)
    rng = np.random.default_rng([seed, 1])
    per = 3
    planted = np.repeat(np.arange(256, dtype=np.uint16), per)
    low = rng.integers(0, 256, planted.size, dtype=np.uint16)
    patt = ((low & 0x80) << 8) | (planted << 7) | (low & 0x7F)
    patt = np.concatenate([patt, np.array(SPECIAL_PATTERNS, np.uint16)]).astype(np.uint16)
    pos = rng.choice(n, size=patt.size, replace=False)
    w[pos] = patt
    return Workload("all_exponents", w, _layout([("w", rows, cols)]))


def random_small(n: int, seed: int, kind: str = "normal") -> np.ndarray:
    """Small flat tensors for edge cases: 'normal', 'single', 'uniform', 'int8',
    and 'geometric' / 'geometric_steep': exponent 127 - j with probability
    proportional to 0.45^j / 0.3^j (codes of about 2 / 1.4 bits on average,
    so 30-45 codes start in a 64-bit slice), random sign|mantissa."""
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return to_bf16((rng.standard_normal(n) * 0.02).astype(np.float32))
    if kind == "single":
        low = rng.integers(0, 256, n, dtype=np.uint16)
        return (((low & 0x80) << 8) | (np.uint16(0x7C) << 7) | (low & 0x7F)).astype(np.uint16)
    if kind == "uniform":
        return rng.integers(0, 1 << 16, n, dtype=np.uint16).astype(np.uint16)
    if kind == "int8":
        return to_bf16((rng.integers(-127, 128, n) * (0.02 / 127)).astype(np.float32))
    if kind in ("geometric", "geometric_steep"):
        q = 0.45 if kind == "geometric" else 0.3
        j = np.minimum(rng.geometric(1.0 - q, n) - 1, 120).astype(np.uint16)
        low = rng.integers(0, 256, n, dtype=np.uint16)
        return (((low & 0x80) << 8) | ((127 - j) << 7) | (low & 0x7F)).astype(np.uint16)
    raise ValueError(kind)


CONFIGS = {
    "linear_4096": linear_4096,
    "llama8b_block": llama8b_block,
    "llama70b_block": llama70b_block,
    "flux_block": flux_block,
    "fibonacci_33": lambda: fibonacci_exponents(33, 5002),
    "fibonacci_34": lambda: fibonacci_exponents(34, 5003),
    "all_exponents": all_exponents,
}
