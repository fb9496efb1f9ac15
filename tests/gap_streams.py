"""A constructed BF16 stream whose gap fields take every value 0..31 and
whose code book has 32-bit codes: the Fibonacci exponent histogram (exponent
121 - j with count F(33 - j), j = 0..32) laid out so that, for each v in
1..31, a code of more than v bits ends exactly v bits into a 64-bit slice.
Shared by the host and the GPU tests; holds no codec arithmetic beyond the
code lengths the library's code book gives."""
import numpy as np


def fibonacci_hist(k: int = 33) -> np.ndarray:
    fib = [1, 1]
    while len(fib) < k + 1:
        fib.append(fib[-1] + fib[-2])
    hist = np.zeros(256, np.uint64)
    for j in range(k):
        hist[121 - j] = fib[k - 1 - j]
    return hist


def every_gap_stream(code_lengths: np.ndarray, hist: np.ndarray, seed: int = 7) -> np.ndarray:
    """Exponent sequence with histogram `hist` (lengths `code_lengths` from
    its code book) arranged so that codes end at every offset 1..31 of some
    slice, then the rest shuffled; returned as BF16 words with random
    sign|mantissa bytes."""
    rng = np.random.default_rng(seed)
    left = hist.astype(np.int64).copy()
    ln = code_lengths.astype(np.int64)
    one = int(np.argmax(np.where(left > 0, (ln == 1) * left, 0)))  # the 1-bit symbol
    assert ln[one] == 1
    seq, pos = [], 0
    for v in range(1, 32):
        # a symbol whose code is longer than v bits, still available
        cands = [s for s in range(256) if left[s] > 0 and ln[s] > v and s != one]
        s = min(cands, key=lambda c: (ln[c], c))
        start = (v - int(ln[s])) % 64  # the code then ends v bits into the next slice
        while pos % 64 != start:
            seq.append(one)
            left[one] -= 1
            pos += 1
        seq.append(s)
        left[s] -= 1
        pos += int(ln[s])
        assert left[one] >= 0 and left[s] >= 0
    rest = np.repeat(np.arange(256), left)
    rng.shuffle(rest)
    e = np.concatenate([np.array(seq, np.int64), rest]).astype(np.uint16)
    low = rng.integers(0, 256, e.size).astype(np.uint16)
    return (((low & 0x80) << 8) | (e << 7) | (low & 0x7F)).astype(np.uint16)


def gap_values(gaps_packed: np.ndarray, count: int) -> np.ndarray:
    """The first `count` 5-bit fields of a packed gaps array (LSB-first)."""
    bits = np.unpackbits(gaps_packed, bitorder="little")[: 5 * count].reshape(-1, 5)
    return (bits.astype(np.int64) << np.arange(5)).sum(1)
