"""Generators of BF16 inputs for the property tests (seeded numpy draws
shaped by hypothesis; no part of the method's arithmetic)."""
import numpy as np
from hypothesis import strategies as st


@st.composite
def bf16_words(draw, max_n=12_000):
    """Flat BF16 bit patterns: exponents geometric (long code tails), from a
    few values, Zipf over a random subset, or any 16-bit word at all."""
    n = draw(st.integers(1, max_n))
    seed = draw(st.integers(0, 2**31 - 1))
    kind = draw(st.sampled_from(["geometric", "few", "subset", "any"]))
    rng = np.random.default_rng(seed)
    if kind == "any":
        return rng.integers(0, 1 << 16, n, dtype=np.uint32).astype(np.uint16)
    if kind == "geometric":
        p = draw(st.floats(0.05, 0.95))
        e = 127 - np.minimum(rng.geometric(p, n) - 1, 120)
    elif kind == "few":
        k = draw(st.integers(1, 3))
        e = rng.choice(rng.integers(0, 256, k), n)
    else:
        k = draw(st.integers(2, 60))
        pool = rng.choice(256, k, replace=False)
        e = pool[np.minimum(rng.zipf(1.6, n) - 1, k - 1)]
    sm = rng.integers(0, 256, n)
    return (((sm & 0x80) << 8) | (e.astype(np.int64) << 7) | (sm & 0x7F)).astype(np.uint16)
