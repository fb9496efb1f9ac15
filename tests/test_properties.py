"""Property tests of the host encoder against the oracle on generated inputs
(lengths, exponent distributions, code-length limits): whatever the input,
the product's arrays decode back to it bit for bit through the oracle's
bit-by-bit decoder, and each array equals what the oracle computes from its
definition."""
import math

import numpy as np
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

import huffman_decode_amd as hd  # noqa: E402
import oracle  # noqa: E402
from gen_words import bf16_words  # noqa: E402


@settings(max_examples=600, deadline=None, database=None, derandomize=True)
@given(w=bf16_words(), slack=st.integers(0, 31))
def test_encoder_output_decodes_back_and_matches_the_oracle(w, slack):
    e, _ = oracle.split_bf16(w)
    hist = oracle.histogram(e)
    n_sym = int((hist > 0).sum())
    floor = max(1, math.ceil(math.log2(n_sym))) if n_sym > 1 else 1
    max_len = min(32, floor + slack)
    enc = hd.encode(w, max_code_len=max_len)
    lengths = enc.codebook.lengths
    s = enc.sizes
    n, total, nb = int(s.n), int(s.total_bits), int(s.n_blocks)
    assert n == w.size and int(lengths.max()) <= max_len
    # the code book: the oracle's limited lengths, a complete prefix code
    want_len, _ = oracle.limited_lengths(hist, max_len)
    assert np.array_equal(lengths, want_len)
    used = lengths[hist > 0].astype(np.int64)
    if n_sym > 1:
        assert sum(2.0 ** -int(x) for x in used) == 1.0
    assert total == int((hist.astype(np.int64) * lengths.astype(np.int64)).sum())
    # the stream decodes back through the oracle, bit by bit
    ex, end = oracle.decode(enc.stream, total, 0, n, lengths)
    assert end == total
    assert np.array_equal(oracle.join_bf16(ex, enc.signmant[:n]), w)
    # gaps and block positions by definition
    gaps, bp = oracle.aux(e, lengths, 64 * nb + 1, nb + 1)
    assert np.array_equal(enc.block_pos[: nb + 1], bp)
    assert np.array_equal(enc.gaps[: s.gaps_bytes], oracle.pack_gaps(gaps, int(s.gaps_bytes)))
    # every block decodes on its own from its first slice's gap
    for b in sorted({0, nb // 2, nb - 1}):
        start = 4096 * b + int(gaps[64 * b])
        stop = 4096 * (b + 1) if b + 1 < nb else total
        got = oracle.decode_range(enc.stream, total, start, stop, lengths,
                                  int(bp[b + 1]) - int(bp[b]))
        assert np.array_equal(got, e[int(bp[b]): int(bp[b + 1])])
