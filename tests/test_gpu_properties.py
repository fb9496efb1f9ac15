"""Property tests on the GPU: generated inputs through df11_decode (the
result must be the original words, bit for bit) and generated matrix lists
and batches through the tiled product in its exact mode (every sum must
equal numpy's fp64 product bit for bit), and generated matrix lists through
the tile-order encoding and its decode back to row-major (bit for bit).  Each
case prints what it runs."""
import numpy as np
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings, strategies as st  # noqa: E402

import huffman_decode_amd as hd  # noqa: E402
from gen_words import bf16_words  # noqa: E402
from test_gpu_parity import _gpu_decode  # noqa: E402
from test_gpu_tiled import _check, _exact_weights  # noqa: E402

pytestmark = pytest.mark.gpu

_SETTINGS = dict(deadline=None, database=None, derandomize=True,
                 suppress_health_check=[HealthCheck.function_scoped_fixture,
                                        HealthCheck.too_slow])


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


@settings(max_examples=100, **_SETTINGS)
@given(w=bf16_words(max_n=200_000), cap=st.integers(20, 32))
def test_decode_generated_inputs(torch, w, cap):
    enc = hd.encode(w, max_code_len=cap)
    got = _gpu_decode(torch, enc, f"generated cap={cap}")
    assert np.array_equal(got, w)


@st.composite
def matrix_lists(draw):
    k = draw(st.integers(1, 4))
    shapes = [(16 * draw(st.integers(1, 8)), 32 * draw(st.integers(1, 128))) for _ in range(k)]
    return shapes


@settings(max_examples=60, **_SETTINGS)
@given(shapes=matrix_lists(), batch=st.integers(1, 64), seed=st.integers(0, 10_000),
       kind=st.sampled_from(["normal", "single", "geometric"]))
def test_tiled_generated_shapes_exact(torch, shapes, batch, seed, kind):
    w = _exact_weights(sum(r * c for r, c in shapes), seed, kind)
    # keep every row's sum of |w| below 2^9: |w| < 2^(e - 126) for exponent
    # field e, so cols |w| < 2^9 once e <= 135 - log2(cols), cols rounded up
    # to a power of two
    e_max = min(254, 135 - int(np.ceil(np.log2(max(c for _, c in shapes)))))
    big = ((w >> 7) & 0xFF) > e_max
    w[big] = (w[big] & 0x807F) | np.uint16(e_max << 7)
    _check(torch, w, shapes, batch, f"generated {shapes} {kind}", exact=True, seed=seed)


@settings(max_examples=50, **_SETTINGS)
@given(shapes=matrix_lists(), seed=st.integers(0, 10_000),
       kind=st.sampled_from(["normal", "single", "uniform", "geometric"]))
def test_decode_tiled_generated_shapes(torch, shapes, seed, kind):
    """Generated matrix lists through the tile-order encoding and back: the
    decode to row-major must give the original words bit for bit."""
    from huffman_decode_amd import workloads as wl
    from test_gpu_decode_tiled import _decode_tiled
    w = wl.random_small(sum(r * c for r, c in shapes), seed, kind)
    te = hd.encode_tiled(w, shapes)
    assert np.array_equal(_decode_tiled(torch, te, f"generated {shapes} {kind}"), w)
