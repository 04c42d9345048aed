"""Pins of the oracle's temporal convolution with its chunk-boundary cache
(``oracle.temporal_conv_chunk`` / ``temporal_conv_stream``), against things
other than its own formula: numpy's convolution, delta-kernel closed forms,
the separately written visibility-masked sum over the whole sequence, and
the block-causal rule ("Nvidia, MIT ve diğerleri video yapay zeka devrimini
başlattı", section "Sabit Bellekli KV önbelleğe alma mekanizması": later
blocks read earlier ones, never the reverse).  ``test_tconv_mutants_caught``
plants plausible mistakes in the chunk function and checks pins catch each.
"""

import numpy as np
import pytest

import oracle

_chunk = oracle.temporal_conv_chunk


def _case(seed, B=2, F=7, P=3, C=5):
    g = np.random.default_rng(seed)
    return (g.standard_normal((B, F, P, C)), g.standard_normal((C, 3)), g.standard_normal(C),
            g.standard_normal((B, P, C)))


def pin_numpy_convolve():
    """One chunk, no cache, no bias: per (b, p, c) the 'same'-size
    convolution with the reversed taps."""
    x, w, _, _ = _case(1)
    y, _ = oracle.temporal_conv_chunk(x, w)
    B, F, P, C = x.shape
    for b in range(B):
        for p in range(P):
            for c in range(C):
                ref = np.convolve(x[b, :, p, c], w[c, ::-1], mode="same")
                assert np.allclose(y[b, :, p, c], ref, rtol=1e-14, atol=1e-14)


def pin_delta_kernels():
    """Taps (0,1,0): identity plus bias; (1,0,0): the previous frame (the
    cache for frame 0); (0,0,1): the next frame, zero for the last frame of
    the chunk."""
    x, _, bias, cache = _case(2)
    C = x.shape[-1]
    e = np.eye(3)
    y, out_cache = oracle.temporal_conv_chunk(x, np.tile(e[1], (C, 1)), bias, cache)
    assert np.array_equal(y, x + bias)
    assert np.array_equal(out_cache, x[:, -1])
    y, _ = oracle.temporal_conv_chunk(x, np.tile(e[0], (C, 1)), None, cache)
    assert np.array_equal(y[:, 0], cache) and np.array_equal(y[:, 1:], x[:, :-1])
    y, _ = oracle.temporal_conv_chunk(x, np.tile(e[2], (C, 1)), None, cache)
    assert np.array_equal(y[:, :-1], x[:, 1:]) and np.all(y[:, -1] == 0.0)


def pin_stream_equals_masked_sum():
    """Carrying the one-frame cache across chunks gives the whole-sequence
    masked sum, for several chunkings (including one-frame chunks)."""
    x, w, bias, cache = _case(3, F=11)
    for Tf in (1, 2, 4, 11, 20):
        chunks = [x[:, f:f + Tf] for f in range(0, x.shape[1], Tf)]
        outs, caches = oracle.temporal_conv_stream(chunks, w, bias, cache)
        ref = oracle.temporal_conv_blockcausal(x, w, bias, Tf, cache)
        assert np.allclose(np.concatenate(outs, axis=1), ref, rtol=1e-13, atol=1e-13), Tf
        assert np.array_equal(caches[-1], x[:, -1])


def pin_no_future_and_boundary_response():
    """A chunk's outputs do not change when the next chunk changes; a change
    d in the last frame of a chunk changes the next chunk's first output by
    exactly w0 d and nothing else of it."""
    x, w, bias, cache = _case(4, F=6)
    c1, c2 = x[:, :3], x[:, 3:]
    y1, k1 = oracle.temporal_conv_chunk(c1, w, bias, cache)
    y1b, _ = oracle.temporal_conv_chunk(c1, w, bias, cache)
    assert np.array_equal(y1, y1b)
    y2, _ = oracle.temporal_conv_chunk(c2, w, bias, k1)
    d = np.random.default_rng(9).standard_normal(k1.shape)
    c1p = c1.copy()
    c1p[:, -1] += d
    _, k1p = oracle.temporal_conv_chunk(c1p, w, bias, cache)
    y2p, _ = oracle.temporal_conv_chunk(c2, w, bias, k1p)
    assert np.allclose(y2p[:, 0] - y2[:, 0], w[:, 0] * d, rtol=1e-12, atol=1e-12)
    assert np.array_equal(y2p[:, 1:], y2[:, 1:])


def pin_linearity():
    """Without bias the output is linear in x (and in the cache) and in w."""
    x1, w, _, c1 = _case(5)
    x2, w2, _, c2 = _case(6)
    a, b = 0.75, -1.5
    y, _ = oracle.temporal_conv_chunk(a * x1 + b * x2, w, None, a * c1 + b * c2)
    ya, _ = oracle.temporal_conv_chunk(x1, w, None, c1)
    yb, _ = oracle.temporal_conv_chunk(x2, w, None, c2)
    assert np.allclose(y, a * ya + b * yb, rtol=1e-12, atol=1e-12)
    yw, _ = oracle.temporal_conv_chunk(x1, a * w + b * w2, None, c1)
    yw2, _ = oracle.temporal_conv_chunk(x1, w2, None, c1)
    assert np.allclose(yw, a * ya + b * yw2, rtol=1e-12, atol=1e-12)


def pin_empty_chunk():
    """No frames: no output and the cache passes through."""
    _, w, bias, cache = _case(7)
    y, k = oracle.temporal_conv_chunk(np.zeros((2, 0, 3, 5)), w, bias, cache)
    assert y.shape == (2, 0, 3, 5) and np.array_equal(k, cache)


PINS = [pin_numpy_convolve, pin_delta_kernels, pin_stream_equals_masked_sum,
        pin_no_future_and_boundary_response, pin_linearity, pin_empty_chunk]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_tconv_pin(pin):
    pin()


def _mut_flipped_taps(x, w, b=None, cache=None):
    return _chunk(x, np.asarray(w)[:, ::-1], b, cache)


def _mut_next_chunk_visible(x, w, b=None, cache=None):
    # uses the chunk's own last frame again instead of zero past the end
    x = np.asarray(x, dtype=np.float64)
    y, k = _chunk(x, w, b, cache)
    if x.shape[1] > 0:
        y = y.copy()
        y[:, -1] += np.asarray(w)[:, 2] * x[:, -1]
    return y, k


def _mut_cache_ignored(x, w, b=None, cache=None):
    return _chunk(x, w, b, None)


def _mut_cache_first_frame(x, w, b=None, cache=None):
    x = np.asarray(x, dtype=np.float64)
    y, k = _chunk(x, w, b, cache)
    return y, (x[:, 0] if x.shape[1] > 0 else k)


def _mut_no_bias(x, w, b=None, cache=None):
    return _chunk(x, w, None, cache)


MUTANTS = {
    "flipped_taps": _mut_flipped_taps,
    "next_chunk_visible": _mut_next_chunk_visible,
    "cache_ignored": _mut_cache_ignored,
    "cache_first_frame": _mut_cache_first_frame,
    "no_bias": _mut_no_bias,
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_tconv_mutants_caught(name, monkeypatch):
    monkeypatch.setattr(oracle, "temporal_conv_chunk", MUTANTS[name])
    caught = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
    print(f"[mutant] {name} caught by {caught}")
