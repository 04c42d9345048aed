"""GPU parity of the Mix-FFN temporal convolution with its chunk-boundary
cache (la_temporal_conv_chunk, la_temporal_conv_blockcausal, through the C
ABI) against the fp64 oracle on the same seeded inputs.

Error: normwise per (b, frame) slice.  Bounds derived from the arithmetic:
a float32 output is three fused multiply-adds of exact inputs (x is bf16 or
float32, the taps float32), so its error is a few float32 ulps of the
largest term: 1e-5; a bfloat16 output adds one rounding: 2^-8.  The cache
out is a copy of the last frame and must match bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import BF16_MISMATCH_MAX, bf16_rounding, dev, host, normwise, report

import block_causal_linear_amd as la

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-5, "bf16": 2.0 ** -8}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.lib()
    yield
    torch.cuda.synchronize()


def tdev(a, dtype):
    return dev(a, dtype)


def err(got, ref):
    return normwise(got, ref, axes=(2, 3))


@pytest.mark.parametrize("xdt", ["bf16", "f32"])
@pytest.mark.parametrize("ydt", ["bf16", "f32"])
@pytest.mark.parametrize("F,P,C", [(1, 7, 8), (5, 36, 64), (21, 13, 200)])
@pytest.mark.parametrize("with_cache", [True, False])
def test_tconv_chunk_small(xdt, ydt, F, P, C, with_cache):
    B = 2
    x, w, b, cache = workloads.random_tconv(11 + F + C, B, F, P, C, dtype=xdt)
    ci = tdev(cache, xdt) if with_cache else None
    y, co = la.temporal_conv_chunk(tdev(x, xdt), dev(w, "f32"), dev(b, "f32") if with_cache else None,
                                   cache_in=ci, out_dtype=torch.bfloat16 if ydt == "bf16" else torch.float32)
    torch.cuda.synchronize()
    ref, ref_cache = oracle.temporal_conv_chunk(x, w, b if with_cache else None,
                                                cache if with_cache else None)
    e = err(host(y), ref)
    report(f"tconv chunk x={xdt} y={ydt} F={F} P={P} C={C} cache={with_cache}", y=e)
    assert e <= TOL[ydt], e
    if ydt == "bf16":
        # against the oracle rounded to bf16 (ties to even), per (b, frame)
        excess, mismatch = bf16_rounding(host(y), ref, (2, 3), 1e-5)
        report("tconv bf16 rounding", ulp_excess=excess, mismatch=mismatch)
        assert excess <= 0.0 and mismatch <= BF16_MISMATCH_MAX, (excess, mismatch)
    assert np.array_equal(host(co), ref_cache)


@pytest.mark.parametrize("xdt", ["bf16", "f32"])
def test_tconv_stream_in_place_cache(xdt):
    """Three chunks with the cache updated in place between them."""
    B, F, P, C = 1, 6, 20, 64
    _, w, b, cache = workloads.random_tconv(21, B, F, P, C, dtype=xdt)
    chunks = [workloads.random_tconv(21, B, F, P, C, dtype=xdt, chunk=n)[0] for n in range(3)]
    c = tdev(cache, xdt)
    wt, bt = dev(w, "f32"), dev(b, "f32")
    outs = []
    for xc in chunks:
        y, c = la.temporal_conv_chunk(tdev(xc, xdt), wt, bt, cache_in=c, cache_out=c,
                                      out_dtype=torch.float32)
        outs.append(host(y))
    torch.cuda.synchronize()
    refs, caches = oracle.temporal_conv_stream(chunks, w, b, cache)
    e = max(err(o, r) for o, r in zip(outs, refs))
    report(f"tconv stream {xdt}", y=e)
    assert e <= TOL["f32"], e
    assert np.array_equal(host(c), caches[-1])


@pytest.mark.parametrize("Tf", [1, 3, 7, 20, 40])
def test_tconv_blockcausal(Tf):
    """A 20-frame sequence in chunks of Tf frames, in one call, against the
    oracle's masked whole-sequence sum."""
    B, F, P, C = 2, 20, 9, 32
    x, w, b, cache = workloads.random_tconv(31 + Tf, B, F, P, C)
    y, co = la.temporal_conv_blockcausal(tdev(x, "bf16"), dev(w, "f32"), Tf, dev(b, "f32"),
                                         cache_in=tdev(cache, "bf16"), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.temporal_conv_blockcausal(x, w, b, Tf, cache)
    e = err(host(y), ref)
    report(f"tconv block-causal Tf={Tf}", y=e)
    assert e <= TOL["f32"], e
    assert np.array_equal(host(co), x[:, -1])


def test_tconv_empty_chunk_passes_cache():
    B, P, C = 1, 5, 16
    _, w, _, cache = workloads.random_tconv(41, B, 1, P, C)
    x = torch.empty((B, 0, P, C), dtype=torch.bfloat16, device="cuda")
    ci = tdev(cache, "bf16")
    _, co = la.temporal_conv_chunk(x, dev(w, "f32"), cache_in=ci)
    torch.cuda.synchronize()
    assert torch.equal(co, ci)


def test_tconv_720p_chunk():
    """The 720p latent (21 frames of 45 x 80 positions) at 2048 channels (the
    attention width there, 32 heads x 64), bf16 in and out, with a cache and
    a bias: every element."""
    B, F, P, C = 1, 21, 3600, 2048
    x, w, b, cache = workloads.random_tconv(51, B, F, P, C)
    y, co = la.temporal_conv_chunk(tdev(x, "bf16"), dev(w, "f32"), dev(b, "f32"),
                                   cache_in=tdev(cache, "bf16"))
    torch.cuda.synchronize()
    ref, ref_cache = oracle.temporal_conv_chunk(x, w, b, cache)
    e = err(host(y), ref)
    report("tconv 720p chunk", y=e)
    assert e <= TOL["bf16"], e
    assert np.array_equal(host(co), ref_cache)


def test_tconv_480p_stream_one_call():
    """The 1-minute 480p stream (12 chunks of 21 frames of 30 x 52 positions)
    at 1024 channels (16 heads x 64) in one block-causal call, bf16 in, float32
    out: every element, against the carried-cache stream of the oracle."""
    B, T, P, C, n = 1, 21, 1560, 1024, 12
    _, w, b, cache = workloads.random_tconv(61, B, T, P, C)
    chunks = [workloads.random_tconv(61, B, T, P, C, chunk=k)[0] for k in range(n)]
    x = np.concatenate(chunks, axis=1)
    y, co = la.temporal_conv_blockcausal(tdev(x, "bf16"), dev(w, "f32"), T, dev(b, "f32"),
                                         cache_in=tdev(cache, "bf16"), out_dtype=torch.float32)
    torch.cuda.synchronize()
    yh = host(y)
    del y
    refs, caches = oracle.temporal_conv_stream(chunks, w, b, cache)
    e = max(err(yh[:, k * T:(k + 1) * T], refs[k]) for k in range(n))
    report("tconv 480p stream one call", y=e)
    assert e <= TOL["f32"], e
    assert np.array_equal(host(co), caches[-1])
