"""Invariants of the launch planners over many shapes (la_plan and
la_backward_plan do no device work, so this runs on the CPU).  Forward:

* the split count is at least 1 and at most the number of KV tiles;
* with more than one split, the partial sums of every split fit in the
  front of `out`, which serves as their scratch:
  splits * (d*d + d) * 4 <= L * d * sizeof(out);
* the readout grid is at least one workgroup and at most one per unit of
  work (the sweep's 4 x 32-token units at d <= 64 with bf16 inputs);
* explicit requests are honoured within those limits.
The backward planner's invariants are stated at its tests below.
"""

import itertools
import os

import pytest
import torch

import block_causal_linear_amd as la

pytestmark = pytest.mark.skipif(not os.path.exists(la.LIB_PATH), reason="liblinattn.so not built")

SHAPES = [(1, 1, 1), (1, 2, 64), (1, 2, 65), (2, 3, 333), (1, 16, 32760), (1, 32, 75600),
          (4, 16, 4096), (1, 1, 1 << 20), (3, 7, 12345), (64, 64, 128), (1, 1, 100_000)]


@pytest.mark.parametrize("B,H,L", SHAPES)
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("in_dt,out_dt", [(torch.bfloat16, torch.float32),
                                          (torch.bfloat16, torch.bfloat16),
                                          (torch.float32, torch.float32)])
def test_plan_invariants(B, H, L, d, in_dt, out_dt):
    tile = 64 if in_dt == torch.bfloat16 else 16
    out_size = 4 if out_dt == torch.float32 else 2
    for req in (0, 1, 3, 16, 1000):
        s, wg = la.plan(B, H, L, d, in_dtype=in_dt, out_dtype=out_dt, kv_splits=req)
        assert 1 <= s <= max(1, -(-L // tile)), (req, s)
        if s > 1:
            assert s * (d * d + d) * 4 <= L * d * out_size, (req, s)
        if req > 0:
            assert s <= req
        assert wg >= 1
        if in_dt == torch.bfloat16 and d < 128:
            units = B * H * -(-L // 128)
            assert wg <= units


def test_plan_requests_honoured_when_they_fit():
    # 720p chunk: 16 splits by default; a request that fits is taken as is
    assert la.plan(1, 32, 75600, 64) == (16, 512)
    for req in (1, 2, 8, 24, 48):
        assert la.plan(1, 32, 75600, 64, kv_splits=req)[0] == req
    for wg in (64, 256, 1000):
        assert la.plan(1, 32, 75600, 64, readout_workgroups=wg)[1] == wg


# ---------------------------------------------------------------------------
# the backward planner (la_backward_plan, no device work)

BWD_SHAPES = [(1, 1, 1, 1), (1, 2, 100, 100), (1, 2, 777, 7), (2, 3, 2085, 500),
              (1, 32, 75600, 75600), (1, 16, 12 * 32760, 32760), (4, 16, 40 * 4096, 4096),
              (1, 1, 1 << 22, 1 << 21), (1, 1, (1 << 22) - 65, 1 << 21), (3, 3, 120000, 9000),
              (64, 64, 128, 128)]
BWD_REQUESTS = [(0, 0), (1, 0), (3, 5), (16, 1000), (10 ** 6, 1)]


@pytest.mark.parametrize("B,H,N,T", BWD_SHAPES)
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("in_dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rope", [False, True])
def test_backward_plan_invariants(B, H, N, T, d, in_dt, rope):
    """Every grid is at least one workgroup and at most one per item or
    sweep unit; split and item counts lie between 1 and the block's tiles;
    a split request is taken up to the tile count; the key-gradient sweep
    serves exactly the bf16 calls at d <= 64 without rotary or a key
    request; the workspace holds the suffix sums plus one partial state per
    query split when there is more than one."""
    bf = in_dt == torch.bfloat16
    tile = 64 if bf else 16
    Tb = min(T, N)
    blocks = -(-N // Tb)
    tiles = -(-Tb // tile)
    pairs = B * H * blocks
    if rope and N >= (1 << 22) - 64:  # beyond the rotary calls' token range
        with pytest.raises(la.LinAttnError):
            la.backward_plan(B, H, N, T, d, in_dt, rope)
        return
    for qreq, kreq in BWD_REQUESTS:
        p = la.backward_plan(B, H, N, T, d, in_dt, rope, qreq, kreq)
        assert p["blocks"] == blocks
        qs = p["query_splits"]
        assert 1 <= qs <= tiles, (qreq, p)
        if qreq > 0:
            assert qs == min(qreq, tiles), (qreq, p)
        if bf:
            assert 1 <= p["query_workgroups"] <= pairs * qs, p
        else:
            assert p["query_workgroups"] == pairs * qs, p
        sweep = bf and d <= 64 and not rope and kreq == 0
        assert (p["key_sweep_units"] > 0) == sweep, (kreq, p)
        if sweep:
            assert p["key_items"] == 0
            assert p["key_sweep_units"] == -(-Tb // 128)
            assert 1 <= p["key_workgroups"] <= min(pairs * p["key_sweep_units"], 512), p
        else:
            ks = p["key_items"]
            assert 1 <= ks <= tiles, (kreq, p)
            if bf:
                assert 1 <= p["key_workgroups"] <= pairs * ks, p
            else:
                assert p["key_workgroups"] == pairs * ks, p
        if (qreq, kreq) == (0, 0):
            need = pairs * (d * d + d) * 4 * (qs + 1 if qs > 1 else 1)
            assert la.backward_workspace_size(B, H, N, T, d, in_dt) == need


def test_backward_plan_bench_shapes():
    # the 720p chunk: 16 query splits on 512 workgroups, the key sweep's 591
    # units of 128 tokens on 512
    assert la.backward_plan(1, 32, 75600, 75600, 64) == dict(
        blocks=1, query_splits=16, query_workgroups=512, key_items=0, key_workgroups=512,
        key_sweep_units=591)
    # config 5 in one call (d = 128): one split and one key item per block, a
    # workgroup per CU
    p = la.backward_plan(4, 16, 40 * 4096, 4096, 128)
    assert (p["blocks"], p["query_splits"], p["key_items"], p["key_sweep_units"]) == (40, 1, 1, 0)
    # a key-workgroup request takes the work items; the rotary calls always do
    assert la.backward_plan(1, 32, 75600, 75600, 64, key_workgroups=1024)["key_sweep_units"] == 0
    assert la.backward_plan(1, 32, 75600, 75600, 64, rope=True)["key_sweep_units"] == 0


def test_backward_plan_fits_the_workspace():
    """A workspace that holds the suffix sums and two partials limits the
    query splits to two; one smaller than the suffix sums is refused, as the
    call itself refuses it; nothing at all for N = 0."""
    B, H, N, T, d = 1, 32, 75600, 75600, 64
    r = B * H * (d * d + d) * 4
    assert la.backward_plan(B, H, N, T, d, workspace_bytes=3 * r)["query_splits"] == 2
    assert la.backward_plan(B, H, N, T, d, workspace_bytes=r)["query_splits"] == 1
    with pytest.raises(la.LinAttnError):
        la.backward_plan(B, H, N, T, d, workspace_bytes=r - 16)
    with pytest.raises(la.LinAttnError):
        la.backward_plan(B, H, N, T, d, query_splits=-1)
    assert la.backward_plan(B, H, 0, 1, d) == dict(
        blocks=0, query_splits=0, query_workgroups=0, key_items=0, key_workgroups=0,
        key_sweep_units=0)
