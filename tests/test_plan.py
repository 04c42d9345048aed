"""Invariants of the forward launch planner over many shapes (la_plan does
no device work, so this runs on the CPU):

* the split count is at least 1 and at most the number of KV tiles;
* with more than one split, the partial sums of every split fit in the
  front of `out`, which serves as their scratch:
  splits * (d*d + d) * 4 <= L * d * sizeof(out);
* the readout grid is at least one workgroup and at most one per unit of
  work (the sweep's 4 x 32-token units at d <= 64 with bf16 inputs);
* explicit requests are honoured within those limits.
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
