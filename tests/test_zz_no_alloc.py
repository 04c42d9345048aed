"""The allocation-free backward entry point, la_blockcausal_backward_noalloc
(through the C ABI): its results against la_blockcausal_backward's (a
caller workspace) on the same inputs, over two calls in a row, the second
with a smaller input than the first (the static scratch keeps the first
call's contents, which the second must not read), plus the oracle's
gradients for each call at the bf16 bound.  Both entry points run the same
kernels with the same plan at these sizes, so the results are bit-identical.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import TOL, dev, host, normwise, report

import block_causal_linear_amd as la

pytestmark = pytest.mark.gpu
EPS = workloads.EPS


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.lib()
    yield
    torch.cuda.synchronize()


def _pack(dS, dz):
    C, B, H, d, _ = dS.shape
    x = np.concatenate([dS.reshape(C, B, H, d * d), dz], axis=-1)
    return np.ascontiguousarray(np.transpose(x, (1, 2, 0, 3)), dtype=np.float32)


def _case(seed, B, H, N, T, d):
    Q, K, V = workloads.random_qkv(seed, B, H, N, d)
    dO = workloads.random_grads(seed + 1, B, H, N, d)
    C = -(-N // T)
    dS, dz = workloads.random_state_grads(seed + 2, B, H, C, d, scale=1e-4)
    S0, z0 = workloads.random_state(seed + 3, B, H, d, tokens=T)
    return Q, K, V, dO, dS, dz, S0, z0


# (B, H, N, T, d): the first call larger than the second; both leave the
# query-gradient split count the same as with a full workspace
CALLS = [(1, 8, 3000, 1000, 64), (2, 2, 777, 200, 128)]


def test_noalloc_matches_workspace_call_twice():
    for n, (B, H, N, T, d) in enumerate(CALLS):
        print(f"[noalloc] call {n}: B={B} H={H} N={N} T={T} d={d}", flush=True)
        ws_need = la.backward_workspace_size(B, H, N, T, d)
        assert ws_need <= la.NOALLOC_SCRATCH_BYTES
        Q, K, V, dO, dS, dz, S0, z0 = _case(900 + 10 * n, B, H, N, T, d)
        q, k, v = dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16")
        si = torch.from_numpy(np.concatenate([S0.reshape(B, H, d * d), z0], -1)).cuda()
        _, states = la.blockcausal_forward(q, k, v, T, state_in=si, eps=EPS)
        do = dev(dO, "f32")
        ds = torch.from_numpy(_pack(dS, dz)).cuda()
        ref = la.blockcausal_backward(q, k, v, states, do, T, dstates=ds, want_dstate_in=True,
                                      eps=EPS)
        # outputs preallocated: the call itself allocates nothing
        outs = [torch.full_like(t, float("nan")) for t in ref]
        got = la.blockcausal_backward_noalloc(q, k, v, states, do, T, dstates=ds, eps=EPS,
                                              dq=outs[0], dk=outs[1], dv=outs[2],
                                              dstate_in=outs[3])
        torch.cuda.synchronize()
        for name, g, r in zip(("dq", "dk", "dv", "dstate_in"), got, ref):
            assert torch.equal(g, r), f"call {n}: {name} differs from the workspace call"
        # and both against the oracle
        bounds = list(range(0, N, T)) + [N]
        oref = oracle.blockcausal_backward(Q, K, V, bounds, dO, EPS, S0=S0, z0=z0, dS=dS, dz=dz)
        errs = {}
        for name, g, r in zip(("dq", "dk", "dv"), got[:3], oref[:3]):
            gn = host(g)
            errs[name] = max(normwise(gn[:, :, a:b], r[:, :, a:b], axes=(2, 3))
                             for a, b in zip(bounds[:-1], bounds[1:]))
        dsi = host(got[3])
        errs["dS_in"] = normwise(dsi[..., : d * d].reshape(B, H, d, d), oref[3], axes=(2, 3))
        errs["dz_in"] = normwise(dsi[..., d * d:], oref[4], axes=(2,))
        report(f"noalloc call {n}", **errs)
        assert max(errs.values()) <= TOL["bf16"], errs


def test_noalloc_rejects_oversize_before_launch():
    # one state slot per head for 2,017 heads at d = 64 is 33.6 MB > 32 MiB
    B, H, N, T, d = 1, 2017, 64, 64, 64
    x = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    st = torch.zeros((B, H, 1, d * d + d), dtype=torch.float32, device="cuda")
    do = torch.zeros((B, H, N, d), dtype=torch.float32, device="cuda")
    with pytest.raises(la.LinAttnError) as e:
        la.blockcausal_backward_noalloc(x, x, x, st, do, T, eps=EPS)
    assert e.value.status == la.LA_E_SCRATCH
