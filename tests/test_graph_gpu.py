"""HIP graph capture of the library's calls (they launch kernels and nothing
else: no allocation, no memset, no synchronisation), replayed several
times with eager work and synchronisations in between; every replay must
match the eager results bit for bit.  The expected values are the eager
calls' own results: this checks capture and replay, not numerics (the
parity tests do that against the oracle)."""

import pytest
import torch

import workloads
from helpers import dev

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


def test_graph_replays_match_eager():
    B, H, L, d = 1, 4, 3000, 64
    Q, K, V = workloads.random_qkv(301, B, H, L, d)
    q, k, v = dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16")
    do = dev(workloads.random_grads(302, B, H, L, d), "f32")
    x, w, b, cache = workloads.random_tconv(303, 1, 5, 40, 64)
    xt, wt, bt, ct = dev(x, "bf16"), dev(w, "f32"), dev(b, "f32"), dev(cache, "bf16")

    state_in = la.new_state(B, H, d)
    la.global_forward(q, k, v, state_out=state_in, eps=EPS)
    out = torch.empty((B, H, L, d), device="cuda")
    st = torch.empty((B, H, d * d + d), device="cuda")
    dq, dk, dv = (torch.empty((B, H, L, d), device="cuda") for _ in range(3))
    dsi = torch.empty_like(st)
    ws = torch.empty(la.backward_workspace_size(B, H, L, L, d), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(xt)
    co = torch.empty_like(ct)
    fresh = torch.empty_like(st)

    out_r = torch.empty_like(out)
    st_r = torch.empty_like(st)
    dq_r, dk_r, dv_r = (torch.empty_like(dq) for _ in range(3))

    def calls():
        la.state_reset(fresh)
        la.chunk_forward(q, k, v, state_in, out=out, state_out=st, eps=EPS)
        la.chunk_forward_rope(q, k, v, state_in, 3, 20, 25, out=out_r, state_out=st_r, eps=EPS)
        la.chunk_backward(q, k, v, st, do, eps=EPS, dq=dq, dk=dk, dv=dv, dstate_in=dsi,
                          workspace=ws)
        la.temporal_conv_chunk(xt, wt, bt, cache_in=ct, y=y, cache_out=co)
        la.blockcausal_backward_rope(q, k, v, st_r.view(B, H, 1, d * d + d), do, L, 3, 20, 25,
                                     eps=EPS, dq=dq_r, dk=dk_r, dv=dv_r, workspace=ws)

    results = [out, st, dq, dk, dv, dsi, y, co, fresh, out_r, st_r, dq_r, dk_r, dv_r]
    calls()
    torch.cuda.synchronize()
    eager = [r.clone() for r in results]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(4):
        for r in results:
            r.fill_(float("nan")) if r.dtype.is_floating_point else r.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        names = "out st dq dk dv dsi y co fresh out_r st_r dq_r dk_r dv_r".split()
        for name, r, e in zip(names, results, eager):
            assert torch.equal(r, e), (rep, name)
        # eager work between replays
        la.chunk_forward(q, k, v, state_in, eps=EPS)
        torch.cuda.synchronize()


def test_concurrent_streams_match_sequential():
    """Calls on two streams with disjoint buffers may overlap on the GPU; each
    result equals the same call run alone (bit for bit)."""
    B, H, L, d = 1, 8, 20000, 64
    sets = []
    for seed in (311, 312):
        Q, K, V = workloads.random_qkv(seed, B, H, L, d)
        q, k, v = dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16")
        st_in = la.new_state(B, H, d)
        la.global_forward(q, k, v, state_out=st_in, eps=EPS)
        sets.append((q, k, v, st_in))
    torch.cuda.synchronize()

    def run(i, rope):
        q, k, v, st_in = sets[i]
        if rope:
            return la.chunk_forward_rope(q, k, v, st_in, 0, 50, 40, eps=EPS)
        return la.chunk_forward(q, k, v, st_in, eps=EPS)

    alone = []
    for i, rope in ((0, False), (1, True)):
        o, st = run(i, rope)
        torch.cuda.synchronize()
        alone.append((o.clone(), st.clone()))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        res = [None, None]
        for i, rope in ((0, False), (1, True)):
            with torch.cuda.stream(streams[i]):
                res[i] = run(i, rope)
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(res[i][0], alone[i][0]) and torch.equal(res[i][1], alone[i][1]), \
                (rep, i)
