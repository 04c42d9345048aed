"""GPU parity of the gradients: la_blockcausal_backward, la_chunk_backward
and la_global_backward (through the C ABI) against the fp64 oracle's
``blockcausal_backward`` on the same seeded inputs.

Error: normwise per (b, h, block) slice, max |got - ref| / max |ref|, the
largest over slices.  Bounds as for the forward: 2e-3 for bfloat16 inputs,
1e-5 for float32 inputs (float32 gradients); bfloat16 gradients are also
rounded once on output, so they get 2^-8.  The backward reads the states
the GPU forward wrote, as a training step would.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import (BF16_MISMATCH_MAX, TOL, bf16_rounding, dev, drawn_chunks, host, normwise,
                     report, state_err, state_np)

import block_causal_linear_amd as la

pytestmark = pytest.mark.gpu
EPS = workloads.EPS
BF16_OUT_TOL = 2.0 ** -8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.lib()
    yield
    torch.cuda.synchronize()


def bounds_of(N, T):
    return list(range(0, N, T)) + [N]


def grad_err(got, ref, bounds):
    """Largest normwise error over (b, h, block) slices."""
    return max(normwise(got[:, :, a:b], ref[:, :, a:b], axes=(2, 3))
               for a, b in zip(bounds[:-1], bounds[1:]))


def pack_dstates(dS, dz):
    """[C, B, H, d, d], [C, B, H, d] -> [B, H, C, d*d + d] float32."""
    C, B, H, d, _ = dS.shape
    x = np.concatenate([dS.reshape(C, B, H, d * d), dz], axis=-1)
    return np.ascontiguousarray(np.transpose(x, (1, 2, 0, 3)), dtype=np.float32)


def gpu_backward(Q, K, V, dO, T, dtype, gdt="f32", state_in=None, dstates=None,
                 want_dstate_in=False, eps=EPS, **opts):
    q, k, v = dev(Q, dtype), dev(K, dtype), dev(V, dtype)
    st_in = None if state_in is None else torch.from_numpy(state_in).cuda()
    _, states = la.blockcausal_forward(q, k, v, T, state_in=st_in, eps=eps)
    ds = None if dstates is None else torch.from_numpy(dstates).cuda()
    dq, dk, dv, dsi = la.blockcausal_backward(q, k, v, states, dev(dO, gdt), T, dstates=ds,
                                              want_dstate_in=want_dstate_in, eps=eps, **opts)
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv), None if dsi is None else host(dsi)


def check(name, got, ref, bounds, tol, dsi=None, dsi_ref=None):
    eq, ek, ev = (grad_err(g, r, bounds) for g, r in zip(got, ref))
    vals = dict(dq=eq, dk=ek, dv=ev)
    if dsi is not None:
        es, ez = state_err(dsi, dsi_ref[0], dsi_ref[1])
        vals.update(dS_in=es, dz_in=ez)
    report(name, **vals)
    assert max(vals.values()) <= tol, vals

def check_bf16_grads(name, got, ref, bounds):
    """bfloat16 gradients against the oracle's rounded to bfloat16 (ties to
    even), per (b, h, block) slice: every element within one ulp plus the
    float32 arithmetic error (5e-5 of the slice's largest value), and equal
    to the rounded oracle almost everywhere (the fraction over all blocks)."""
    vals = {}
    for nm, g, r in zip(("dq", "dk", "dv"), got, ref):
        worst, diff = -1e30, 0.0
        for a, b in zip(bounds[:-1], bounds[1:]):
            e, m = bf16_rounding(g[:, :, a:b], r[:, :, a:b], (2, 3), 5e-5)
            worst, diff = max(worst, e), diff + m * (b - a)
        vals[nm + "_ulp_excess"], vals[nm + "_mismatch"] = worst, diff / bounds[-1]
    report(name + " rounding", **vals)
    assert all(v <= 0.0 for k, v in vals.items() if k.endswith("excess")), vals
    assert all(v <= BF16_MISMATCH_MAX for k, v in vals.items() if k.endswith("mismatch")), vals



# ---------------------------------------------------------------------------
# small shapes: several tiles, ragged tails, one-token blocks, a state input
# and gradients on every block's state


SHAPES = [(1000, 64), (2085, 500), (333, 333), (777, 7)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("N,T", SHAPES)
def test_backward_small(dtype, d, N, T):
    B, H = 2, 3
    Q, K, V = workloads.random_qkv(500 + N + d, B, H, N, d, dtype=dtype)
    dO = workloads.random_grads(600 + N + d, B, H, N, d)
    S0, z0 = workloads.random_state(N + T + d, B, H, d)
    bounds = bounds_of(N, T)
    C = len(bounds) - 1
    dS, dz = workloads.random_state_grads(N + 3 * d, B, H, C, d)
    got = gpu_backward(Q, K, V, dO, T, dtype, state_in=state_np(S0, z0),
                       dstates=pack_dstates(dS, dz), want_dstate_in=True)
    ref = oracle.blockcausal_backward(Q, K, V, bounds, dO, EPS, S0.astype(np.float64),
                                      z0.astype(np.float64), dS.astype(np.float64),
                                      dz.astype(np.float64))
    check(f"backward {dtype} d={d} N={N} T={T}", got[:3], ref[:3], bounds, TOL[dtype],
          got[3], ref[3:])


@pytest.mark.parametrize("d", [32, 64, 128])
def test_backward_bf16_gradients(d):
    """bfloat16 dO in, bfloat16 dq/dk/dv out."""
    B, H, N, T = 1, 2, 1300, 300
    Q, K, V = workloads.random_qkv(41 + d, B, H, N, d)
    dO = workloads.random_grads(42 + d, B, H, N, d, dtype="bf16")
    got = gpu_backward(Q, K, V, dO, T, "bf16", gdt="bf16")
    ref = oracle.blockcausal_backward(Q, K, V, bounds_of(N, T), dO, EPS)
    check(f"backward bf16 grads d={d}", got[:3], ref[:3], bounds_of(N, T), BF16_OUT_TOL)
    check_bf16_grads(f"backward bf16 grads d={d}", got[:3], ref[:3], bounds_of(N, T))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chunk_backward(dtype):
    """One chunk against a carried state, with a gradient on state_out."""
    B, H, L, d = 2, 2, 1500, 64
    Q, K, V = workloads.random_qkv(71, B, H, L, d, dtype=dtype)
    dO = workloads.random_grads(72, B, H, L, d)
    S0, z0 = workloads.random_state(73, B, H, d, tokens=5000)
    dS, dz = workloads.random_state_grads(74, B, H, 1, d)
    q, k, v = dev(Q, dtype), dev(K, dtype), dev(V, dtype)
    _, st = la.chunk_forward(q, k, v, torch.from_numpy(state_np(S0, z0)).cuda(), eps=EPS)
    dso = torch.from_numpy(state_np(dS[0], dz[0])).cuda()
    dq, dk, dv, dsi = la.chunk_backward(q, k, v, st, dev(dO, "f32"), dstate_out=dso, eps=EPS)
    torch.cuda.synchronize()
    ref = oracle.blockcausal_backward(Q, K, V, [0, L], dO, EPS, S0.astype(np.float64),
                                      z0.astype(np.float64), dS.astype(np.float64),
                                      dz.astype(np.float64))
    check(f"chunk backward {dtype}", [host(dq), host(dk), host(dv)], ref[:3], [0, L],
          TOL[dtype], host(dsi), ref[3:])


def test_chunk_backward_empty_passes_state_gradient():
    """L = 0: state_out = state_in, so dstate_in = dstate_out exactly."""
    B, H, d = 1, 3, 64
    S0, z0 = workloads.random_state(81, B, H, d)
    st = torch.from_numpy(state_np(S0, z0)).cuda()
    dS, dz = workloads.random_state_grads(82, B, H, 1, d)
    dso = torch.from_numpy(state_np(dS[0], dz[0])).cuda()
    e = torch.empty((B, H, 0, d), dtype=torch.bfloat16, device="cuda")
    _, _, _, dsi = la.chunk_backward(e, e, e, st, e.float(), dstate_out=dso, eps=EPS)
    torch.cuda.synchronize()
    assert torch.equal(dsi, dso)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_global_backward(dtype):
    B, H, N, d = 1, 4, 3000, 64
    Q, K, V = workloads.random_qkv(91, B, H, N, d, dtype=dtype)
    dO = workloads.random_grads(92, B, H, N, d)
    q, k, v = dev(Q, dtype), dev(K, dtype), dev(V, dtype)
    _, st = la.global_forward(q, k, v, eps=EPS)
    dq, dk, dv = la.global_backward(q, k, v, st, dev(dO, "f32"), eps=EPS)
    torch.cuda.synchronize()
    ref = oracle.blockcausal_backward(Q, K, V, [0, N], dO, EPS)
    check(f"global backward {dtype}", [host(dq), host(dk), host(dv)], ref[:3], [0, N],
          TOL[dtype])


# ---------------------------------------------------------------------------
# full sizes


def test_backward_720p_chunk():
    """The 720p chunk (B=1, H=32, d=64, 75,600 tokens) against the state
    after chunk 0, with a gradient on state_out: every element."""
    w = workloads.CHUNK_720P
    Q0, K0, V0 = workloads.chunk_qkv(w, 0)
    _, S0, z0 = oracle.global_forward(Q0, K0, V0, EPS)
    Q, K, V = workloads.chunk_qkv(w, 1)
    dO = workloads.random_grads(3, w.B, w.H, w.L, w.d, chunk=1)
    dS, dz = workloads.random_state_grads(3, w.B, w.H, 1, w.d, scale=1e-5)
    got = gpu_backward(Q, K, V, dO, w.L, "bf16", state_in=state_np(S0, z0),
                       dstates=pack_dstates(dS, dz), want_dstate_in=True)
    ref = oracle.blockcausal_backward(Q, K, V, [0, w.L], dO, EPS, S0, z0, dS.astype(np.float64),
                                      dz.astype(np.float64))
    check("720p chunk backward", got[:3], ref[:3], [0, w.L], TOL["bf16"], got[3], ref[3:])


def test_backward_480p_one_call():
    """The 1-minute 480p stream (12 blocks of 32,760 tokens, 16 heads) as one
    block-causal sequence: every element, per block."""
    w = workloads.WORKLOADS[4]
    N, T = w.L * w.chunks, w.L
    parts = [workloads.chunk_qkv(w, n) for n in range(w.chunks)]
    Q, K, V = (np.concatenate([p[i] for p in parts], axis=2) for i in range(3))
    del parts
    dO = workloads.random_grads(4, w.B, w.H, N, w.d)
    got = gpu_backward(Q, K, V, dO, T, "bf16")
    bounds = bounds_of(N, T)
    ref = oracle.blockcausal_backward(Q, K, V, bounds, dO, EPS)
    check("480p one-call backward", got[:3], ref[:3], bounds, TOL["bf16"])


def test_backward_long_horizon_d128_one_call():
    """The long-horizon stream (B=4, H=16, d=128, 40 blocks of 4,096 tokens, 1% outlier
    rows) in one call.  The oracle is composed block by block from its own
    steps (readout_backward per block, suffix sums, kv_backward) on eight
    sampled (b, h) pairs, four from each half of the pairs (a call of this
    size runs its halves on two streams), among them the first and last pair
    of each half; dQ, dK and dV of every block are compared there.  Each
    block is drawn once, as it is uploaded."""
    w = workloads.WORKLOADS[5]
    N, T, C = w.L * w.chunks, w.L, w.chunks
    assert la.backward_stream_count(w.B, w.H, N, T, w.d) == 2
    heads = [(0, 0), (0, 13), (1, 6), (1, 15), (2, 0), (2, 9), (3, 2), (3, 15)]
    bi = [b for b, _ in heads]
    hi = [h for _, h in heads]
    q = torch.empty((w.B, w.H, N, w.d), dtype=torch.bfloat16, device="cuda")
    k, v = torch.empty_like(q), torch.empty_like(q)
    do = torch.empty((w.B, w.H, N, w.d), dtype=torch.float32, device="cuda")

    def draw(n):
        return workloads.chunk_qkv(w, n) + (workloads.random_grads(5, w.B, w.H, T, w.d, chunk=n),)

    kept = []  # the sampled pairs' Q, K, V, dO per block, as [1, 8, T, d]
    for n, (Qn, Kn, Vn, dOn) in drawn_chunks(draw, range(C)):
        sl = slice(n * T, (n + 1) * T)
        q[:, :, sl], k[:, :, sl], v[:, :, sl] = dev(Qn, "bf16"), dev(Kn, "bf16"), dev(Vn, "bf16")
        do[:, :, sl] = dev(dOn, "f32")
        kept.append(tuple(x[bi, hi][None] for x in (Qn, Kn, Vn, dOn)))
    _, states = la.blockcausal_forward(q, k, v, T, eps=EPS)
    dq, dk, dv, _ = la.blockcausal_backward(q, k, v, states, do, T, eps=EPS)
    torch.cuda.synchronize()
    del states, q, k, v, do
    bt = torch.tensor(bi, device="cuda")
    ht = torch.tensor(hi, device="cuda")

    def sampled(t, n):
        return host(t[bt, ht, n * T:(n + 1) * T])[None]

    S = np.zeros((1, len(heads), w.d, w.d))
    z = np.zeros((1, len(heads), w.d))
    GS, Gz, worst = [], [], 0.0
    for n, (Qn, Kn, Vn, dOn) in enumerate(kept):
        KV, kk = oracle.kv_of_block(Kn, Vn)
        S, z = S + KV, z + kk
        dQn, dSn, dzn = oracle.readout_backward(Qn, S, z, dOn, EPS)
        GS.append(dSn)
        Gz.append(dzn)
        e = normwise(sampled(dq, n), dQn, axes=(2, 3))
        worst = max(worst, e)
        report(f"long-horizon backward block {n}", dq=e)
    RS, Rz = GS[:], Gz[:]
    for n in range(C - 2, -1, -1):
        RS[n] = RS[n] + RS[n + 1]
        Rz[n] = Rz[n] + Rz[n + 1]
    for n, (_, Kn, Vn, _) in enumerate(kept):
        dKn, dVn = oracle.kv_backward(Kn, Vn, RS[n], Rz[n])
        ek = normwise(sampled(dk, n), dKn, axes=(2, 3))
        ev = normwise(sampled(dv, n), dVn, axes=(2, 3))
        report(f"long-horizon backward block {n}", dk=ek, dv=ev)
        worst = max(worst, ek, ev)
    assert worst <= TOL["bf16"], worst


# ---------------------------------------------------------------------------
# launch shapes, reproducibility, degenerate rows


def test_backward_splits_and_reproducibility():
    """Different workgroup counts change results only by float32 summation
    order; the same launch twice gives identical bits."""
    B, H, N, T, d = 1, 2, 20000, 20000, 64
    Q, K, V = workloads.random_qkv(111, B, H, N, d)
    dO = workloads.random_grads(112, B, H, N, d)
    a = gpu_backward(Q, K, V, dO, T, "bf16", want_dstate_in=True)
    b = gpu_backward(Q, K, V, dO, T, "bf16", want_dstate_in=True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    for ks, kw in ((1, 1), (5, 3), (40, 300)):
        c = gpu_backward(Q, K, V, dO, T, "bf16", want_dstate_in=True, kv_splits=ks,
                         readout_workgroups=kw)
        errs = [normwise(x, y, axes=(2, 3) if x.ndim == 4 else (2,)) for x, y in zip(a, c)]
        report(f"backward splits={ks} key workgroups={kw}", max_rel_diff=max(errs))
        assert max(errs) <= 1e-5, errs


@pytest.mark.parametrize("B,H,N,T,d,gdt", [
    (1, 4, 3000, 3000, 64, torch.float32),     # one block, ragged last unit
    (2, 3, 2085, 500, 64, torch.float32),      # several blocks, short last block, B > 1
    (1, 2, 777, 7, 64, torch.float32),         # 7-token blocks: most wave tiles store nothing
    (1, 2, 100, 100, 64, torch.float32),       # less than one unit: a one-workgroup grid
    (1, 3, 5000, 1200, 32, torch.bfloat16),    # d = 32, bfloat16 gradients
    (1, 32, 40000, 40000, 64, torch.float32),  # 10,016 units over the 512-workgroup grid
    (1, 8, 75600, 75600, 64, torch.float32),   # a block longer than the grid's 512 units
])
def test_backward_key_sweep_matches_items(B, H, N, T, d, gdt):
    """bf16 inputs at d <= 64 take the key-gradient sweep; a key-workgroup
    request takes the work-item kernel.  Both compute every token's dk and dv
    with the same operands and the same MFMA order: bit for bit equal (and
    dq, dstate_in untouched by the choice).  Both run on one stream."""
    print(f"[key sweep] B={B} H={H} N={N} T={T} d={d} grads={gdt}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(B * 100 + H * 10 + d + N)
    q, k, v = (torch.randn((B, H, N, d), generator=g, device="cuda").to(torch.bfloat16)
               for _ in range(3))
    do = torch.randn((B, H, N, d), generator=g, device="cuda").to(gdt)
    st_in = torch.rand((B, H, d * d + d), generator=g, device="cuda") * 10
    _, states = la.blockcausal_forward(q, k, v, T, state_in=st_in, eps=EPS)
    ds = torch.randn(states.shape, generator=g, device="cuda") * 1e-4
    kw = dict(dstates=ds, want_dstate_in=True, eps=EPS)
    sweep = [t.clone() for t in la.blockcausal_backward(q, k, v, states, do, T, **kw)]
    items = [t.clone() for t in la.blockcausal_backward(q, k, v, states, do, T,
                                                       readout_workgroups=1024, **kw)]
    again = [t.clone() for t in la.blockcausal_backward(q, k, v, states, do, T, **kw)]
    torch.cuda.synchronize()
    for name, a, b, c in zip(("dq", "dk", "dv", "dstate_in"), sweep, items, again):
        assert torch.isfinite(a).all(), name
        assert torch.equal(a, b), name
        assert torch.equal(a, c), name
    report(f"key sweep against work items B={B} H={H} N={N} T={T} d={d}", bitwise=1.0)


def test_backward_zero_eps_ragged():
    """eps = 0 (every denominator kept > 0 by one positive feature per row):
    the rows past the end of a ragged last tile and block stay out of every
    sum, so nothing turns into NaN, and the result matches the oracle."""
    B, H, N, T, d = 1, 2, 1000, 300, 64
    Q, K, V = workloads.random_qkv(121, B, H, N, d)
    Q[..., 0] = np.abs(Q[..., 0]) + 0.25
    K[..., 0] = np.abs(K[..., 0]) + 0.25
    # both sides must see the same (bfloat16) values
    Q, K = workloads.bf16_round(Q), workloads.bf16_round(K)
    dO = workloads.random_grads(122, B, H, N, d)
    got = gpu_backward(Q, K, V, dO, T, "bf16", eps=0.0)
    assert all(np.all(np.isfinite(x)) for x in got[:3])
    ref = oracle.blockcausal_backward(Q, K, V, bounds_of(N, T), dO, 0.0)
    check("backward eps=0", got[:3], ref[:3], bounds_of(N, T), TOL["bf16"])


def test_backward_degenerate_rows():
    """A query row with no positive entry gets dq = 0 exactly; a key row with
    no positive entry gets dk = 0 and dv = 0 exactly."""
    B, H, N, T, d = 1, 2, 1000, 300, 64
    Q, K, V = workloads.random_qkv(123, B, H, N, d)
    Q[:, :, 17] = -np.abs(Q[:, :, 17])
    K[:, :, 450] = -np.abs(K[:, :, 450])
    dO = workloads.random_grads(124, B, H, N, d)
    dq, dk, dv, _ = gpu_backward(Q, K, V, dO, T, "bf16")
    assert np.all(dq[:, :, 17] == 0.0)
    assert np.all(dk[:, :, 450] == 0.0) and np.all(dv[:, :, 450] == 0.0)
    ref = oracle.blockcausal_backward(Q, K, V, bounds_of(N, T), dO, EPS)
    check("backward degenerate rows", [dq, dk, dv], ref[:3], bounds_of(N, T), TOL["bf16"])


# ---------------------------------------------------------------------------
# two streams: a bfloat16 call of at least 2^20 token-heads runs its two halves
# of (b, h) pairs on the caller's stream and the library's second stream


@pytest.mark.parametrize("B,H,N,T,d,rope,gdt", [
    (1, 16, 70000, 70000, 128, False, torch.float32),  # one block, even pair count
    (1, 5, 300000, 300000, 64, True, torch.float32),   # odd: halves of 2 and 3 pairs
    (3, 3, 120000, 9000, 128, False, torch.float32),   # several blocks, B > 1, ragged last block
    (2, 4, 140000, 140000, 32, True, torch.float32),   # rotary at d = 32
    (1, 8, 140000, 70000, 64, True, torch.bfloat16),   # bfloat16 gradients
])
def test_backward_two_streams_bitwise(B, H, N, T, d, rope, gdt):
    """Against the same call on one stream (stage events keep a call on the
    caller's stream), bit for bit: each half keeps the whole call's query
    splits, so nothing differs but the stream.  With a state input and state
    gradients, and the caller's stream a side stream."""
    assert B * H * N >= 1 << 20 and la.backward_stream_count(B, H, N, T, d, rope=rope) == 2
    print(f"[two streams] B={B} H={H} N={N} T={T} d={d} rope={rope} grads={gdt}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(B * 1000 + H * 10 + d)
    q, k, v = (torch.randn((B, H, N, d), generator=g, device="cuda").to(torch.bfloat16)
               for _ in range(3))
    do = torch.randn((B, H, N, d), generator=g, device="cuda").to(gdt)
    st_in = torch.rand((B, H, d * d + d), generator=g, device="cuda") * 10
    grid = (7, 40, 60)
    if rope:
        _, states = la.blockcausal_forward_rope(q, k, v, T, *grid, state_in=st_in, eps=EPS)
    else:
        _, states = la.blockcausal_forward(q, k, v, T, state_in=st_in, eps=EPS)
    ds = torch.randn(states.shape, generator=g, device="cuda") * 1e-4

    def run(events):
        kw = dict(dstates=ds, want_dstate_in=True, eps=EPS, stage_events=events)
        if rope:
            return la.blockcausal_backward_rope(q, k, v, states, do, T, *grid, **kw)
        return la.blockcausal_backward(q, k, v, states, do, T, **kw)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one = [t.clone() for t in run(la.StageEvents())]   # one stream
        two = [t.clone() for t in run(None)]               # two halves on two streams
        again = [t.clone() for t in run(None)]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for name, a, b, c in zip(("dq", "dk", "dv", "dstate_in"), one, two, again):
        assert torch.equal(a, b), name
        assert torch.equal(b, c), name
        assert torch.isfinite(b).all(), name
    report(f"two-stream backward B={B} H={H} N={N} d={d} rope={rope} grads={gdt}", bitwise=1.0)


def test_backward_two_streams_from_two_threads():
    """Two host threads, each with its own stream, issue large backward calls
    at once (both fork onto the device's one second stream): every result
    equals the same call issued alone, bit for bit."""
    import threading

    B, H, N, T, d = 1, 16, 70000, 70000, 128
    assert la.backward_stream_count(B, H, N, T, d) == 2
    g = torch.Generator(device="cuda").manual_seed(77)
    cases = []
    for _ in range(2):
        q, k, v = (torch.randn((B, H, N, d), generator=g, device="cuda").to(torch.bfloat16)
                   for _ in range(3))
        do = torch.randn((B, H, N, d), generator=g, device="cuda")
        _, states = la.blockcausal_forward(q, k, v, T, eps=EPS)
        cases.append((q, k, v, states, do))
    torch.cuda.synchronize()
    alone = []
    for q, k, v, states, do in cases:
        grads = la.blockcausal_backward(q, k, v, states, do, T, eps=EPS)[:3]
        alone.append([t.clone() for t in grads])
    torch.cuda.synchronize()

    results = [None, None]
    errors = []

    def work(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = []
                for _ in range(3):
                    q, k, v, states, do = cases[i]
                    outs = la.blockcausal_backward(q, k, v, states, do, T, eps=EPS)[:3]
                s.synchronize()
                results[i] = [t.clone() for t in outs]
        except Exception as e:  # surfaced below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        for a, b in zip(alone[i], results[i]):
            assert torch.equal(a, b)
    report("two-stream backward from two host threads", bitwise=1.0)
