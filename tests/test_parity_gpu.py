"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on
the same seeded inputs.

Bounds (normwise per (b, h, block) slice, max |got - ref| / max |ref|):
1e-5 for float32 inputs, 2e-3 for bfloat16 inputs with float32 output.
The state (S, z) is compared the same way.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import (BF16_MISMATCH_MAX, TOL, bf16_rounding, dev, drawn_chunks, host, out_err,
                     report, state_err, state_np)

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


def run_chunk(Q, K, V, S_in_np, dtype, kv_splits=0, out_dtype=torch.float32):
    st_in = torch.from_numpy(S_in_np).cuda()
    out, st = la.chunk_forward(dev(Q, dtype), dev(K, dtype), dev(V, dtype), st_in,
                               eps=EPS, kv_splits=kv_splits, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return host(out), host(st)


def check_chunk(name, Q, K, V, S_in, z_in, dtype, kv_splits=0):
    O_ref, S_ref, z_ref = oracle.chunk_forward(Q, K, V, S_in, z_in, EPS)
    O, st = run_chunk(Q, K, V, state_np(S_in, z_in), dtype, kv_splits)
    eo = out_err(O, O_ref)
    es, ez = state_err(st, S_ref, z_ref)
    report(name, out=eo, S=es, z=ez)
    assert eo <= TOL[dtype], eo
    assert es <= TOL[dtype] and ez <= TOL[dtype], (es, ez)
    return O, st


# ---------------------------------------------------------------------------
# small shapes spanning several tiles and a ragged tail


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("L", [1, 15, 64, 333, 2085])
def test_chunk_small(dtype, d, L):
    B, H = 2, 3
    Q, K, V = workloads.random_qkv(1000 + L, B, H, L, d, dtype=dtype)
    S_in, z_in = workloads.random_state(L + d, B, H, d)
    S_in, z_in = S_in.astype(np.float64), z_in.astype(np.float64)
    check_chunk(f"chunk {dtype} d={d} L={L}", Q, K, V, S_in, z_in, dtype)


# One block at d = 128 over 64 or more (b, h) pairs takes the quadrant KV
# kernel (no token split, the state written directly); head counts that are
# not a multiple of 8 leave idle workgroups in its grid.
@pytest.mark.parametrize("B,H,L", [(1, 64, 300), (2, 33, 130), (1, 65, 1), (4, 16, 4096)])
def test_chunk_d128_quadrants(B, H, L):
    d = 128
    assert la.plan(B, H, L, d)[0] == 1  # the quadrant path
    Q, K, V = workloads.random_qkv(3100 + H, B, H, L, d)
    S_in, z_in = workloads.random_state(3200 + H, B, H, d)
    S_in, z_in = S_in.astype(np.float64), z_in.astype(np.float64)
    O, st = check_chunk(f"chunk quadrants B={B} H={H} L={L}", Q, K, V, S_in, z_in, "bf16")
    # in place (state_out = state_in) gives the same bits
    st_io = torch.from_numpy(state_np(S_in, z_in)).cuda()
    out, st2 = la.chunk_forward(dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), st_io,
                                state_out=st_io, eps=EPS)
    torch.cuda.synchronize()
    assert st2.data_ptr() == st_io.data_ptr()
    assert np.array_equal(host(st2), st) and np.array_equal(host(out), O)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_global_small(dtype, d):
    B, H, N = 1, 2, 1500
    Q, K, V = workloads.random_qkv(77, B, H, N, d, dtype=dtype)
    O_ref, S_ref, z_ref = oracle.global_forward(Q, K, V, EPS)
    out, st = la.global_forward(dev(Q, dtype), dev(K, dtype), dev(V, dtype), eps=EPS)
    torch.cuda.synchronize()
    eo = out_err(host(out), O_ref)
    es, ez = state_err(host(st), S_ref, z_ref)
    report(f"global {dtype} d={d}", out=eo, S=es, z=ez)
    assert eo <= TOL[dtype] and es <= TOL[dtype] and ez <= TOL[dtype]


# ---------------------------------------------------------------------------
# the five workloads at full size


def test_tiny_f32_stream_4x64():
    w = workloads.WORKLOADS[1]
    state = la.new_state(w.B, w.H, w.d)
    blocks = [workloads.chunk_qkv(w, n) for n in range(w.chunks)]
    outs, states = oracle.stream_forward(blocks, EPS)
    for n, (Q, K, V) in enumerate(blocks):
        out, state = la.chunk_forward(dev(Q, "f32"), dev(K, "f32"), dev(V, "f32"), state,
                                      state_out=state, eps=EPS)
        torch.cuda.synchronize()
        eo = out_err(host(out), outs[n])
        es, ez = state_err(host(state), *states[n])
        report(f"tiny f32 stream chunk {n}", out=eo, S=es, z=ez)
        assert eo <= TOL["f32"] and es <= TOL["f32"] and ez <= TOL["f32"]


@pytest.mark.parametrize("cid", [2, 3])
def test_global_video_latent(cid):
    w = workloads.WORKLOADS[cid]
    Q, K, V = workloads.chunk_qkv(w, 0)
    out, st = la.global_forward(dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), eps=EPS)
    torch.cuda.synchronize()
    O_ref, S_ref, z_ref = oracle.global_forward(Q, K, V, EPS)
    eo = out_err(host(out), O_ref)
    es, ez = state_err(host(st), S_ref, z_ref)
    report(w.name, out=eo, S=es, z=ez)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"] and ez <= TOL["bf16"]


def test_chunk_720p():
    """The timed workload: chunk 1 of a 720p latent against chunk 0's state,
    in the launch configuration the benchmark uses."""
    w = workloads.CHUNK_720P
    Q0, K0, V0 = workloads.chunk_qkv(w, 0)
    Q1, K1, V1 = workloads.chunk_qkv(w, 1)
    del Q0
    KV0, k0 = oracle.kv_of_block(K0, V0)
    del K0, V0
    st0_np = state_np(KV0, k0)          # the float32 state the GPU receives
    d = w.d
    S0 = st0_np[..., : d * d].reshape(KV0.shape).astype(np.float64)
    z0 = st0_np[..., d * d:].astype(np.float64)
    st0 = torch.from_numpy(st0_np).cuda()
    out, st1 = la.chunk_forward(dev(Q1, "bf16"), dev(K1, "bf16"), dev(V1, "bf16"), st0, eps=EPS)
    torch.cuda.synchronize()
    O_ref, S_ref, z_ref = oracle.chunk_forward(Q1, K1, V1, S0, z0, EPS)
    eo = out_err(host(out), O_ref)
    es, ez = state_err(host(st1), S_ref, z_ref)
    report("720p chunk", out=eo, S=es, z=ez)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"] and ez <= TOL["bf16"]


def test_stream_480p_1min():
    """12 chunks with the state resident on the GPU (in place); every chunk's
    output and state checked against a full-sequence recomputation that
    takes all block KVs first and prefix-sums them."""
    w = workloads.WORKLOADS[4]
    state = la.new_state(w.B, w.H, w.d)
    KVs, ks = [], []
    worst = [0.0, 0.0, 0.0]
    for n, (Q, K, V) in drawn_chunks(lambda c: workloads.chunk_qkv(w, c), range(w.chunks)):
        out, state = la.chunk_forward(dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), state,
                                      state_out=state, eps=EPS)
        KV, k = oracle.kv_of_block(K, V)
        KVs.append(KV)
        ks.append(k)
        S_pre = np.sum(np.stack(KVs), axis=0)
        z_pre = np.sum(np.stack(ks), axis=0)
        O_ref = oracle.readout(Q, S_pre, z_pre, EPS)
        torch.cuda.synchronize()
        eo = out_err(host(out), O_ref)
        es, ez = state_err(host(state), S_pre, z_pre)
        report(f"480p stream chunk {n}", out=eo, S=es, z=ez)
        worst = [max(a, b) for a, b in zip(worst, (eo, es, ez))]
    assert max(worst) <= TOL["bf16"], worst


def test_long_horizon_d128():
    """40 chunks, B=4, H=16, d=128, 1% outlier rows x8; per-chunk drift of
    S and z (every head) and O against the fp64 carried state.  O is
    compared on every head at the first and last chunk and on eight sampled
    (b, h) pairs at the others (the oracle's chunk step, composed of its KV
    and readout steps, with the readout on those pairs)."""
    w = workloads.WORKLOADS[5]
    heads = [(0, 0), (0, 13), (1, 6), (1, 15), (2, 0), (2, 9), (3, 2), (3, 15)]
    bi = [b for b, _ in heads]
    hi = [h for _, h in heads]
    bt = torch.tensor(bi, device="cuda")
    ht = torch.tensor(hi, device="cuda")
    state = la.new_state(w.B, w.H, w.d)
    S = np.zeros((w.B, w.H, w.d, w.d))
    z = np.zeros((w.B, w.H, w.d))
    worst = 0.0
    for n, (Q, K, V) in drawn_chunks(lambda c: workloads.chunk_qkv(w, c), range(w.chunks)):
        out, state = la.chunk_forward(dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), state,
                                      state_out=state, eps=EPS)
        KV, kk = oracle.kv_of_block(K, V)
        S, z = S + KV, z + kk
        if n in (0, w.chunks - 1):
            O_ref = oracle.readout(Q, S, z, EPS)
            got = out
        else:
            O_ref = oracle.readout(Q[bi, hi][None], S[bi, hi][None], z[bi, hi][None], EPS)
            got = out[bt, ht][None]
        torch.cuda.synchronize()
        eo = out_err(host(got), O_ref)
        es, ez = state_err(host(state), S, z)
        report(f"long-horizon chunk {n}", out=eo, S=es, z=ez)
        worst = max(worst, eo, es, ez)
    assert worst <= TOL["bf16"], worst


# ---------------------------------------------------------------------------
# invariances, reproducibility, state handling, edge cases


def test_split_invariance_and_reproducibility():
    B, H, L, d = 1, 4, 9000, 64
    Q, K, V = workloads.random_qkv(5, B, H, L, d)
    S_in, z_in = workloads.random_state(6, B, H, d)
    O_ref, S_ref, z_ref = oracle.chunk_forward(Q, K, V, S_in, z_in, 1e-6)
    base = None
    for splits in (0, 1, 2, 5, 17, 100):
        O, st = run_chunk(Q, K, V, state_np(S_in, z_in), "bf16", kv_splits=splits)
        eo = out_err(O, O_ref)
        es, _ = state_err(st, S_ref, z_ref)
        report(f"splits={splits}", out=eo, S=es)
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]
        if base is None:
            base = (O, st)
        else:
            # only float32 summation order differs between split counts
            assert out_err(O, base[0]) < 1e-5
    O2, st2 = run_chunk(Q, K, V, state_np(S_in, z_in), "bf16", kv_splits=0)
    assert np.array_equal(O2, base[0]) and np.array_equal(st2, base[1])


def test_in_place_state_matches_out_of_place():
    B, H, L, d = 2, 2, 700, 64
    Q, K, V = workloads.random_qkv(8, B, H, L, d)
    S_in, z_in = workloads.random_state(9, B, H, d)
    st_np = state_np(S_in, z_in)
    q, k, v = dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16")
    a_in = torch.from_numpy(st_np).cuda()
    out_a, st_a = la.chunk_forward(q, k, v, a_in, eps=EPS)
    b_state = torch.from_numpy(st_np).cuda()
    out_b, st_b = la.chunk_forward(q, k, v, b_state, state_out=b_state, eps=EPS)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b) and torch.equal(st_a, st_b)
    assert torch.equal(a_in.cpu(), torch.from_numpy(st_np))  # state_in untouched


def test_state_checkpoint_roundtrip_is_bitwise():
    B, H, L, d = 1, 2, 500, 64
    chunks = [workloads.random_qkv(30 + n, B, H, L, d) for n in range(4)]
    dv = [tuple(dev(x, "bf16") for x in c) for c in chunks]
    st = la.new_state(B, H, d)
    outs = []
    for q, k, v in dv:
        o, st = la.chunk_forward(q, k, v, st, state_out=st, eps=EPS)
        outs.append(o.clone())
    st2 = la.new_state(B, H, d)
    for q, k, v in dv[:2]:
        _, st2 = la.chunk_forward(q, k, v, st2, state_out=st2, eps=EPS)
    saved = st2.cpu()
    st3 = saved.cuda()
    for i, (q, k, v) in enumerate(dv[2:]):
        o, st3 = la.chunk_forward(q, k, v, st3, state_out=st3, eps=EPS)
        assert torch.equal(o, outs[2 + i])
    torch.cuda.synchronize()
    assert torch.equal(st3, st)


def test_empty_chunk_and_sequence():
    B, H, d = 1, 3, 64
    S_in, z_in = workloads.random_state(11, B, H, d)
    st_in = torch.from_numpy(state_np(S_in, z_in)).cuda()
    e = torch.empty((B, H, 0, d), dtype=torch.bfloat16, device="cuda")
    out, st = la.chunk_forward(e, e, e, st_in, eps=EPS)
    torch.cuda.synchronize()
    assert out.shape == (B, H, 0, d) and torch.equal(st, st_in)
    out, st = la.global_forward(e, e, e, eps=EPS)
    torch.cuda.synchronize()
    assert torch.count_nonzero(st) == 0


def test_degenerate_rows():
    """All-non-positive query rows give exactly 0; all-non-positive key rows
    contribute nothing (their values can be anything: the result is bitwise
    unchanged, and equals the oracle with those tokens removed)."""
    B, H, L, d = 1, 2, 300, 64
    Q, K, V = workloads.random_qkv(12, B, H, L, d)
    Q[:, :, 7] = -np.abs(Q[:, :, 7])
    K[:, :, 100:150] = -np.abs(K[:, :, 100:150])
    V2 = V.copy()
    V2[:, :, 100:150] = workloads.random_qkv(99, B, H, 50, d)[2]
    out, st = la.global_forward(dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), eps=EPS)
    out2, st2 = la.global_forward(dev(Q, "bf16"), dev(K, "bf16"), dev(V2, "bf16"), eps=EPS)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[:, :, 7]) == 0
    assert torch.equal(out, out2) and torch.equal(st, st2)
    Kd = np.delete(K, np.s_[100:150], axis=2)
    Vd = np.delete(V, np.s_[100:150], axis=2)
    O_ref, _, _ = oracle.global_forward(Q, Kd, Vd, EPS)
    assert out_err(host(out), O_ref) <= TOL["bf16"]


# every readout that writes bfloat16 rows: the sweep (d = 32, 64), the item
# readout (d = 128, after the split KV reduction or, over 64 heads, the
# quadrant one) and the float32-input readout
@pytest.mark.parametrize("B,H,L,d,dtype", [(1, 4, 3000, 64, "bf16"), (1, 4, 3000, 32, "bf16"),
                                           (1, 4, 3000, 128, "bf16"), (4, 16, 700, 128, "bf16"),
                                           (1, 2, 1000, 64, "f32")])
def test_bf16_output(B, H, L, d, dtype):
    Q, K, V = workloads.random_qkv(13, B, H, L, d)
    S_in, z_in = workloads.random_state(14, B, H, d)
    O_ref, _, _ = oracle.chunk_forward(Q, K, V, S_in, z_in, EPS)
    O, _ = run_chunk(Q, K, V, state_np(S_in, z_in), dtype, out_dtype=torch.bfloat16)
    eo = out_err(O, O_ref)
    # against the oracle rounded to bf16 (ties to even): within one ulp plus
    # the float32 arithmetic error, and equal to it almost everywhere
    excess, mismatch = bf16_rounding(O, O_ref, (2, 3), 2e-5)
    report(f"bf16 out B={B} H={H} L={L} d={d} {dtype} in", out=eo, ulp_excess=excess,
           mismatch=mismatch)
    assert excess <= 0.0 and mismatch <= BF16_MISMATCH_MAX, (excess, mismatch)


def test_binding_rejects_bad_buffers():
    B, H, L, d = 1, 1, 128, 64
    x = torch.zeros((B, H, L, d), dtype=torch.bfloat16, device="cuda")
    st = la.new_state(B, H, d)
    with pytest.raises(la.LinAttnError) as e:
        la.chunk_forward(x, x, x, st, out=x, eps=EPS)
    assert e.value.status == la.LA_E_ALIAS
    flat = torch.zeros(B * H * L * d + 8, dtype=torch.bfloat16, device="cuda")
    mis = flat[4:4 + B * H * L * d].view(B, H, L, d)
    with pytest.raises(la.LinAttnError) as e:
        la.global_forward(mis, x, x, eps=EPS)
    assert e.value.status == la.LA_E_ALIGN
    out = torch.empty((B, H, L, d), dtype=torch.float32, device="cuda")
    with pytest.raises(la.LinAttnError) as e:
        la.chunk_forward(x, x, x, st, out=out, state_out=out.view(-1)[: d * d + d].view(1, 1, -1),
                         eps=EPS)
    assert e.value.status == la.LA_E_ALIAS


# ---------------------------------------------------------------------------
# whole-sequence block-causal call (one call for all blocks)


def _prefix_ref(Q, K, V, T, S_in, z_in):
    """Oracle route that takes every block's KV first, prefix-sums them and
    then reads each block's queries (oracle.prefix_forward), plus S_in."""
    N = Q.shape[2]
    bounds = list(range(0, N, T)) + [N]
    O, S_pre, z_pre = oracle.prefix_forward(Q, K, V, bounds, EPS)
    if S_in is not None:
        # a non-zero initial state adds to every prefix; re-read the queries
        S_pre = S_pre + S_in[None]
        z_pre = z_pre + z_in[None]
        for n in range(len(bounds) - 1):
            a, b = bounds[n], bounds[n + 1]
            O[:, :, a:b] = oracle.readout(Q[:, :, a:b], S_pre[n], z_pre[n], EPS)
    return O, S_pre, z_pre


def _states_err(got, S_pre, z_pre):
    """max normwise error over blocks of a [B, H, C, d*d + d] states tensor."""
    worst = 0.0
    for n in range(S_pre.shape[0]):
        es, ez = state_err(got[:, :, n], S_pre[n], z_pre[n])
        worst = max(worst, es, ez)
    return worst


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d,N,T", [(64, 1000, 64), (64, 2085, 500), (32, 777, 7), (128, 1300, 256),
                                   (64, 300, 1), (64, 640, 640), (64, 500, 900), (128, 100, 33)])
def test_blockcausal_small(dtype, d, N, T):
    B, H = 2, 3
    Q, K, V = workloads.random_qkv(2000 + N + T, B, H, N, d, dtype=dtype)
    S_in, z_in = workloads.random_state(N + 7, B, H, d)
    S_in, z_in = S_in.astype(np.float64), z_in.astype(np.float64)
    O_ref, S_pre, z_pre = _prefix_ref(Q, K, V, T, S_in, z_in)
    st_in = torch.from_numpy(state_np(S_in, z_in)).cuda()
    out, states = la.blockcausal_forward(dev(Q, dtype), dev(K, dtype), dev(V, dtype), T,
                                         state_in=st_in, eps=EPS)
    torch.cuda.synchronize()
    eo = out_err(host(out), O_ref)
    es = _states_err(host(states), S_pre, z_pre)
    report(f"blockcausal {dtype} d={d} N={N} T={T}", out=eo, states=es)
    assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)
    assert torch.equal(st_in.cpu(), torch.from_numpy(state_np(S_in, z_in)))  # state_in untouched


def test_blockcausal_matches_chunk_calls():
    """One block-causal call == the same blocks through la_chunk_forward with
    the state carried (float32 summation order aside); zero initial state."""
    B, H, N, T, d = 1, 4, 5000, 1024, 64
    Q, K, V = workloads.random_qkv(31, B, H, N, d)
    q, k, v = dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16")
    out, states = la.blockcausal_forward(q, k, v, T, eps=EPS)
    st = la.new_state(B, H, d)
    for n, a in enumerate(range(0, N, T)):
        b = min(N, a + T)
        o, st = la.chunk_forward(q[:, :, a:b].contiguous(), k[:, :, a:b].contiguous(),
                                 v[:, :, a:b].contiguous(), st, state_out=st, eps=EPS)
        torch.cuda.synchronize()
        assert out_err(host(out[:, :, a:b]), host(o)) < 1e-5, n
        assert out_err(host(states[:, :, n]).reshape(B, H, -1, 1),
                       host(st).reshape(B, H, -1, 1)) < 1e-5, n
    # repeated runs are bitwise identical
    out2, states2 = la.blockcausal_forward(q, k, v, T, eps=EPS)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(states, states2)


def test_blockcausal_480p_1min_one_call():
    """The 1-minute 480p stream (12 blocks x 32,760 tokens, 16 heads) in one
    call, checked block by block against the prefix route."""
    w = workloads.WORKLOADS[4]
    N, T = w.L * w.chunks, w.L
    q = torch.empty((w.B, w.H, N, w.d), dtype=torch.bfloat16, device="cuda")
    k, v = torch.empty_like(q), torch.empty_like(q)
    blocks = []
    for n, (Qn, Kn, Vn) in drawn_chunks(lambda c: workloads.chunk_qkv(w, c), range(w.chunks)):
        sl = slice(n * T, (n + 1) * T)
        q[:, :, sl], k[:, :, sl], v[:, :, sl] = dev(Qn, "bf16"), dev(Kn, "bf16"), dev(Vn, "bf16")
        blocks.append((Qn, Kn, Vn))
    out, states = la.blockcausal_forward(q, k, v, T, eps=EPS)
    torch.cuda.synchronize()
    KVs, ks, worst = [], [], [0.0, 0.0]
    for n, (Qn, Kn, Vn) in enumerate(blocks):
        KV, kk = oracle.kv_of_block(Kn, Vn)
        KVs.append(KV)
        ks.append(kk)
        S = np.sum(np.stack(KVs), axis=0)
        z = np.sum(np.stack(ks), axis=0)
        O_ref = oracle.readout(Qn, S, z, EPS)
        eo = out_err(host(out[:, :, n * T:(n + 1) * T]), O_ref)
        es = max(state_err(host(states[:, :, n]), S, z))
        report(f"480p one-call block {n}", out=eo, state=es)
        worst = [max(worst[0], eo), max(worst[1], es)]
    assert max(worst) <= TOL["bf16"], worst


def test_blockcausal_long_horizon_d128_one_call():
    """The 40-block d = 128 long-horizon sequence (B=4, H=16, 163,840 tokens)
    in one call: every block's state, and the outputs of every fourth block
    and the last, against the fp64 carried state.  Each block is drawn once:
    the oracle's carried state and sampled outputs are formed as the blocks
    are uploaded."""
    w = workloads.WORKLOADS[5]
    N, T = w.L * w.chunks, w.L
    q = torch.empty((w.B, w.H, N, w.d), dtype=torch.bfloat16, device="cuda")
    k, v = torch.empty_like(q), torch.empty_like(q)
    S = np.zeros((w.B, w.H, w.d, w.d))
    z = np.zeros((w.B, w.H, w.d))
    ref_states, ref_outs = [], {}
    for n, (Qn, Kn, Vn) in drawn_chunks(lambda c: workloads.chunk_qkv(w, c), range(w.chunks)):
        sl = slice(n * T, (n + 1) * T)
        q[:, :, sl], k[:, :, sl], v[:, :, sl] = dev(Qn, "bf16"), dev(Kn, "bf16"), dev(Vn, "bf16")
        KV, kk = oracle.kv_of_block(Kn, Vn)
        S, z = S + KV, z + kk
        ref_states.append((S, z))
        if n % 4 == 0 or n == w.chunks - 1:
            ref_outs[n] = oracle.readout(Qn, S, z, EPS)
    out, states = la.blockcausal_forward(q, k, v, T, eps=EPS)
    torch.cuda.synchronize()
    worst = 0.0
    for n, (S, z) in enumerate(ref_states):
        es = max(state_err(host(states[:, :, n]), S, z))
        eo = 0.0
        if n in ref_outs:
            eo = out_err(host(out[:, :, n * T:(n + 1) * T]), ref_outs[n])
            report(f"long-horizon one-call block {n}", out=eo, state=es)
        else:
            report(f"long-horizon one-call block {n}", state=es)
        worst = max(worst, eo, es)
    assert worst <= TOL["bf16"], worst


# ---------------------------------------------------------------------------
# the largest sequence the ABI accepts: N * d < 2^31 elements per head


def test_max_size_sequence():
    """One head of 2^25 - 1 tokens at d = 64 (N * d = 2^31 - 64), drawn on
    the GPU from a seeded generator: la_global_forward and
    la_blockcausal_forward with two blocks of 2^24 tokens.  The states are
    compared whole against the oracle's fp64 sums (accumulated over host
    chunks), the outputs on sampled rows that include the first and last
    token of each block."""
    N, d, T = (1 << 25) - 1, 64, 1 << 24
    gen = torch.Generator(device="cuda").manual_seed(20251203)
    q, k, v = (torch.randn((1, 1, N, d), generator=gen, device="cuda").to(torch.bfloat16)
               for _ in range(3))
    out = torch.empty((1, 1, N, d), dtype=torch.float32, device="cuda")
    _, st = la.global_forward(q, k, v, out=out, eps=EPS)
    torch.cuda.synchronize()

    S = np.zeros((1, 1, d, d))
    z = np.zeros((1, 1, d))
    S_half = z_half = None
    step = 1 << 21
    for c0 in range(0, N, step):
        Kc = host(k[:, :, c0:c0 + step])
        Vc = host(v[:, :, c0:c0 + step])
        KV, kk = oracle.kv_of_block(Kc, Vc)
        S, z = S + KV, z + kk
        if c0 + step == T:
            S_half, z_half = S.copy(), z.copy()
    es, ez = state_err(host(st), S, z)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, T - 1, T, N - 2, N - 1],
                                     rng.integers(0, N, 4000)]))
    Qs = host(q[:, :, torch.from_numpy(rows).cuda()])
    eo = out_err(host(out[:, :, torch.from_numpy(rows).cuda()]), oracle.readout(Qs, S, z, EPS))
    report("max-size global", out=eo, S=es, z=ez)
    assert max(eo, es, ez) <= TOL["bf16"], (eo, es, ez)

    _, states = la.blockcausal_forward(q, k, v, T, out=out, eps=EPS)
    torch.cuda.synchronize()
    e0 = max(state_err(host(states[:, :, 0]), S_half, z_half))
    e1 = max(state_err(host(states[:, :, 1]), S, z))
    o = host(out[:, :, torch.from_numpy(rows).cuda()])
    first = rows < T
    eo0 = out_err(o[:, :, first], oracle.readout(Qs[:, :, first], S_half, z_half, EPS))
    eo1 = out_err(o[:, :, ~first], oracle.readout(Qs[:, :, ~first], S, z, EPS))
    report("max-size block-causal", out0=eo0, out1=eo1, state0=e0, state1=e1)
    assert max(e0, e1, eo0, eo1) <= TOL["bf16"], (e0, e1, eo0, eo1)
