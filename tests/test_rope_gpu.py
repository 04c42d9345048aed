"""GPU parity of the rotary-position calls (la_chunk_forward_rope,
la_blockcausal_forward_rope) against the fp64 oracle (``oracle.rope_*``) on
the same seeded inputs.  Bounds as for the plain calls: normwise per (b, h)
slice, 1e-5 for float32 inputs and 2e-3 for bfloat16 inputs (float32
output); states compared the same way.  Latent grids per workload come from
``workloads.GRIDS``.
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
THETA = workloads.ROPE_THETA


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.lib()
    yield
    torch.cuda.synchronize()


def _bounds(N, T):
    return list(range(0, N, T)) + [N]


def _states_err(got, S_pre, z_pre):
    worst = 0.0
    for n in range(S_pre.shape[0]):
        worst = max(worst, *state_err(got[:, :, n], S_pre[n], z_pre[n]))
    return worst


# ---------------------------------------------------------------------------
# small shapes: several tiles, ragged tails, frames that do not divide the block


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("L", [1, 15, 333, 2085])
def test_rope_chunk_small(dtype, d, L):
    B, H, gh, gw, f0 = 2, 3, 3, 5, 7
    Q, K, V = workloads.random_qkv(3000 + L, B, H, L, d, dtype=dtype)
    S_in, z_in = workloads.random_state(L + d + 1, B, H, d)
    S_in, z_in = S_in.astype(np.float64), z_in.astype(np.float64)
    O_ref, S_ref, z_ref = oracle.rope_chunk_forward(Q, K, V, S_in, z_in, EPS, f0, gh, gw, THETA)
    st_in = torch.from_numpy(state_np(S_in, z_in)).cuda()
    out, st = la.chunk_forward_rope(dev(Q, dtype), dev(K, dtype), dev(V, dtype), st_in, f0, gh,
                                    gw, THETA, eps=EPS)
    torch.cuda.synchronize()
    eo = out_err(host(out), O_ref)
    es, ez = state_err(host(st), S_ref, z_ref)
    report(f"rope chunk {dtype} d={d} L={L}", out=eo, S=es, z=ez)
    assert eo <= TOL[dtype] and es <= TOL[dtype] and ez <= TOL[dtype], (eo, es, ez)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d,N,T,gh,gw,f0", [(64, 1000, 64, 4, 4, 0), (64, 2085, 500, 5, 10, 3),
                                            (32, 777, 7, 1, 7, 11), (128, 1300, 256, 8, 8, 0),
                                            (64, 300, 1, 1, 1, 2), (128, 100, 33, 2, 3, 5)])
def test_rope_blockcausal_small(dtype, d, N, T, gh, gw, f0):
    B, H = 2, 3
    Q, K, V = workloads.random_qkv(4000 + N + T, B, H, N, d, dtype=dtype)
    S_in, z_in = workloads.random_state(N + 17, B, H, d)
    S_in, z_in = S_in.astype(np.float64), z_in.astype(np.float64)
    O_ref, S_pre, z_pre = oracle.rope_prefix_forward(Q, K, V, _bounds(N, T), EPS, f0, gh, gw,
                                                     THETA, S_in, z_in)
    st_in = torch.from_numpy(state_np(S_in, z_in)).cuda()
    out, states = la.blockcausal_forward_rope(dev(Q, dtype), dev(K, dtype), dev(V, dtype), T, f0,
                                              gh, gw, THETA, state_in=st_in, eps=EPS)
    torch.cuda.synchronize()
    eo = out_err(host(out), O_ref)
    es = _states_err(host(states), S_pre, z_pre)
    report(f"rope blockcausal {dtype} d={d} N={N} T={T}", out=eo, states=es)
    assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rope_global_form(dtype):
    """T >= N with no state_in: the global form (one block)."""
    B, H, N, d, gh, gw = 1, 2, 1500, 64, 6, 10
    Q, K, V = workloads.random_qkv(41, B, H, N, d, dtype=dtype)
    O_ref, S_pre, z_pre = oracle.rope_prefix_forward(Q, K, V, [0, N], EPS, 0, gh, gw, THETA)
    out, states = la.blockcausal_forward_rope(dev(Q, dtype), dev(K, dtype), dev(V, dtype), N, 0,
                                              gh, gw, THETA, eps=EPS)
    torch.cuda.synchronize()
    eo = out_err(host(out), O_ref)
    es = _states_err(host(states), S_pre, z_pre)
    report(f"rope global {dtype}", out=eo, state=es)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rope_global_call(dtype):
    """la_global_forward_rope against the oracle, and bit for bit against the
    block-causal call with one block (the same kernels)."""
    B, H, N, d, gh, gw, f0 = 2, 2, 2500, 64, 7, 9, 3
    Q, K, V = workloads.random_qkv(45, B, H, N, d, dtype=dtype)
    O_ref, S_pre, z_pre = oracle.rope_prefix_forward(Q, K, V, [0, N], EPS, f0, gh, gw, THETA)
    q, k, v = dev(Q, dtype), dev(K, dtype), dev(V, dtype)
    out, st = la.global_forward_rope(q, k, v, f0, gh, gw, THETA, eps=EPS)
    out2, sts = la.blockcausal_forward_rope(q, k, v, N, f0, gh, gw, THETA, eps=EPS)
    torch.cuda.synchronize()
    eo = out_err(host(out), O_ref)
    es, ez = state_err(host(st), S_pre[0], z_pre[0])
    report(f"rope global call {dtype}", out=eo, S=es, z=ez)
    assert max(eo, es, ez) <= TOL[dtype]
    assert torch.equal(out, out2) and torch.equal(st, sts[:, :, 0])


def test_rope_global_call_empty():
    """N = 0: the state is zero."""
    e = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    _, st = la.global_forward_rope(e, e, e, 0, 4, 4, THETA, eps=EPS)
    torch.cuda.synchronize()
    assert torch.count_nonzero(st) == 0


@pytest.mark.parametrize("f0", [4_000_000, -3_000_001])
def test_rope_large_frame_offset(f0):
    """Tokens millions of frames into a stream (or before its origin, which
    the ABI allows): the angle reduction keeps float resolution in turns
    (bf16 and f32 inputs)."""
    B, H, L, d, gh, gw = 1, 2, 700, 64, 5, 7
    for dtype in ("bf16", "f32"):
        Q, K, V = workloads.random_qkv(43, B, H, L, d, dtype=dtype)
        S_in, z_in = workloads.random_state(44, B, H, d)
        S_in, z_in = S_in.astype(np.float64), z_in.astype(np.float64)
        O_ref, S_ref, z_ref = oracle.rope_chunk_forward(Q, K, V, S_in, z_in, EPS, f0, gh, gw,
                                                        THETA)
        st_in = torch.from_numpy(state_np(S_in, z_in)).cuda()
        out, st = la.chunk_forward_rope(dev(Q, dtype), dev(K, dtype), dev(V, dtype), st_in, f0,
                                        gh, gw, THETA, eps=EPS)
        torch.cuda.synchronize()
        eo = out_err(host(out), O_ref)
        es, ez = state_err(host(st), S_ref, z_ref)
        report(f"rope frame0={f0} {dtype}", out=eo, S=es, z=ez)
        assert eo <= TOL[dtype] and es <= TOL[dtype] and ez <= TOL[dtype], (eo, es, ez)


def test_rope_bf16_output_and_theta():
    B, H, L, d, gh, gw = 1, 4, 3000, 64, 10, 10
    Q, K, V = workloads.random_qkv(45, B, H, L, d)
    S_in, z_in = workloads.random_state(46, B, H, d)
    S_in, z_in = S_in.astype(np.float64), z_in.astype(np.float64)
    st_in = torch.from_numpy(state_np(S_in, z_in)).cuda()
    for theta, out_dtype in ((THETA, torch.bfloat16), (500.0, torch.float32), (1.0, torch.float32)):
        O_ref, _, _ = oracle.rope_chunk_forward(Q, K, V, S_in, z_in, EPS, 2, gh, gw, theta)
        out, _ = la.chunk_forward_rope(dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), st_in, 2,
                                       gh, gw, theta, eps=EPS, out_dtype=out_dtype)
        torch.cuda.synchronize()
        eo = out_err(host(out), O_ref)
        report(f"rope theta={theta} out={out_dtype}", out=eo)
        if out_dtype == torch.bfloat16:
            # against the oracle rounded to bf16 (ties to even)
            excess, mismatch = bf16_rounding(host(out), O_ref, (2, 3), 2e-5)
            report(f"rope theta={theta} bf16 rounding", ulp_excess=excess, mismatch=mismatch)
            assert excess <= 0.0 and mismatch <= BF16_MISMATCH_MAX, (excess, mismatch)
        else:
            assert eo <= TOL["bf16"], eo


def test_rope_chunk_calls_match_one_call():
    """Block calls with frame0 advanced by the frames of each block (the
    state carried in place) == one block-causal call (float32 summation
    order aside); repeated calls are bitwise identical."""
    B, H, N, T, d, gh, gw = 1, 4, 5120, 1024, 64, 16, 16
    Q, K, V = workloads.random_qkv(47, B, H, N, d)
    q, k, v = dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16")
    out, states = la.blockcausal_forward_rope(q, k, v, T, 3, gh, gw, THETA, eps=EPS)
    st = la.new_state(B, H, d)
    for n, a in enumerate(range(0, N, T)):
        o, st = la.chunk_forward_rope(q[:, :, a:a + T].contiguous(), k[:, :, a:a + T].contiguous(),
                                      v[:, :, a:a + T].contiguous(), st, 3 + a // (gh * gw), gh,
                                      gw, THETA, state_out=st, eps=EPS)
        torch.cuda.synchronize()
        assert out_err(host(out[:, :, a:a + T]), host(o)) < 1e-5, n
        assert out_err(host(states[:, :, n]).reshape(B, H, -1, 1),
                       host(st).reshape(B, H, -1, 1)) < 1e-5, n
    out2, states2 = la.blockcausal_forward_rope(q, k, v, T, 3, gh, gw, THETA, eps=EPS)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(states, states2)


def test_rope_empty():
    B, H, d = 1, 3, 64
    S_in, z_in = workloads.random_state(48, B, H, d)
    st_in = torch.from_numpy(state_np(S_in, z_in)).cuda()
    e = torch.empty((B, H, 0, d), dtype=torch.bfloat16, device="cuda")
    out, st = la.chunk_forward_rope(e, e, e, st_in, 0, 4, 4, THETA, eps=EPS)
    torch.cuda.synchronize()
    assert out.shape == (B, H, 0, d) and torch.equal(st, st_in)


# ---------------------------------------------------------------------------
# the video workloads at full size


def test_rope_720p_chunk():
    """Chunk 1 of a 720p latent (frames 21..41 of 45 x 80 tokens) against the
    state left by chunk 0 (frames 0..20), both rotated by absolute position."""
    w = workloads.CHUNK_720P
    gh, gw = workloads.GRIDS[w.cid]
    Q0, K0, V0 = workloads.chunk_qkv(w, 0)
    S0, z0 = oracle.zero_state(w.B, w.H, w.d)
    _, S0, z0 = oracle.rope_chunk_forward(Q0, K0, V0, S0, z0, EPS, 0, gh, gw, THETA)
    del Q0, K0, V0
    st0_np = state_np(S0, z0)  # the float32 state the GPU receives
    d = w.d
    S0 = st0_np[..., : d * d].reshape(S0.shape).astype(np.float64)
    z0 = st0_np[..., d * d:].astype(np.float64)
    Q1, K1, V1 = workloads.chunk_qkv(w, 1)
    f1 = workloads.chunk_frame0(w, 1)
    out, st1 = la.chunk_forward_rope(dev(Q1, "bf16"), dev(K1, "bf16"), dev(V1, "bf16"),
                                     torch.from_numpy(st0_np).cuda(), f1, gh, gw, THETA, eps=EPS)
    torch.cuda.synchronize()
    O_ref, S_ref, z_ref = oracle.rope_chunk_forward(Q1, K1, V1, S0, z0, EPS, f1, gh, gw, THETA)
    eo = out_err(host(out), O_ref)
    es, ez = state_err(host(st1), S_ref, z_ref)
    report("rope 720p chunk", out=eo, S=es, z=ez)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"] and ez <= TOL["bf16"]


def test_rope_480p_1min_one_call():
    """The 1-minute 480p stream (12 blocks of 21 frames of 30 x 52 tokens) in
    one call: every block's state and the outputs of blocks 0, 5 and 11
    against the oracle's carried state."""
    w = workloads.WORKLOADS[4]
    gh, gw = workloads.GRIDS[w.cid]
    N, T = w.L * w.chunks, w.L
    q = torch.empty((w.B, w.H, N, w.d), dtype=torch.bfloat16, device="cuda")
    k, v = torch.empty_like(q), torch.empty_like(q)
    # each block is drawn once: the oracle carries its state as the blocks are uploaded
    S, z = oracle.zero_state(w.B, w.H, w.d)
    ref_states, ref_outs = [], {}
    for n, (Qn, Kn, Vn) in drawn_chunks(lambda c: workloads.chunk_qkv(w, c), range(w.chunks)):
        sl = slice(n * T, (n + 1) * T)
        q[:, :, sl], k[:, :, sl], v[:, :, sl] = dev(Qn, "bf16"), dev(Kn, "bf16"), dev(Vn, "bf16")
        O_ref, S, z = oracle.rope_chunk_forward(Qn, Kn, Vn, S, z, EPS, workloads.chunk_frame0(w, n),
                                                gh, gw, THETA)
        ref_states.append((S, z))
        if n in (0, 5, w.chunks - 1):
            ref_outs[n] = O_ref
    out, states = la.blockcausal_forward_rope(q, k, v, T, 0, gh, gw, THETA, eps=EPS)
    torch.cuda.synchronize()
    worst = 0.0
    for n, (S, z) in enumerate(ref_states):
        es = max(state_err(host(states[:, :, n]), S, z))
        if n in ref_outs:
            eo = out_err(host(out[:, :, n * T:(n + 1) * T]), ref_outs[n])
            report(f"rope 480p one-call block {n}", out=eo, state=es)
            worst = max(worst, eo)
        else:
            report(f"rope 480p one-call block {n}", state=es)
        worst = max(worst, es)
    assert worst <= TOL["bf16"], worst


def test_rope_long_horizon_d128_one_call():
    """The 40-block d = 128 sequence (B=4, H=16, 163,840 tokens, four 32 x 32
    frames per block, 1% outlier rows) in one call; the oracle checks heads
    (0, 0), (1, 7) and (3, 15) whole: every block's state and output."""
    w = workloads.WORKLOADS[5]
    gh, gw = workloads.GRIDS[w.cid]
    N, T = w.L * w.chunks, w.L
    heads = [(0, 0), (1, 7), (3, 15)]
    q = torch.empty((w.B, w.H, N, w.d), dtype=torch.bfloat16, device="cuda")
    k, v = torch.empty_like(q), torch.empty_like(q)
    Qs, Ks, Vs = ([np.empty((N, w.d), dtype=np.float32) for _ in heads] for _ in range(3))
    for n, (Qn, Kn, Vn) in drawn_chunks(lambda c: workloads.chunk_qkv(w, c), range(w.chunks)):
        sl = slice(n * T, (n + 1) * T)
        q[:, :, sl], k[:, :, sl], v[:, :, sl] = dev(Qn, "bf16"), dev(Kn, "bf16"), dev(Vn, "bf16")
        for i, (b, h) in enumerate(heads):
            Qs[i][sl], Ks[i][sl], Vs[i][sl] = Qn[b, h], Kn[b, h], Vn[b, h]
    out, states = la.blockcausal_forward_rope(q, k, v, T, 0, gh, gw, THETA, eps=EPS)
    torch.cuda.synchronize()
    worst = 0.0
    for i, (b, h) in enumerate(heads):
        O_ref, S_pre, z_pre = oracle.rope_prefix_forward(
            Qs[i][None, None], Ks[i][None, None], Vs[i][None, None], _bounds(N, T), EPS, 0, gh,
            gw, THETA)
        eo = max(out_err(host(out[b:b + 1, h:h + 1, a:a + T]), O_ref[:, :, a:a + T])
                 for a in range(0, N, T))
        es = _states_err(host(states[b:b + 1, h:h + 1]), S_pre, z_pre)
        report(f"rope long-horizon one-call head ({b},{h})", out=eo, states=es)
        worst = max(worst, eo, es)
    assert worst <= TOL["bf16"], worst


# ---------------------------------------------------------------------------
# the longest rotary sequence the ABI accepts: token indices below 2^22 - 64


def test_rope_max_size_sequence():
    """One head of 2^22 - 65 tokens at d = 64 on a 32 x 64 grid starting at
    frame 1,000,003, drawn on the GPU: la_blockcausal_forward_rope with two
    blocks of 2^21 tokens.  Both block states are compared whole against the
    oracle's sums over frame-aligned host chunks (rope_chunk_forward carrying
    the state); the outputs on whole sampled frames, including the last frame
    of block 0, the first of block 1 and the ragged last frame, against
    rope_chunk_forward of that frame with keys that phi maps to zero (so the
    block's state is read unchanged)."""
    d, gh, gw, f0 = 64, 32, 64, 1_000_003
    hw = gh * gw
    N, T = (1 << 22) - 65, 1 << 21
    gen = torch.Generator(device="cuda").manual_seed(20261203)
    q, k, v = (torch.randn((1, 1, N, d), generator=gen, device="cuda").to(torch.bfloat16)
               for _ in range(3))
    out, states = la.blockcausal_forward_rope(q, k, v, T, f0, gh, gw, THETA, eps=EPS)
    torch.cuda.synchronize()

    S, z = oracle.zero_state(1, 1, d)
    block_states = []
    step = 1 << 20  # a whole number of frames
    for c0 in range(0, N, step):
        Kc, Vc = host(k[:, :, c0:c0 + step]), host(v[:, :, c0:c0 + step])
        _, S, z = oracle.rope_chunk_forward(-np.ones_like(Kc), Kc, Vc, S, z, EPS,
                                            f0 + c0 // hw, gh, gw, THETA)
        if c0 + step in (T, N) or c0 + step > N:
            block_states.append((S.copy(), z.copy()))
    assert len(block_states) == 2
    es = [max(state_err(host(states[:, :, n]), *block_states[n])) for n in range(2)]

    last = (N - 1) // hw
    frames = sorted({0, T // hw - 1, T // hw, last} | set(
        np.random.default_rng(9).integers(0, last, 3).tolist()))
    worst = 0.0
    for f in frames:
        a, b = f * hw, min(N, (f + 1) * hw)
        n = 0 if a < T else 1
        Qf = host(q[:, :, a:b])
        O_ref, S_chk, _ = oracle.rope_chunk_forward(Qf, -np.ones_like(Qf), np.zeros_like(Qf),
                                                    *block_states[n], EPS, f0 + f, gh, gw, THETA)
        assert np.array_equal(S_chk, block_states[n][0])
        eo = out_err(host(out[:, :, a:b]), O_ref)
        report(f"rope max-size frame {f} (block {n}, {b - a} tokens)", out=eo)
        worst = max(worst, eo)
    report("rope max-size states", S0=es[0], S1=es[1])
    assert max(worst, *es) <= TOL["bf16"], (worst, es)


def test_rope_degenerate_rows():
    """With the rotation, as without: an all-non-positive query row gives
    exactly 0, and all-non-positive key rows contribute nothing (the result
    is bitwise unchanged whatever their values)."""
    B, H, N, T, d, gh, gw, f0 = 1, 2, 700, 300, 64, 5, 8, 2
    Q, K, V = workloads.random_qkv(131, B, H, N, d)
    Q[:, :, 7] = -np.abs(Q[:, :, 7])
    K[:, :, 100:150] = -np.abs(K[:, :, 100:150])
    V2 = V.copy()
    V2[:, :, 100:150] = workloads.random_qkv(132, B, H, 50, d)[2]
    args = (T, f0, gh, gw, THETA)
    out, st = la.blockcausal_forward_rope(dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), *args,
                                          eps=EPS)
    out2, st2 = la.blockcausal_forward_rope(dev(Q, "bf16"), dev(K, "bf16"), dev(V2, "bf16"),
                                            *args, eps=EPS)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[:, :, 7]) == 0
    assert torch.equal(out, out2) and torch.equal(st, st2)
    O_ref, _, _ = oracle.rope_prefix_forward(Q, K, V, _bounds(N, T), EPS, f0, gh, gw, THETA)
    assert out_err(host(out), O_ref) <= TOL["bf16"]


def test_rope_zero_eps_ragged():
    """eps = 0 with every denominator kept > 0: rows past the ragged end of a
    tile and of a block stay out of every sum, so nothing turns into NaN."""
    B, H, N, T, d, gh, gw = 1, 2, 1000, 300, 64, 7, 9
    Q, K, V = workloads.random_qkv(133, B, H, N, d)
    Q[..., 0] = np.abs(Q[..., 0]) + 0.25
    K[..., 0] = np.abs(K[..., 0]) + 0.25
    Q, K = workloads.bf16_round(Q), workloads.bf16_round(K)
    out, st = la.blockcausal_forward_rope(dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), T, 4,
                                          gh, gw, THETA, eps=0.0)
    torch.cuda.synchronize()
    got = host(out)
    assert np.all(np.isfinite(got))
    O_ref, S_pre, z_pre = oracle.rope_prefix_forward(Q, K, V, _bounds(N, T), 0.0, 4, gh, gw,
                                                     THETA)
    eo = out_err(got, O_ref)
    es = _states_err(host(st), S_pre, z_pre)
    report("rope eps=0", out=eo, state=es)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("d,dtype", [(32, "bf16"), (128, "bf16"), (64, "f32")])
def test_rope_bf16_output_every_readout(d, dtype):
    """bfloat16 rows from the rotary readouts not covered above (d = 32 and
    128 on bf16 inputs, the float32-input readout): against the oracle
    rounded to bf16, within one ulp plus the float32 arithmetic error and
    equal to it almost everywhere."""
    B, H, L, gh, gw = 1, 3, 2085, 3, 5
    Q, K, V = workloads.random_qkv(47 + d, B, H, L, d)
    S_in, z_in = workloads.random_state(48 + d, B, H, d)
    S_in, z_in = S_in.astype(np.float64), z_in.astype(np.float64)
    O_ref, _, _ = oracle.rope_chunk_forward(Q, K, V, S_in, z_in, EPS, 7, gh, gw, THETA)
    st_in = torch.from_numpy(state_np(S_in, z_in)).cuda()
    out, _ = la.chunk_forward_rope(dev(Q, dtype), dev(K, dtype), dev(V, dtype), st_in, 7, gh, gw,
                                   THETA, eps=EPS, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    excess, mismatch = bf16_rounding(host(out), O_ref, (2, 3), 2e-5)
    report(f"rope bf16 out d={d} {dtype} in", out=out_err(host(out), O_ref), ulp_excess=excess,
           mismatch=mismatch)
    assert excess <= 0.0 and mismatch <= BF16_MISMATCH_MAX, (excess, mismatch)
