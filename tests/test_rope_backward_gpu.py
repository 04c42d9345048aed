"""GPU parity of the rotary-position gradients (la_blockcausal_backward_rope,
through the C ABI) against the fp64 oracle's ``rope_blockcausal_backward``
on the same seeded inputs.

Error: normwise per (b, h, block) slice, max |got - ref| / max |ref|, the
largest over slices.  Bounds as for the plain backward: 2e-3 for bfloat16
inputs, 1e-5 for float32 inputs (float32 gradients), 2^-8 for bfloat16
gradients.  The backward reads the states the GPU's rotary forward wrote.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import (BF16_MISMATCH_MAX, TOL, bf16_rounding, dev, host, normwise, report,
                     state_err, state_np)

import block_causal_linear_amd as la

pytestmark = pytest.mark.gpu
EPS = workloads.EPS
THETA = workloads.ROPE_THETA
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
    return max(normwise(got[:, :, a:b], ref[:, :, a:b], axes=(2, 3))
               for a, b in zip(bounds[:-1], bounds[1:]))


def pack_dstates(dS, dz):
    """[C, B, H, d, d], [C, B, H, d] -> [B, H, C, d*d + d] float32."""
    C, B, H, d, _ = dS.shape
    x = np.concatenate([dS.reshape(C, B, H, d * d), dz], axis=-1)
    return np.ascontiguousarray(np.transpose(x, (1, 2, 0, 3)), dtype=np.float32)


def gpu_backward(Q, K, V, dO, T, dtype, f0, gh, gw, gdt="f32", state_in=None, dstates=None,
                 want_dstate_in=False, theta=THETA):
    q, k, v = dev(Q, dtype), dev(K, dtype), dev(V, dtype)
    st_in = None if state_in is None else torch.from_numpy(state_in).cuda()
    _, states = la.blockcausal_forward_rope(q, k, v, T, f0, gh, gw, theta, state_in=st_in,
                                            eps=EPS)
    ds = None if dstates is None else torch.from_numpy(dstates).cuda()
    dq, dk, dv, dsi = la.blockcausal_backward_rope(q, k, v, states, dev(dO, gdt), T, f0, gh, gw,
                                                   theta, dstates=ds,
                                                   want_dstate_in=want_dstate_in, eps=EPS)
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv), None if dsi is None else host(dsi)


def check(name, got, ref, bounds, tol, dsi=None, dsi_ref=None):
    vals = dict(zip(("dq", "dk", "dv"), (grad_err(g, r, bounds) for g, r in zip(got, ref))))
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
# small shapes: several tiles, ragged tails, frames that do not divide the
# block, one-token blocks, a state input and gradients on every block's state

CASES = [(1000, 64, 4, 4, 0), (2085, 500, 5, 10, 3), (777, 7, 1, 7, 11), (1300, 256, 8, 8, 0),
         (300, 1, 1, 1, 2), (100, 33, 2, 3, 5)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("N,T,gh,gw,f0", CASES)
def test_rope_backward_small(dtype, d, N, T, gh, gw, f0):
    B, H = 2, 3
    Q, K, V = workloads.random_qkv(5000 + N + d, B, H, N, d, dtype=dtype)
    dO = workloads.random_grads(5100 + N + d, B, H, N, d)
    S0, z0 = workloads.random_state(N + T + d, B, H, d)
    bounds = bounds_of(N, T)
    C = len(bounds) - 1
    dS, dz = workloads.random_state_grads(N + 5 * d, B, H, C, d)
    got = gpu_backward(Q, K, V, dO, T, dtype, f0, gh, gw, state_in=state_np(S0, z0),
                       dstates=pack_dstates(dS, dz), want_dstate_in=True)
    ref = oracle.rope_blockcausal_backward(Q, K, V, bounds, dO, EPS, f0, gh, gw, THETA,
                                           S0.astype(np.float64), z0.astype(np.float64),
                                           dS.astype(np.float64), dz.astype(np.float64))
    check(f"rope backward {dtype} d={d} N={N} T={T} grid={gh}x{gw} f0={f0}", got[:3], ref[:3],
          bounds, TOL[dtype], got[3], ref[3:])


@pytest.mark.parametrize("d", [32, 64, 128])
def test_rope_backward_bf16_gradients(d):
    """bfloat16 dO in, bfloat16 dq/dk/dv out."""
    B, H, N, T, gh, gw = 1, 2, 1300, 300, 6, 9
    Q, K, V = workloads.random_qkv(51 + d, B, H, N, d)
    dO = workloads.random_grads(52 + d, B, H, N, d, dtype="bf16")
    got = gpu_backward(Q, K, V, dO, T, "bf16", 4, gh, gw, gdt="bf16")
    ref = oracle.rope_blockcausal_backward(Q, K, V, bounds_of(N, T), dO, EPS, 4, gh, gw, THETA)
    check(f"rope backward bf16 grads d={d}", got[:3], ref[:3], bounds_of(N, T), BF16_OUT_TOL)
    check_bf16_grads(f"rope backward bf16 grads d={d}", got[:3], ref[:3], bounds_of(N, T))


@pytest.mark.parametrize("f0", [4_000_000, -3_000_001])
def test_rope_backward_large_frame_offset(f0):
    """Frame indices in the millions (and negative): the angles are reduced
    to turns in two parts, so the gradients keep their accuracy."""
    B, H, N, T, d, gh, gw = 1, 2, 1500, 400, 64, 3, 7
    Q, K, V = workloads.random_qkv(61, B, H, N, d)
    dO = workloads.random_grads(62, B, H, N, d)
    S0, z0 = workloads.random_state(63, B, H, d)
    C = len(bounds_of(N, T)) - 1
    dS, dz = workloads.random_state_grads(64, B, H, C, d)
    got = gpu_backward(Q, K, V, dO, T, "bf16", f0, gh, gw, state_in=state_np(S0, z0),
                       dstates=pack_dstates(dS, dz), want_dstate_in=True)
    ref = oracle.rope_blockcausal_backward(Q, K, V, bounds_of(N, T), dO, EPS, f0, gh, gw, THETA,
                                           S0.astype(np.float64), z0.astype(np.float64),
                                           dS.astype(np.float64), dz.astype(np.float64))
    check(f"rope backward f0={f0}", got[:3], ref[:3], bounds_of(N, T), TOL["bf16"], got[3],
          ref[3:])


def test_rope_backward_theta_and_one_frame_blocks():
    """Another base (theta = 500) and blocks of exactly one frame."""
    B, H, d, gh, gw = 1, 3, 64, 4, 5
    T, N = gh * gw, 7 * gh * gw
    Q, K, V = workloads.random_qkv(71, B, H, N, d)
    dO = workloads.random_grads(72, B, H, N, d)
    got = gpu_backward(Q, K, V, dO, T, "bf16", 1, gh, gw, theta=500.0)
    ref = oracle.rope_blockcausal_backward(Q, K, V, bounds_of(N, T), dO, EPS, 1, gh, gw, 500.0)
    check("rope backward theta=500", got[:3], ref[:3], bounds_of(N, T), TOL["bf16"])


def test_rope_backward_reproducible():
    """The same launch twice gives identical bits."""
    B, H, N, T, d = 1, 2, 20000, 20000, 64
    Q, K, V = workloads.random_qkv(81, B, H, N, d)
    dO = workloads.random_grads(82, B, H, N, d)
    a = gpu_backward(Q, K, V, dO, T, "bf16", 0, 30, 52, want_dstate_in=True)
    b = gpu_backward(Q, K, V, dO, T, "bf16", 0, 30, 52, want_dstate_in=True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_rope_backward_empty():
    """N = 0: no blocks, nothing to write; the call succeeds."""
    e = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    states = torch.empty((1, 2, 0, 64 * 64 + 64), dtype=torch.float32, device="cuda")
    dq, dk, dv, _ = la.blockcausal_backward_rope(e, e, e, states, e.float(), 16, 0, 4, 4, THETA,
                                                 eps=EPS)
    torch.cuda.synchronize()
    assert dq.shape == e.shape and dk.shape == e.shape and dv.shape == e.shape


# ---------------------------------------------------------------------------
# full size


def test_rope_backward_720p_chunk():
    """Chunk 1 of a 720p latent (B=1, H=32, d=64, 75,600 tokens, frames
    21..41 of 45 x 80 tokens) against the rotated state left by chunk 0, with
    a gradient on state_out: every element."""
    w = workloads.CHUNK_720P
    gh, gw = workloads.GRIDS[w.cid]
    Q0, K0, V0 = workloads.chunk_qkv(w, 0)
    S0, z0 = oracle.zero_state(w.B, w.H, w.d)
    _, S0, z0 = oracle.rope_chunk_forward(Q0, K0, V0, S0, z0, EPS, 0, gh, gw, THETA)
    del Q0, K0, V0
    st0 = state_np(S0, z0)  # the float32 state the GPU receives
    d = w.d
    S0 = st0[..., : d * d].reshape(S0.shape).astype(np.float64)
    z0 = st0[..., d * d:].astype(np.float64)
    Q, K, V = workloads.chunk_qkv(w, 1)
    f1 = workloads.chunk_frame0(w, 1)
    dO = workloads.random_grads(3, w.B, w.H, w.L, w.d, chunk=1)
    dS, dz = workloads.random_state_grads(3, w.B, w.H, 1, w.d, scale=1e-5)
    got = gpu_backward(Q, K, V, dO, w.L, "bf16", f1, gh, gw, state_in=st0,
                       dstates=pack_dstates(dS, dz), want_dstate_in=True)
    ref = oracle.rope_blockcausal_backward(Q, K, V, [0, w.L], dO, EPS, f1, gh, gw, THETA, S0, z0,
                                           dS.astype(np.float64), dz.astype(np.float64))
    check("rope 720p chunk backward", got[:3], ref[:3], [0, w.L], TOL["bf16"], got[3], ref[3:])


def test_rope_backward_max_size_sequence():
    """The longest rotary sequence accepted (2^22 - 65 tokens at d = 64, a
    32 x 64 grid from frame 1,000,003, two blocks of 2^21 tokens).  The
    oracle runs per frame-aligned host chunk, from its own functions only:
      * the block states: rope_chunk_forward carrying the state;
      * dq of every query: rope_blockcausal_backward of the chunk as one
        block whose keys phi maps to zero, reading the block's state; its
        dS0, dz0 are the chunk's share of the block's state gradient;
      * dk, dv of every key in two chunks (the last of block 0 and the ragged
        last one): rope_blockcausal_backward with dO = 0 and the suffix of
        the blocks' state gradients given as the block's state gradient."""
    d, gh, gw, f0 = 64, 32, 64, 1_000_003
    hw = gh * gw
    N, T = (1 << 22) - 65, 1 << 21
    gen = torch.Generator(device="cuda").manual_seed(20261204)
    q, k, v = (torch.randn((1, 1, N, d), generator=gen, device="cuda").to(torch.bfloat16)
               for _ in range(3))
    do = torch.randn((1, 1, N, d), generator=gen, device="cuda")
    _, states = la.blockcausal_forward_rope(q, k, v, T, f0, gh, gw, THETA, eps=EPS)
    dq, dk, dv, _ = la.blockcausal_backward_rope(q, k, v, states, do, T, f0, gh, gw, THETA,
                                                 eps=EPS)
    torch.cuda.synchronize()
    del states

    step = 1 << 20  # a whole number of frames; blocks are two steps each
    chunks = [(c0, min(N, c0 + step)) for c0 in range(0, N, step)]
    block_of = [0 if c0 < T else 1 for c0, _ in chunks]
    S, z = oracle.zero_state(1, 1, d)
    block_states = []
    for (a, b), n in zip(chunks, block_of):
        Kc, Vc = host(k[:, :, a:b]), host(v[:, :, a:b])
        _, S, z = oracle.rope_chunk_forward(-np.ones_like(Kc), Kc, Vc, S, z, EPS, f0 + a // hw,
                                            gh, gw, THETA)
        if b in (T, N):
            block_states.append((S.copy(), z.copy()))

    dSb = [np.zeros((1, 1, d, d)) for _ in range(2)]
    dzb = [np.zeros((1, 1, d)) for _ in range(2)]
    worst = 0.0
    for (a, b), n in zip(chunks, block_of):
        Qc, dOc = host(q[:, :, a:b]), host(do[:, :, a:b])
        dQc, _, _, dS0, dz0 = oracle.rope_blockcausal_backward(
            Qc, -np.ones_like(Qc), np.zeros_like(Qc), [0, b - a], dOc, EPS, f0 + a // hw, gh, gw,
            THETA, *block_states[n])
        dSb[n] += dS0
        dzb[n] += dz0
        e = normwise(host(dq[:, :, a:b]), dQc, axes=(2, 3))
        report(f"rope max-size backward dq tokens {a}..{b}", dq=e)
        worst = max(worst, e)
    G = [dSb[0] + dSb[1], dSb[1]]
    g = [dzb[0] + dzb[1], dzb[1]]
    for (a, b), n in [(chunks[1], block_of[1]), (chunks[-1], block_of[-1])]:
        Kc, Vc = host(k[:, :, a:b]), host(v[:, :, a:b])
        _, dKc, dVc, _, _ = oracle.rope_blockcausal_backward(
            -np.ones_like(Kc), Kc, Vc, [0, b - a], np.zeros_like(Kc), EPS, f0 + a // hw, gh, gw,
            THETA, *block_states[n], G[n][None], g[n][None])
        ek = normwise(host(dk[:, :, a:b]), dKc, axes=(2, 3))
        ev = normwise(host(dv[:, :, a:b]), dVc, axes=(2, 3))
        report(f"rope max-size backward dk/dv tokens {a}..{b}", dk=ek, dv=ev)
        worst = max(worst, ek, ev)
    assert worst <= TOL["bf16"], worst


def test_rope_backward_degenerate_rows():
    """A query row with no positive entry gets dq = 0 exactly; a key row with
    no positive entry gets dk = 0 and dv = 0 exactly (its rotated phi(k) is
    zero)."""
    B, H, N, T, d, gh, gw = 1, 2, 1000, 300, 64, 6, 10
    Q, K, V = workloads.random_qkv(141, B, H, N, d)
    Q[:, :, 17] = -np.abs(Q[:, :, 17])
    K[:, :, 450] = -np.abs(K[:, :, 450])
    dO = workloads.random_grads(142, B, H, N, d)
    dq, dk, dv, _ = gpu_backward(Q, K, V, dO, T, "bf16", 3, gh, gw)
    assert np.all(dq[:, :, 17] == 0.0)
    assert np.all(dk[:, :, 450] == 0.0) and np.all(dv[:, :, 450] == 0.0)
    ref = oracle.rope_blockcausal_backward(Q, K, V, bounds_of(N, T), dO, EPS, 3, gh, gw, THETA)
    check("rope backward degenerate rows", [dq, dk, dv], ref[:3], bounds_of(N, T), TOL["bf16"])


def test_rope_backward_zero_eps_ragged():
    """eps = 0 with every denominator kept > 0: the padding rows past a
    ragged tile and block (whose positions are still turned) stay out of
    every sum, so nothing turns into NaN."""
    B, H, N, T, d, gh, gw = 1, 2, 1000, 300, 64, 7, 9
    Q, K, V = workloads.random_qkv(143, B, H, N, d)
    Q[..., 0] = np.abs(Q[..., 0]) + 0.25
    K[..., 0] = np.abs(K[..., 0]) + 0.25
    Q, K = workloads.bf16_round(Q), workloads.bf16_round(K)
    dO = workloads.random_grads(144, B, H, N, d)
    q, k, v = dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16")
    _, states = la.blockcausal_forward_rope(q, k, v, T, 4, gh, gw, THETA, eps=0.0)
    dq, dk, dv, _ = la.blockcausal_backward_rope(q, k, v, states, dev(dO, "f32"), T, 4, gh, gw,
                                                 THETA, eps=0.0)
    torch.cuda.synchronize()
    got = [host(dq), host(dk), host(dv)]
    assert all(np.all(np.isfinite(x)) for x in got)
    ref = oracle.rope_blockcausal_backward(Q, K, V, bounds_of(N, T), dO, 0.0, 4, gh, gw, THETA)
    check("rope backward eps=0", got, ref[:3], bounds_of(N, T), TOL["bf16"])


# ---------------------------------------------------------------------------
# the chunk form: la_chunk_backward_rope


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_rope_chunk_backward(dtype, d):
    """One chunk against a carried state, with a gradient on state_out."""
    B, H, L, gh, gw, f0 = 2, 2, 1500, 6, 11, 9
    Q, K, V = workloads.random_qkv(151 + d, B, H, L, d, dtype=dtype)
    dO = workloads.random_grads(152 + d, B, H, L, d)
    S0, z0 = workloads.random_state(153 + d, B, H, d, tokens=5000)
    dS, dz = workloads.random_state_grads(154 + d, B, H, 1, d)
    q, k, v = dev(Q, dtype), dev(K, dtype), dev(V, dtype)
    _, st = la.chunk_forward_rope(q, k, v, torch.from_numpy(state_np(S0, z0)).cuda(), f0, gh, gw,
                                  THETA, eps=EPS)
    dso = torch.from_numpy(state_np(dS[0], dz[0])).cuda()
    dq, dk, dv, dsi = la.chunk_backward_rope(q, k, v, st, dev(dO, "f32"), f0, gh, gw, THETA,
                                             dstate_out=dso, eps=EPS)
    torch.cuda.synchronize()
    ref = oracle.rope_blockcausal_backward(Q, K, V, [0, L], dO, EPS, f0, gh, gw, THETA,
                                           S0.astype(np.float64), z0.astype(np.float64),
                                           dS.astype(np.float64), dz.astype(np.float64))
    check(f"rope chunk backward {dtype} d={d}", [host(dq), host(dk), host(dv)], ref[:3], [0, L],
          TOL[dtype], host(dsi), ref[3:])


def test_rope_chunk_backward_empty_passes_state_gradient():
    """L = 0: state_out = state_in, so dstate_in = dstate_out exactly."""
    B, H, d = 1, 3, 64
    S0, z0 = workloads.random_state(161, B, H, d)
    st = torch.from_numpy(state_np(S0, z0)).cuda()
    dS, dz = workloads.random_state_grads(162, B, H, 1, d)
    dso = torch.from_numpy(state_np(dS[0], dz[0])).cuda()
    e = torch.empty((B, H, 0, d), dtype=torch.bfloat16, device="cuda")
    _, _, _, dsi = la.chunk_backward_rope(e, e, e, st, e.float(), 5, 4, 4, THETA, dstate_out=dso,
                                          eps=EPS)
    torch.cuda.synchronize()
    assert torch.equal(dsi, dso)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rope_global_backward(dtype):
    """la_global_backward_rope against the oracle (one block, no state)."""
    B, H, N, d, gh, gw, f0 = 1, 3, 2000, 64, 5, 9, 2
    Q, K, V = workloads.random_qkv(171, B, H, N, d, dtype=dtype)
    dO = workloads.random_grads(172, B, H, N, d)
    q, k, v = dev(Q, dtype), dev(K, dtype), dev(V, dtype)
    _, st = la.global_forward_rope(q, k, v, f0, gh, gw, THETA, eps=EPS)
    dq, dk, dv = la.global_backward_rope(q, k, v, st, dev(dO, "f32"), f0, gh, gw, THETA, eps=EPS)
    torch.cuda.synchronize()
    ref = oracle.rope_blockcausal_backward(Q, K, V, [0, N], dO, EPS, f0, gh, gw, THETA)
    check(f"rope global backward {dtype}", [host(dq), host(dk), host(dv)], ref[:3], [0, N],
          TOL[dtype])
