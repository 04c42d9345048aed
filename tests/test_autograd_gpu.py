"""linear_attention (the autograd glue over the forward and backward calls):
its gradients equal the direct backward call's bit for bit, and the fp64
oracle's chain rule (``oracle.blockcausal_backward``) within the backward
bounds, for the global and the block-causal form, with and without a state
input, and with a loss that also reads the returned states; the same for the
rotary form against ``oracle.rope_blockcausal_backward``; and two chained calls
(the second reading the first's state) against the two-block sequence."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import TOL, dev, host, state_np

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


def _err(got, ref):
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-300))


@pytest.mark.parametrize("T,with_state", [(None, False), (None, True), (100, True), (37, False)])
def test_autograd_matches_oracle(T, with_state):
    B, H, N, d = 1, 2, 300, 64
    Q, K, V = workloads.random_qkv(501 + N, B, H, N, d, dtype="f32")
    dO = workloads.random_grads(502, B, H, N, d)
    q, k, v = (dev(x, "f32").requires_grad_() for x in (Q, K, V))
    S0 = z0 = st = None
    if with_state:
        S0, z0 = workloads.random_state(503, B, H, d)
        S0, z0 = S0.astype(np.float64), z0.astype(np.float64)
        st = torch.from_numpy(state_np(S0, z0)).cuda().requires_grad_()
    out, states = la.linear_attention(q, k, v, T=T, state_in=st, eps=EPS)
    # the loss reads the output and the last state
    w = torch.from_numpy(np.random.default_rng(7).standard_normal(states.shape[-1]) * 1e-3).float().cuda()
    loss = (out * dev(dO, "f32")).sum() + (states[:, :, -1] * w).sum()
    loss.backward()
    torch.cuda.synchronize()

    Tb = N if T is None else T
    bounds = list(range(0, N, Tb)) + [N]
    C = len(bounds) - 1
    E = d * d + d
    dS = np.zeros((C, B, H, d, d))
    dz = np.zeros((C, B, H, d))
    wn = host(w)
    dS[-1] = np.broadcast_to(wn[: d * d].reshape(d, d), (B, H, d, d))
    dz[-1] = np.broadcast_to(wn[d * d:], (B, H, d))
    dQ, dK, dV, dS0, dz0 = oracle.blockcausal_backward(Q, K, V, bounds, dO, EPS, S0, z0, dS, dz)
    errs = [_err(host(q.grad), dQ), _err(host(k.grad), dK), _err(host(v.grad), dV)]
    if with_state:
        g = host(st.grad)
        errs += [_err(g[..., : d * d].reshape(dS0.shape), dS0), _err(g[..., d * d:], dz0)]
    print(f"[parity] autograd T={T} state={with_state} " + " ".join(f"{e:.2e}" for e in errs),
          flush=True)
    assert max(errs) <= TOL["f32"], errs
    assert states.shape == (B, H, C, E)


def test_autograd_equals_direct_backward_bf16():
    B, H, N, d, T = 1, 4, 2000, 64, 500
    Q, K, V = workloads.random_qkv(511, B, H, N, d)
    dO = dev(workloads.random_grads(512, B, H, N, d), "f32")
    q, k, v = (dev(x, "bf16").requires_grad_() for x in (Q, K, V))
    out, states = la.linear_attention(q, k, v, T=T, eps=EPS)
    (out * dO).sum().backward()
    qd, kd, vd = (dev(x, "bf16") for x in (Q, K, V))
    _, st2 = la.blockcausal_forward(qd, kd, vd, T, eps=EPS)
    dq, dk, dv, _ = la.blockcausal_backward(qd, kd, vd, st2, dO, T, eps=EPS)
    torch.cuda.synchronize()
    assert q.grad.dtype == torch.bfloat16
    assert torch.equal(q.grad, dq.to(torch.bfloat16))
    assert torch.equal(k.grad, dk.to(torch.bfloat16))
    assert torch.equal(v.grad, dv.to(torch.bfloat16))


@pytest.mark.parametrize("T,with_state", [(None, False), (100, True)])
def test_autograd_rope_matches_oracle(T, with_state):
    """The rotary form through linear_attention(rope=...) against the oracle's
    rotary chain rule (``oracle.rope_blockcausal_backward``)."""
    B, H, N, d, f0, gh, gw = 1, 2, 300, 64, 3, 4, 6
    Q, K, V = workloads.random_qkv(521 + N, B, H, N, d, dtype="f32")
    dO = workloads.random_grads(522, B, H, N, d)
    q, k, v = (dev(x, "f32").requires_grad_() for x in (Q, K, V))
    S0 = z0 = st = None
    if with_state:
        S0, z0 = workloads.random_state(523, B, H, d)
        S0, z0 = S0.astype(np.float64), z0.astype(np.float64)
        st = torch.from_numpy(state_np(S0, z0)).cuda().requires_grad_()
    out, states = la.linear_attention(q, k, v, T=T, state_in=st, eps=EPS, rope=(f0, gh, gw))
    w = torch.from_numpy(np.random.default_rng(8).standard_normal(states.shape[-1]) * 1e-3).float().cuda()
    loss = (out * dev(dO, "f32")).sum() + (states[:, :, -1] * w).sum()
    loss.backward()
    torch.cuda.synchronize()

    Tb = N if T is None else T
    bounds = list(range(0, N, Tb)) + [N]
    C = len(bounds) - 1
    dS = np.zeros((C, B, H, d, d))
    dz = np.zeros((C, B, H, d))
    wn = host(w)
    dS[-1] = np.broadcast_to(wn[: d * d].reshape(d, d), (B, H, d, d))
    dz[-1] = np.broadcast_to(wn[d * d:], (B, H, d))
    dQ, dK, dV, dS0, dz0 = oracle.rope_blockcausal_backward(
        Q, K, V, bounds, dO, EPS, f0, gh, gw, workloads.ROPE_THETA, S0, z0, dS, dz)
    errs = [_err(host(q.grad), dQ), _err(host(k.grad), dK), _err(host(v.grad), dV)]
    if with_state:
        g = host(st.grad)
        errs += [_err(g[..., : d * d].reshape(dS0.shape), dS0), _err(g[..., d * d:], dz0)]
    print(f"[parity] autograd rope T={T} state={with_state} "
          + " ".join(f"{e:.2e}" for e in errs), flush=True)
    assert max(errs) <= TOL["f32"], errs


def test_autograd_rope_equals_direct_backward_bf16():
    B, H, N, d, T = 1, 4, 2000, 128, 500
    rope = (2, 5, 8, 2000.0)
    Q, K, V = workloads.random_qkv(531, B, H, N, d)
    dO = dev(workloads.random_grads(532, B, H, N, d), "f32")
    q, k, v = (dev(x, "bf16").requires_grad_() for x in (Q, K, V))
    out, states = la.linear_attention(q, k, v, T=T, eps=EPS, rope=rope)
    (out * dO).sum().backward()
    qd, kd, vd = (dev(x, "bf16") for x in (Q, K, V))
    _, st2 = la.blockcausal_forward_rope(qd, kd, vd, T, *rope, eps=EPS)
    dq, dk, dv, _ = la.blockcausal_backward_rope(qd, kd, vd, st2, dO, T, *rope, eps=EPS)
    torch.cuda.synchronize()
    assert torch.equal(q.grad, dq.to(torch.bfloat16))
    assert torch.equal(k.grad, dk.to(torch.bfloat16))
    assert torch.equal(v.grad, dv.to(torch.bfloat16))


@pytest.mark.parametrize("rope", [False, True])
def test_autograd_chained_calls_equal_one_sequence(rope):
    """Streaming training: two calls, the second reading the state the first
    returned, and one loss over both outputs.  Gradients reach the first
    call's q, k, v through the carried state and equal the oracle's on the
    two-block sequence."""
    B, H, L, d, gh, gw = 1, 2, 400, 64, 4, 10
    Q, K, V = workloads.random_qkv(541, B, H, 2 * L, d, dtype="f32")
    dO = workloads.random_grads(542, B, H, 2 * L, d)
    f1 = L // (gh * gw)  # the second chunk starts at frame 10
    q1, k1, v1 = (dev(x[:, :, :L], "f32").requires_grad_() for x in (Q, K, V))
    q2, k2, v2 = (dev(x[:, :, L:], "f32").requires_grad_() for x in (Q, K, V))
    r1 = (0, gh, gw) if rope else None
    r2 = (f1, gh, gw) if rope else None
    o1, s1 = la.linear_attention(q1, k1, v1, eps=EPS, rope=r1)
    o2, _ = la.linear_attention(q2, k2, v2, state_in=s1[:, :, -1], eps=EPS, rope=r2)
    loss = (o1 * dev(dO[:, :, :L], "f32")).sum() + (o2 * dev(dO[:, :, L:], "f32")).sum()
    loss.backward()
    torch.cuda.synchronize()
    if rope:
        ref = oracle.rope_blockcausal_backward(Q, K, V, [0, L, 2 * L], dO, EPS, 0, gh, gw,
                                               workloads.ROPE_THETA)
    else:
        ref = oracle.blockcausal_backward(Q, K, V, [0, L, 2 * L], dO, EPS)
    errs = []
    for (a, b), grads in (((0, L), (q1, k1, v1)), ((L, 2 * L), (q2, k2, v2))):
        for g, r in zip(grads, ref[:3]):
            errs.append(_err(host(g.grad), r[:, :, a:b]))
    print(f"[parity] autograd chained rope={rope} " + " ".join(f"{e:.2e}" for e in errs),
          flush=True)
    assert max(errs) <= TOL["f32"], errs
