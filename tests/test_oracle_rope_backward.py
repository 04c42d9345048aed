"""Pins of the oracle's RoPE'd gradients (``oracle.rope_blockcausal_backward``)
against things other than its own formulas: central finite differences of the
RoPE'd forward (``rope_prefix_forward``, itself pinned in test_oracle_rope.py),
torch float64 autograd through a separately written quadratic form with
explicit rotation matrices, the plain gradients where no pair turns, and the
invariance of dq, dk, dv to a shift of every position.
``test_rope_backward_mutants_caught`` plants plausible mistakes (by editing the
function's source) and checks that the pins catch each.
"""

import inspect
import textwrap

import numpy as np
import pytest
import torch

import oracle

THETA = 100.0  # small base: the frequencies of one group differ widely


def _case(seed, B=1, H=2, n=7, d=12, away=0.05):
    g = np.random.default_rng(seed)
    Q, K, V = (g.standard_normal((B, H, n, d)) for _ in range(3))
    # keep q and k away from the kink of max(x, 0)
    Q = np.sign(Q) * (np.abs(Q) + away)
    K = np.sign(K) * (np.abs(K) + away)
    return Q, K, V


def _loss_parts(seed, C, B, H, n, d):
    g = np.random.default_rng(seed)
    W = g.standard_normal((B, H, n, d))
    A = g.standard_normal((C, B, H, d, d)) * 0.1
    a = g.standard_normal((C, B, H, d)) * 0.1
    return W, A, a


def pin_finite_differences():
    """Every entry of dQ, dK, dV, dS0, dz0 against central differences of
    L = sum O*W + sum_n (S_n*A_n + z_n*a_n) (three blocks, ragged against a
    1 x 2 grid, non-zero S0 and z0)."""
    B, H, n, d = 1, 1, 7, 12
    Q, K, V = _case(1, B, H, n, d)
    bounds = [0, 3, 4, 7]
    C = len(bounds) - 1
    g = np.random.default_rng(2)
    S0, z0 = g.standard_normal((B, H, d, d)), g.uniform(0.5, 1.0, (B, H, d))
    W, A, a = _loss_parts(3, C, B, H, n, d)
    eps, f0, gh, gw = 0.1, 2, 1, 2

    def loss(Q, K, V, S0, z0):
        O, Sp, zp = oracle.rope_prefix_forward(Q, K, V, bounds, eps, f0, gh, gw, THETA, S0, z0)
        return float(np.sum(O * W) + np.sum(Sp * A) + np.sum(zp * a))

    got = oracle.rope_blockcausal_backward(Q, K, V, bounds, W, eps, f0, gh, gw, THETA, S0, z0,
                                           A, a)
    args = [Q, K, V, S0, z0]
    h = 1e-6
    for which, grad in enumerate(got):
        x = args[which]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = loss(*args)
            x[idx] = old - h
            lm = loss(*args)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        err = np.abs(num - grad).max() / max(np.abs(num).max(), 1e-30)
        assert err < 1e-7, (which, err)


def _torch_quadratic(Q, K, V, block_id, eps, pos, axis_of_pair, freqs):
    """O of the RoPE'd block-causal form as an explicit T x T computation with
    d x d rotation matrices (torch float64, differentiable)."""
    n, d = Q.shape[-2], Q.shape[-1]
    fq, fk = torch.relu(Q), torch.relu(K)
    rots = []
    for t in range(n):
        R = torch.zeros((d, d), dtype=torch.float64)
        for m in range(d // 2):
            ang = pos[t][axis_of_pair[m]] * freqs[m]
            c, s = np.cos(ang), np.sin(ang)
            R[2 * m, 2 * m], R[2 * m, 2 * m + 1] = c, -s
            R[2 * m + 1, 2 * m], R[2 * m + 1, 2 * m + 1] = s, c
        rots.append(R)
    R = torch.stack(rots)                                   # [n, d, d]
    rq = torch.einsum("tab,...tb->...ta", R, fq)
    rk = torch.einsum("tab,...tb->...ta", R, fk)
    bid = torch.tensor(block_id)
    mask = (bid[None, :] <= bid[:, None]).double()
    Wm = torch.matmul(rq, rk.transpose(-1, -2)) * mask
    Dm = torch.matmul(fq, fk.transpose(-1, -2)) * mask
    return torch.matmul(Wm, V) / (Dm.sum(-1, keepdim=True) + eps)


def pin_autograd_quadratic():
    """dQ, dK, dV equal torch autograd through the explicit quadratic form,
    whose positions and frequencies are written out here (grid walked in
    row-major order; a geometric sequence per group of 4, 4, 4 features)."""
    B, H, n, d = 1, 2, 9, 12
    Q, K, V = _case(4, B, H, n, d)
    bounds = [0, 4, 9]
    bid = [0] * 4 + [1] * 5
    f0, gh, gw, eps = 3, 2, 2, 1e-3
    pos = []
    f = f0
    while len(pos) < n:
        for r in range(gh):
            for c in range(gw):
                pos.append((f, r, c))
        f += 1
    pos = pos[:n]
    axis_of_pair = [0, 0, 1, 1, 2, 2]
    freqs = list(np.geomspace(1.0, THETA ** (-2.0 / 4.0), 2)) * 3
    dO = np.random.default_rng(5).standard_normal((B, H, n, d))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    O = _torch_quadratic(tq, tk, tv, bid, eps, pos, axis_of_pair, freqs)
    (O * torch.tensor(dO)).sum().backward()
    got = oracle.rope_blockcausal_backward(Q, K, V, bounds, dO, eps, f0, gh, gw, THETA)
    for ref, g in zip((tq.grad, tk.grad, tv.grad), got[:3]):
        ref = ref.numpy()
        assert np.abs(ref - g).max() / np.abs(ref).max() < 1e-10


def pin_still_pairs_reduce_to_plain():
    """One-token frames leave the row and column pairs still; with q and k
    supported on them, the gradients are the plain oracle's."""
    B, H, n, d = 1, 2, 8, 12
    Q, K, V = _case(6, B, H, n, d)
    dt = oracle.rope_axes(d)[0]
    Q[..., :dt] = -1.0
    K[..., :dt] = -1.0
    bounds = [0, 3, 8]
    dO = np.random.default_rng(7).standard_normal((B, H, n, d))
    got = oracle.rope_blockcausal_backward(Q, K, V, bounds, dO, 1e-3, 5, 1, 1, THETA)
    ref = oracle.blockcausal_backward(Q, K, V, bounds, dO, 1e-3)
    for r, g in zip(ref, got):
        assert np.allclose(r, g, rtol=1e-12, atol=1e-12)


def pin_shift_invariance():
    """With no state input, only position differences matter: dq, dk, dv do
    not change when every token moves by whole frames."""
    B, H, n, d = 1, 2, 10, 12
    Q, K, V = _case(8, B, H, n, d)
    bounds = [0, 4, 10]
    dO = np.random.default_rng(9).standard_normal((B, H, n, d))
    a = oracle.rope_blockcausal_backward(Q, K, V, bounds, dO, 1e-3, 0, 2, 2, THETA)
    b = oracle.rope_blockcausal_backward(Q, K, V, bounds, dO, 1e-3, 11, 2, 2, THETA)
    for x, y in zip(a[:3], b[:3]):
        assert np.abs(x - y).max() / np.abs(x).max() < 1e-12
    assert not np.allclose(a[3], b[3])  # the state gradient is not invariant


PINS = [pin_finite_differences, pin_autograd_quadratic, pin_still_pairs_reduce_to_plain,
        pin_shift_invariance]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_rope_backward_pin(pin):
    pin()


# ---------------------------------------------------------------------------
# Planted mistakes: each edits one line of the function's source.

MUTANTS = {
    "dq_not_turned_back": ("dfq = rope_rotate(drq, -ang[a:b])", "dfq = drq"),
    "dq_turned_forward": ("dfq = rope_rotate(drq, -ang[a:b])", "dfq = rope_rotate(drq, ang[a:b])"),
    "dS_from_unrotated_q": ("dSn = np.matmul(np.swapaxes(rQ[:, :, a:b], -1, -2), dnum)",
                            "dSn = np.matmul(np.swapaxes(fQ[:, :, a:b], -1, -2), dnum)"),
    "dz_from_rotated_q": ("dzn = np.matmul(np.swapaxes(fQ[:, :, a:b], -1, -2), dden)[..., 0]",
                          "dzn = np.matmul(np.swapaxes(rQ[:, :, a:b], -1, -2), dden)[..., 0]"),
    "dk_not_turned_back": ("dfk = rope_rotate(drk, -ang[a:b]) + Rz[c][..., None, :]",
                           "dfk = drk + Rz[c][..., None, :]"),
    "dv_from_unrotated_k": ("dV[:, :, a:b] = np.matmul(rK[:, :, a:b], RS[c])",
                            "dV[:, :, a:b] = np.matmul(fK[:, :, a:b], RS[c])"),
    "den_uses_rotated": ("den = np.matmul(fQ[:, :, a:b], z[..., :, None]) + float(eps)",
                         "den = np.matmul(rQ[:, :, a:b], z[..., :, None]) + float(eps)"),
}


def _mutant(old, new):
    src = textwrap.dedent(inspect.getsource(oracle.rope_blockcausal_backward))
    assert src.count(old) == 1, old
    ns = dict(vars(oracle))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns["rope_blockcausal_backward"]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_rope_backward_mutants_caught(name, monkeypatch):
    fn = _mutant(*MUTANTS[name])
    monkeypatch.setattr(oracle, "rope_blockcausal_backward", fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
    print(f"[mutant] {name} caught by {caught}")
