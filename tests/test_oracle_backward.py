"""Pins of the oracle's gradients (``oracle.blockcausal_backward``) against
things other than its own formulas.

The gradients are the chain rule applied to the forward definition (the
pages train with the same block-causal attention, "SANA-Video: Efficient
Video Generation with Block Linear Diffusion Transformer", abstract, and
"Nvidia, MIT ve diğerleri video yapay zeka devrimini başlattı", section
"Sabit Bellekli KV önbelleğe alma mekanizması"; they print no gradient).
What pins them:

* central finite differences of the (separately pinned) fp64 forward,
  including the state input and the gradients of every block's state;
* torch fp64 autograd through the explicit T x T masked quadratic form, a
  different formulation of the same function;
* Euler's theorem: with eps = 0 and no state input the output is
  homogeneous of degree 0 in Q and in K and of degree 1 in V;
* with only state gradients, closed forms for dQ (zero), dS0, dz0 and the
  homogeneity sums.

``test_backward_mutants_caught`` plants plausible mistakes in the oracle's
gradient steps (on the CPU, by monkeypatching one step) and checks that
pins catch each.
"""

import numpy as np
import pytest

import oracle


def _f64_sign_away(g, shape, lo=0.3, hi=1.3):
    """Values with |x| in [lo, hi] and a random sign: far from the kink of
    max(x, 0), so finite differences never cross it."""
    mag = g.uniform(lo, hi, shape)
    return np.where(g.random(shape) < 0.5, -mag, mag)


def _case(seed, B=1, H=2, T=7, d=3, bounds=(0, 3, 5, 7), state=True, dstate=True):
    g = np.random.default_rng(seed)
    Q, K, V, dO = (_f64_sign_away(g, (B, H, T, d)) for _ in range(4))
    C = len(bounds) - 1
    S0 = z0 = dS = dz = None
    if state:
        S0 = g.standard_normal((B, H, d, d))
        z0 = g.uniform(0.5, 1.5, (B, H, d))
    if dstate:
        dS = g.standard_normal((C, B, H, d, d))
        dz = g.standard_normal((C, B, H, d))
    return Q, K, V, list(bounds), dO, S0, z0, dS, dz


def _loss(Q, K, V, bounds, dO, eps, S0, z0, dS, dz):
    blocks = [(Q[:, :, bounds[n]:bounds[n + 1]], K[:, :, bounds[n]:bounds[n + 1]],
               V[:, :, bounds[n]:bounds[n + 1]]) for n in range(len(bounds) - 1)]
    outs, states = oracle.stream_forward(blocks, eps, S0, z0)
    L = float(np.sum(np.concatenate(outs, axis=2) * dO))
    if dS is not None:
        for n, (S, z) in enumerate(states):
            L += float(np.sum(S * dS[n]) + np.sum(z * dz[n]))
    return L


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# --------------------------------------------------------------------------
# pins


def pin_finite_differences():
    """Every gradient entry against a central difference of the forward."""
    eps = 1e-3
    for seed in (0, 1):
        Q, K, V, bounds, dO, S0, z0, dS, dz = _case(seed)
        got = oracle.blockcausal_backward(Q, K, V, bounds, dO, eps, S0, z0, dS, dz)
        args = [Q, K, V, S0, z0]
        h = 1e-6
        for which, grad in zip(range(5), got):
            x = args[which]
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                keep = x[idx]
                x[idx] = keep + h
                lp = _loss(Q, K, V, bounds, dO, eps, S0, z0, dS, dz)
                x[idx] = keep - h
                lm = _loss(Q, K, V, bounds, dO, eps, S0, z0, dS, dz)
                x[idx] = keep
                fd[idx] = (lp - lm) / (2 * h)
            assert _rel(grad, fd) < 1e-7, (which, _rel(grad, fd))


def pin_autograd_quadratic():
    """dQ, dK, dV against torch fp64 autograd of the explicit masked T x T
    form o_i = sum_j W_ij v_j / (sum_j W_ij + eps), W_ij = phi(q_i).phi(k_j)
    [block(j) <= block(i)]."""
    import torch

    eps = 1e-6
    for seed, T, d, bounds in ((2, 9, 4, (0, 4, 9)), (3, 6, 5, (0, 1, 2, 3, 4, 5, 6)),
                               (4, 8, 3, (0, 8))):
        g = np.random.default_rng(seed)
        Q, K, V, dO = (g.standard_normal((1, 2, T, d)) for _ in range(4))
        bid = np.empty(T, dtype=np.int64)
        for n in range(len(bounds) - 1):
            bid[bounds[n]:bounds[n + 1]] = n
        mask = torch.tensor((bid[None, :] <= bid[:, None]).astype(np.float64))
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
        W = torch.relu(tq) @ torch.relu(tk).transpose(-1, -2) * mask
        O = (W @ tv) / (W.sum(-1, keepdim=True) + eps)
        (O * torch.tensor(dO)).sum().backward()
        dQ, dK, dV, _, _ = oracle.blockcausal_backward(Q, K, V, list(bounds), dO, eps)
        for got, ref in ((dQ, tq.grad), (dK, tk.grad), (dV, tv.grad)):
            assert _rel(got, ref.numpy()) < 1e-10, _rel(got, ref.numpy())


def pin_euler_homogeneity():
    """eps = 0, no state input: o(aQ) = o(Q), o(bK) = o(K), o(cV) = c o(V)
    for a, b, c > 0, so sum dQ*Q = 0, sum dK*K = 0, sum dV*V = sum dO*O."""
    for seed in (5, 6):
        g = np.random.default_rng(seed)
        Q, K, V, dO = (g.standard_normal((2, 2, 12, 4)) for _ in range(4))
        # one positive feature in every row keeps every denominator > 0
        Q[..., 0] = np.abs(Q[..., 0]) + 0.1
        K[..., 0] = np.abs(K[..., 0]) + 0.1
        bounds = [0, 5, 12]
        dQ, dK, dV, _, _ = oracle.blockcausal_backward(Q, K, V, bounds, dO, 0.0)
        O, _, _ = oracle.prefix_forward(Q, K, V, bounds, 0.0)
        scale = np.sum(np.abs(dO * O))
        assert abs(np.sum(dQ * Q)) < 1e-12 * scale
        assert abs(np.sum(dK * K)) < 1e-12 * scale
        assert abs(np.sum(dV * V) - np.sum(dO * O)) < 1e-12 * scale


def pin_state_only_gradients():
    """dO = 0 with gradients only on the block states: dQ = 0, dS0 = sum_n
    dS_n, dz0 = sum_n dz_n; the states are linear in V and in phi(K), so
    sum dV*V = sum_n dS_n.(S_n - S0) and
    sum dK*K = sum_n dS_n.(S_n - S0) + dz_n.(z_n - z0)."""
    Q, K, V, bounds, _, S0, z0, dS, dz = _case(7, B=2, H=1, T=10, d=4, bounds=(0, 2, 7, 10))
    dO = np.zeros_like(Q)
    dQ, dK, dV, dS0, dz0 = oracle.blockcausal_backward(Q, K, V, bounds, dO, 1e-6,
                                                       S0, z0, dS, dz)
    assert np.all(dQ == 0.0)
    assert _rel(dS0, dS.sum(axis=0)) < 1e-14
    assert _rel(dz0, dz.sum(axis=0)) < 1e-14
    _, S_pre, z_pre = oracle.prefix_forward(Q, K, V, bounds, 1e-6)
    sv = float(np.sum(dS * S_pre))
    sk = sv + float(np.sum(dz * z_pre))
    assert abs(np.sum(dV * V) - sv) < 1e-12 * np.sum(np.abs(dS * S_pre))
    assert abs(np.sum(dK * K) - sk) < 1e-12 * (np.sum(np.abs(dS * S_pre)) +
                                                np.sum(np.abs(dz * z_pre)))


def pin_zero_rows():
    """A query row with no positive entry has o = 0 and dq = 0; a key row
    with no positive entry contributes nothing, so its dk = 0 (phi'(x) = 0
    for x <= 0) while its dv = 0 as well (phi(k) = 0)."""
    g = np.random.default_rng(8)
    Q, K, V, dO = (g.standard_normal((1, 1, 8, 4)) for _ in range(4))
    Q[0, 0, 3] = -np.abs(Q[0, 0, 3])
    K[0, 0, 5] = -np.abs(K[0, 0, 5])
    dQ, dK, dV, _, _ = oracle.blockcausal_backward(Q, K, V, [0, 4, 8], dO, 1e-6)
    assert np.all(dQ[0, 0, 3] == 0.0)
    assert np.all(dK[0, 0, 5] == 0.0)
    assert np.all(dV[0, 0, 5] == 0.0)


PINS = [pin_finite_differences, pin_autograd_quadratic, pin_euler_homogeneity,
        pin_state_only_gradients, pin_zero_rows]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_backward_pin(pin):
    pin()


# --------------------------------------------------------------------------
# mutants: plausible mistakes in the gradient steps

_readout_backward = oracle.readout_backward
_kv_backward = oracle.kv_backward
_suffix_sums = oracle._suffix_sums


def _rb_parts(Q, S, z, dO, eps):
    fQ = oracle.phi(Q)
    den = fQ @ z[..., :, None] + eps
    O = fQ @ S / den
    return fQ, den, O


def _mut_no_dden(Q, S, z, dO, eps):
    fQ, den, O = _rb_parts(Q, S, z, dO, eps)
    dnum = dO / den
    dQ = np.where(Q > 0, dnum @ np.swapaxes(S, -1, -2), 0.0)
    return dQ, np.swapaxes(fQ, -1, -2) @ dnum, np.zeros_like(z)


def _mut_dden_sign(Q, S, z, dO, eps):
    dQ, dS, dz = _readout_backward(Q, S, z, dO, eps)
    fQ, den, O = _rb_parts(Q, S, z, dO, eps)
    dden = -np.sum(dO * O, axis=-1, keepdims=True) / den
    dQ = dQ - 2 * np.where(Q > 0, dden * z[..., None, :], 0.0)
    return dQ, dS, -dz


def _mut_dnum_unscaled(Q, S, z, dO, eps):
    fQ, den, O = _rb_parts(Q, S, z, dO, eps)
    dden = -np.sum(dO * O, axis=-1, keepdims=True) / den
    dQ = np.where(Q > 0, dO @ np.swapaxes(S, -1, -2) + dden * z[..., None, :], 0.0)
    fQt = np.swapaxes(fQ, -1, -2)
    return dQ, fQt @ dO, (fQt @ dden)[..., 0]


def _mut_dq_unmasked(Q, S, z, dO, eps):
    fQ, den, O = _rb_parts(Q, S, z, dO, eps)
    dnum = dO / den
    dden = -np.sum(dO * O, axis=-1, keepdims=True) / den
    dQ = dnum @ np.swapaxes(S, -1, -2) + dden * z[..., None, :]
    fQt = np.swapaxes(fQ, -1, -2)
    return dQ, fQt @ dnum, (fQt @ dden)[..., 0]


def _mut_kv_transposed(K, V, dKV, dk):
    return _kv_backward(K, V, np.swapaxes(dKV, -1, -2), dk)


def _mut_kv_no_dk(K, V, dKV, dk):
    return _kv_backward(K, V, dKV, np.zeros_like(dk))


def _mut_dv_transposed(K, V, dKV, dk):
    dK, _ = _kv_backward(K, V, dKV, dk)
    return dK, oracle.phi(K) @ np.swapaxes(dKV, -1, -2)


def _mut_prefix_not_suffix(xs):
    out, acc = [], None
    for x in xs:
        acc = x if acc is None else acc + x
        out.append(acc)
    return out


def _mut_own_block_only(xs):
    return list(xs)


MUTANTS = {
    "no_dden": ("readout_backward", _mut_no_dden),
    "dden_sign": ("readout_backward", _mut_dden_sign),
    "dnum_unscaled": ("readout_backward", _mut_dnum_unscaled),
    "dq_unmasked": ("readout_backward", _mut_dq_unmasked),
    "kv_transposed": ("kv_backward", _mut_kv_transposed),
    "kv_no_dk": ("kv_backward", _mut_kv_no_dk),
    "dv_transposed": ("kv_backward", _mut_dv_transposed),
    "prefix_not_suffix": ("_suffix_sums", _mut_prefix_not_suffix),
    "own_block_only": ("_suffix_sums", _mut_own_block_only),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_mutants_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(oracle, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
    print(f"[mutant] {name} caught by {caught}")
