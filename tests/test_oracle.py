"""Pins of the fp64 oracle against things other than itself.

Each pin is a function that raises AssertionError when it fails; the
tests run every pin on the oracle as written, and ``test_mutants_caught``
plants plausible mistakes in the oracle (on the CPU, by monkeypatching one
step) and checks that at least one pin catches each.

Sources: "Nvidia, MIT ve diğerleri video yapay zeka devrimini başlattı",
section "Sabit Bellekli KV önbelleğe alma mekanizması" (block-causal rule,
KV1 -> KV1-2 -> global KV, token-order split is mathematically
equivalent); sd114.wiki article, section "1. 线性 DiT" (kernel mapping +
global aggregation without the N x N matrix).
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
EPS = workloads.EPS


def _split(x, bounds):
    return [x[:, :, bounds[i]:bounds[i + 1]] for i in range(len(bounds) - 1)]


def _stream(Q, K, V, bounds, eps):
    blocks = list(zip(_split(Q, bounds), _split(K, bounds), _split(V, bounds)))
    outs, states = oracle.stream_forward(blocks, eps)
    return np.concatenate(outs, axis=2), states


def _block_ids(bounds):
    ids = np.empty(bounds[-1], dtype=np.int64)
    for n in range(len(bounds) - 1):
        ids[bounds[n]:bounds[n + 1]] = n
    return ids


def _rand(seed, B, H, T, d, scale=1.0):
    g = np.random.default_rng(seed)
    return tuple(g.standard_normal((B, H, T, d)) * scale for _ in range(3))


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# --------------------------------------------------------------------------
# pins


def pin_worked_example():
    """Hand-derived four-token example (tests/golden/worked_d2.md)."""
    with open(os.path.join(GOLDEN, "worked_d2.json")) as f:
        g = json.load(f)
    Q, K, V = (np.array(g[n], dtype=np.float64)[None, None] for n in ("q", "k", "v"))
    eps = float(Fraction(g["eps"]))
    exact = np.array([[float(Fraction(x)) for x in row] for row in g["out"]])
    O, _ = _stream(Q, K, V, [0, 2, 4], eps)
    assert np.allclose(O[0, 0], exact, rtol=1e-15, atol=1e-15), (O[0, 0], exact)


def pin_exact_rational():
    """Exact quadratic-form solutions of random small-integer cases."""
    with open(os.path.join(GOLDEN, "exact_random.json")) as f:
        cases = json.load(f)
    for c in cases:
        Q, K, V = (np.array(c[n], dtype=np.float64)[None, None] for n in ("q", "k", "v"))
        ids = c["blocks"]
        bounds = [0] + [t for t in range(1, len(ids)) if ids[t] != ids[t - 1]] + [len(ids)]
        O, _ = _stream(Q, K, V, bounds, float(Fraction(c["eps"])))
        exact = np.array([[float(Fraction(x)) for x in row] for row in c["out"]])
        err = np.max(np.abs(O[0, 0] - exact) / (np.abs(exact) + 1e-300 + (exact == 0)))
        assert err < 1e-13, (err, c)


def pin_quadratic_form():
    """Linear form == explicit masked pairwise weights, random floats."""
    Q, K, V = _rand(1, 2, 3, 24, 8)
    bounds = [0, 5, 6, 17, 24]
    O, _ = _stream(Q, K, V, bounds, EPS)
    R = oracle.quadratic_forward(Q, K, V, _block_ids(bounds), EPS)
    assert _rel(O, R) < 1e-12, _rel(O, R)


def pin_constant_value_closed_form():
    """phi(q) = phi(k) = 1 and v_j = c for all j: every query of block n
    sees D = d * (tokens in blocks 0..n) and returns c * D / (D + eps)."""
    B, H, d, L, C = 1, 2, 4, 3, 3
    T = L * C
    Q = np.ones((B, H, T, d))
    K = np.ones((B, H, T, d))
    c = np.array([1.5, -2.0, 0.25, 3.0])
    V = np.broadcast_to(c, (B, H, T, d)).copy()
    eps = 2.0
    O, _ = _stream(Q, K, V, [0, 3, 6, 9], eps)
    for n in range(C):
        D = d * L * (n + 1)
        want = c * D / (D + eps)
        assert np.allclose(O[:, :, n * L:(n + 1) * L], want, rtol=1e-14), (n, O[0, 0, n * L], want)


def pin_identity_values_give_weights():
    """V = I (T = d): row i of the output is the normalised kernel-weight
    row, computed here by explicit loops."""
    g = np.random.default_rng(5)
    T = d = 6
    q = g.standard_normal((T, d))
    k = g.standard_normal((T, d))
    ids = [0, 0, 1, 1, 1, 2]
    eps = 0.5
    O, _ = _stream(q[None, None], k[None, None], np.eye(d)[None, None], [0, 2, 5, 6], eps)
    for i in range(T):
        w = []
        for j in range(T):
            s = 0.0
            if ids[j] <= ids[i]:
                for a in range(d):
                    s += max(q[i, a], 0.0) * max(k[j, a], 0.0)
            w.append(s)
        tot = sum(w) + eps
        assert np.allclose(O[0, 0, i], [x / tot for x in w], rtol=1e-13, atol=1e-15), i


def pin_token_causal_recurrence():
    """One token per block reduces to the token-causal linear-attention
    recurrence S_t = S_{t-1} + phi(k_t) v_t^T, written here as a loop."""
    Q, K, V = _rand(3, 1, 2, 10, 3)
    T = 10
    O, _ = _stream(Q, K, V, list(range(T + 1)), EPS)
    for b in range(1):
        for h in range(2):
            S = np.zeros((3, 3))
            z = np.zeros(3)
            for t in range(T):
                fk = np.maximum(K[b, h, t], 0)
                fq = np.maximum(Q[b, h, t], 0)
                S = S + np.outer(fk, V[b, h, t])
                z = z + fk
                want = fq @ S / (fq @ z + EPS)
                assert np.allclose(O[b, h, t], want, rtol=1e-12, atol=1e-14)


def pin_block_rules():
    """One block == global; the first block == global over itself; the last
    block's rows == global rows (it sees everything)."""
    Q, K, V = _rand(7, 1, 2, 20, 5)
    bounds = [0, 7, 13, 20]
    O, _ = _stream(Q, K, V, bounds, EPS)
    G, _, _ = oracle.global_forward(Q, K, V, EPS)
    O1, _ = _stream(Q, K, V, [0, 20], EPS)
    assert _rel(O1, G) < 1e-14
    G0, _, _ = oracle.global_forward(Q[:, :, :7], K[:, :, :7], V[:, :, :7], EPS)
    assert _rel(O[:, :, :7], G0) < 1e-13
    assert _rel(O[:, :, 13:], G[:, :, 13:]) < 1e-13
    # the middle block differs from the global result (it must not see the last block)
    assert _rel(O[:, :, 7:13], G[:, :, 7:13]) > 1e-3


def pin_state_prefix_sum():
    """State after block n == KV1 + ... + KVn, each KV summed here token by
    token; the final state is the same for every chunking."""
    Q, K, V = _rand(11, 1, 1, 15, 3)
    bounds = [0, 4, 9, 15]
    _, states = _stream(Q, K, V, bounds, EPS)
    S = np.zeros((3, 3))
    z = np.zeros(3)
    for n in range(3):
        for t in range(bounds[n], bounds[n + 1]):
            fk = np.maximum(K[0, 0, t], 0)
            S = S + np.outer(fk, V[0, 0, t])
            z = z + fk
        assert np.allclose(states[n][0][0, 0], S, rtol=1e-13, atol=1e-13)
        assert np.allclose(states[n][1][0, 0], z, rtol=1e-13, atol=1e-13)
    for other in ([0, 15], [0, 1, 2, 3, 15], [0, 14, 15]):
        _, st = _stream(Q, K, V, other, EPS)
        assert np.allclose(st[-1][0], states[-1][0], rtol=1e-13, atol=1e-13)
        assert np.allclose(st[-1][1], states[-1][1], rtol=1e-13, atol=1e-13)


def pin_invariants():
    """Linearity in V (phi must not touch V); invariance to permuting tokens
    inside a block (keys with their values); zero query rows give zero."""
    Q, K, V1 = _rand(13, 1, 2, 12, 4)
    V2 = np.random.default_rng(14).standard_normal(V1.shape)
    bounds = [0, 5, 12]
    a, b = -1.75, 0.5
    O1, _ = _stream(Q, K, V1, bounds, EPS)
    O2, _ = _stream(Q, K, V2, bounds, EPS)
    O12, _ = _stream(Q, K, a * V1 + b * V2, bounds, EPS)
    assert _rel(O12, a * O1 + b * O2) < 1e-12
    perm = np.concatenate([np.random.default_rng(2).permutation(5), 5 + np.arange(7)[::-1]])
    Op, _ = _stream(Q, K[:, :, perm], V1[:, :, perm], bounds, EPS)
    assert _rel(Op, O1) < 1e-12
    Qz = Q.copy()
    Qz[:, :, 3] = -np.abs(Qz[:, :, 3])
    Oz, _ = _stream(Qz, K, V1, bounds, EPS)
    assert np.all(Oz[:, :, 3] == 0.0)


def pin_stream_equals_prefix_route():
    """Carried state == all-block KV, prefix sum, then readout."""
    Q, K, V = _rand(17, 2, 2, 30, 6)
    bounds = [0, 8, 16, 23, 30]
    O, states = _stream(Q, K, V, bounds, EPS)
    P, S_pre, z_pre = oracle.prefix_forward(Q, K, V, bounds, EPS)
    assert _rel(O, P) < 1e-13
    for n in range(4):
        assert _rel(states[n][0], S_pre[n]) < 1e-13


PINS = [
    pin_worked_example,
    pin_exact_rational,
    pin_quadratic_form,
    pin_constant_value_closed_form,
    pin_identity_values_give_weights,
    pin_token_causal_recurrence,
    pin_block_rules,
    pin_state_prefix_sum,
    pin_invariants,
    pin_stream_equals_prefix_route,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# --------------------------------------------------------------------------
# planted mistakes: each must fail at least one pin


def _mut_transpose_kv(K, V):
    KV, k = _orig["kv_of_block"](K, V)
    return np.swapaxes(KV, -1, -2), k


def _mut_phi_on_values(K, V):
    return _orig["kv_of_block"](K, oracle.phi(V))


def _mut_no_eps(Q, S, z, eps):
    return _orig["readout"](Q, S, z, 0.0)


def _mut_eps_outside(Q, S, z, eps):
    fQ = oracle.phi(Q)
    return np.matmul(fQ, S) / np.maximum(np.matmul(fQ, z[..., :, None]), eps)


def _mut_no_carry(Q, K, V, S_in, z_in, eps):
    return _orig["chunk_forward"](Q, K, V, np.zeros_like(S_in), np.zeros_like(z_in), eps)


def _mut_reads_old_state(Q, K, V, S_in, z_in, eps):
    O, S, z = _orig["chunk_forward"](Q, K, V, S_in, z_in, eps)
    if np.any(S_in):
        O = _orig["readout"](Q, S_in, z_in, eps)
    return O, S, z


def _mut_phi_identity(x):
    return np.asarray(x, dtype=np.float64)


def _mut_phi_abs(x):
    return np.abs(np.asarray(x, dtype=np.float64))


def _mut_den_unphi(Q, S, z, eps):
    num = np.matmul(oracle.phi(Q), S)
    return num / (np.matmul(np.asarray(Q, np.float64), z[..., :, None]) + eps)


def _mut_z_from_values(K, V):
    KV, _ = _orig["kv_of_block"](K, V)
    return KV, oracle.phi(V).sum(axis=-2)


_orig = {n: getattr(oracle, n) for n in ("kv_of_block", "readout", "chunk_forward", "phi")}

MUTANTS = {
    "transpose_kv": ("kv_of_block", _mut_transpose_kv),
    "phi_on_values": ("kv_of_block", _mut_phi_on_values),
    "z_from_values": ("kv_of_block", _mut_z_from_values),
    "no_eps": ("readout", _mut_no_eps),
    "eps_as_floor": ("readout", _mut_eps_outside),
    "den_without_phi": ("readout", _mut_den_unphi),
    "no_state_carry": ("chunk_forward", _mut_no_carry),
    "excludes_own_block": ("chunk_forward", _mut_reads_old_state),
    "phi_identity": ("phi", _mut_phi_identity),
    "phi_abs": ("phi", _mut_phi_abs),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(oracle, attr, fn)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, FloatingPointError, ZeroDivisionError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name} passed every pin"


# --------------------------------------------------------------------------
# recovery by replay and save/restore of the state (the state is the whole
# checkpoint of a stream: it is a prefix sum of block KVs)


def test_state_checkpoint_and_replay():
    Q, K, V = _rand(21, 1, 2, 40, 4)
    bounds = [0, 10, 20, 30, 40]
    blocks = list(zip(_split(Q, bounds), _split(K, bounds), _split(V, bounds)))
    outs, states = oracle.stream_forward(blocks, EPS)
    # restore after block 1 and continue
    S, z = (x.copy() for x in states[1])
    outs2, _ = oracle.stream_forward(blocks[2:], EPS, S0=S, z0=z)
    for a, b in zip(outs2, outs[2:]):
        assert _rel(a, b) < 1e-15
    # lost state: replay blocks 0..2 from zero, then continue
    _, st = oracle.stream_forward(blocks[:3], EPS)
    outs3, _ = oracle.stream_forward(blocks[3:], EPS, S0=st[-1][0], z0=st[-1][1])
    assert _rel(outs3[0], outs[3]) < 1e-12


def test_nonfinite_inputs_propagate():
    """A NaN value reaches every output that gives its token weight."""
    Q, K, V = _rand(23, 1, 1, 6, 2)
    Q = np.abs(Q)
    K = np.abs(K)
    V[0, 0, 1, 0] = np.nan
    O, _ = _stream(Q, K, V, [0, 3, 6], EPS)
    assert np.all(np.isnan(O[0, 0, :, 0]))
    assert np.all(np.isfinite(O[0, 0, :, 1]))


def test_generator_properties():
    w = workloads.WORKLOADS[5]
    small = workloads.Workload(5, "t", "chunk", 2, 3, 8, 500, 1, "bf16",
                               outlier_frac=0.01, outlier_scale=8.0)
    Q, K, V = workloads.chunk_qkv(small, 0)
    Q2, _, _ = workloads.chunk_qkv(small, 0)
    assert np.array_equal(Q, Q2)
    # bf16-representable
    for x in (Q, K, V):
        assert np.all((x.view(np.uint32) & 0xFFFF) == 0)
    assert w.tokens == 163840
    assert workloads.WORKLOADS[3].L == 75600 and workloads.WORKLOADS[2].L == 32760
