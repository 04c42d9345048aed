"""Pins of the oracle's rotary-position linear attention (``oracle.rope_*``)
against things other than its own formulas: closed forms with every
frequency 1, one-dimensional RoPE written with complex exponentials and a
geometric frequency sequence, the explicit quadratic form, invariance to a
shift of every position, norm preservation, the plain (unrotated) oracle
where the rotation is the identity, and the carried state against the
prefix route.  ``test_rope_mutants_caught`` plants plausible mistakes and
checks that the pins catch each one.

The reading pinned (RoPE is named on the pages, [ZH] sd114.wiki section
"1. 线性 DiT", with no placement): 3-D positions (frame, row, column) on
interleaved feature pairs, groups d_t, d_h = d_w = 2 floor(d/6), rotation on
phi(q), phi(k) in the numerator only (RoFormer, section 3.4.3).
"""

import numpy as np
import pytest

import oracle


def _grid_positions(n, frame0, gh, gw):
    """(frame, row, column) of the first n tokens, by walking the grid in
    row-major order (no integer division)."""
    out = []
    f = frame0
    while len(out) < n:
        for r in range(gh):
            for c in range(gw):
                out.append((f, r, c))
        f += 1
    return out[:n]


def _pair_axis(d):
    """Axis (0 frame, 1 row, 2 column) of each feature pair, from the group
    sizes of the reading written out per d."""
    groups = {32: (12, 10, 10), 64: (24, 20, 20), 128: (44, 42, 42)}[d]
    axis = []
    for a, g in enumerate(groups):
        axis += [a] * (g // 2)
    return axis


def pin_axis_split():
    for d in (32, 64, 128):
        dt, dh, dw = oracle.rope_axes(d)
        assert (dt + dh + dw, dt % 2, dh % 2, dw % 2) == (d, 0, 0, 0)
        assert len(_pair_axis(d)) == d // 2
        assert [dt, dh, dw] == [2 * _pair_axis(d).count(a) for a in range(3)]


def pin_theta_one_closed_form():
    """theta = 1 sets every frequency to 1, so pair m turns by the token's
    position on its axis.  With q_i = a_i e_{2m} and k_j = b_j e_{2m} +
    c_j e_{2m+1} (all positive), one block:
      o_i = sum_j a_i (b_j cos D_ij + c_j sin(-D_ij)) v_j / (sum_j a_i b_j + eps)
    with D_ij = p_j - p_i on pair m's axis."""
    g = np.random.default_rng(11)
    d, n, frame0, gh, gw, eps = 32, 14, 2, 2, 3, 1e-3
    pos = _grid_positions(n, frame0, gh, gw)
    axis = _pair_axis(d)
    for m in range(d // 2):
        a = g.uniform(0.5, 1.5, n)
        b = g.uniform(0.5, 1.5, n)
        c = g.uniform(0.5, 1.5, n)
        V = g.standard_normal((1, 1, n, d))
        Q = np.zeros((1, 1, n, d))
        K = np.zeros((1, 1, n, d))
        Q[0, 0, :, 2 * m] = a
        K[0, 0, :, 2 * m] = b
        K[0, 0, :, 2 * m + 1] = c
        S0, z0 = oracle.zero_state(1, 1, d)
        O, _, _ = oracle.rope_chunk_forward(Q, K, V, S0, z0, eps, frame0, gh, gw, 1.0)
        p = np.array([t[axis[m]] for t in pos], dtype=np.float64)
        D = p[None, :] - p[:, None]
        W = a[:, None] * (b[None, :] * np.cos(D) - c[None, :] * np.sin(D))
        den = a * b.sum() + eps
        ref = (W @ V[0, 0]) / den[:, None]
        assert np.allclose(O[0, 0], ref, rtol=1e-12, atol=1e-12), m


def pin_one_dimensional_rope():
    """A grid one token wide and high leaves the row and column pairs still
    and turns the frame pairs as 1-D RoPE does: feature pair m as the
    complex number x + iy times exp(i p w_m), w_m the geometric sequence
    from 1 down to theta^(-(d_t - 2)/d_t) over the d_t/2 frame pairs.  A
    one-frame grid of one row (or one column) does the same for the column
    (or row) pairs."""
    g = np.random.default_rng(12)
    for d in (32, 64, 128):
        dt, dh, dw = oracle.rope_axes(d)
        n, theta = 9, 10000.0
        X = g.standard_normal((n, d))
        z = X[:, 0::2] + 1j * X[:, 1::2]
        for gh, gw, a0, size in ((1, 1, 0, dt), (n, 1, dt // 2, dh), (1, n, (dt + dh) // 2, dw)):
            frame0 = 5 if (gh, gw) == (1, 1) else 0
            p = np.arange(n) + frame0 if (gh, gw) == (1, 1) else np.arange(n)
            w = np.geomspace(1.0, theta ** (-(size - 2) / size), size // 2)
            ref = z.copy()
            ref[:, a0:a0 + size // 2] *= np.exp(1j * p[:, None] * w[None, :])
            R = oracle.rope_rotate(X, oracle.rope_angles(n, d, frame0, gh, gw, theta))
            got = R[:, 0::2] + 1j * R[:, 1::2]
            assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), (d, gh, gw)


def pin_norm_preserved():
    g = np.random.default_rng(13)
    X = g.standard_normal((2, 3, 40, 64))
    R = oracle.rope_rotate(X, oracle.rope_angles(40, 64, 3, 4, 5, 10000.0))
    assert np.allclose(np.linalg.norm(R, axis=-1), np.linalg.norm(X, axis=-1), rtol=1e-13)
    assert not np.allclose(R, X)


def pin_linear_equals_quadratic():
    """The prefix route equals the explicit quadratic form (blocks of 7, 5
    and 8 tokens, ragged against the 2 x 3 frame grid)."""
    g = np.random.default_rng(14)
    Q, K, V = (g.standard_normal((2, 2, 20, 32)) for _ in range(3))
    bounds = [0, 7, 12, 20]
    bid = np.repeat(np.arange(3), np.diff(bounds))
    O, _, _ = oracle.rope_prefix_forward(Q, K, V, bounds, 1e-6, 3, 2, 3, 10000.0)
    R = oracle.rope_quadratic_forward(Q, K, V, bid, 1e-6, 3, 2, 3, 10000.0)
    assert np.max(np.abs(O - R)) / np.max(np.abs(R)) < 1e-12


def pin_shift_invariance():
    """Only position differences enter the product of a rotated query and
    key, so moving every token by whole frames changes no output (the states
    do change)."""
    g = np.random.default_rng(15)
    Q, K, V = (g.standard_normal((1, 2, 24, 64)) for _ in range(3))
    bounds = [0, 12, 24]
    O0, S0, _ = oracle.rope_prefix_forward(Q, K, V, bounds, 1e-6, 0, 3, 4, 10000.0)
    O1, S1, _ = oracle.rope_prefix_forward(Q, K, V, bounds, 1e-6, 9, 3, 4, 10000.0)
    assert np.max(np.abs(O0 - O1)) / np.max(np.abs(O0)) < 1e-12
    assert not np.allclose(S0, S1)


def pin_still_pairs_reduce_to_plain():
    """With one-token frames the row and column pairs never turn; queries and
    keys supported on them give the plain (unrotated) oracle's result."""
    g = np.random.default_rng(16)
    d = 64
    dt = oracle.rope_axes(d)[0]
    Q, K, V = (g.standard_normal((1, 2, 10, d)) for _ in range(3))
    Q[..., :dt] = 0.0
    K[..., :dt] = 0.0
    S0, z0 = oracle.zero_state(1, 2, d)
    S0 = g.standard_normal(S0.shape)
    S0[..., :dt, :] = 0.0
    z0 = g.uniform(1.0, 2.0, z0.shape)
    O, S, z = oracle.rope_chunk_forward(Q, K, V, S0, z0, 1e-6, 4, 1, 1, 10000.0)
    Op, Sp, zp = oracle.chunk_forward(Q, K, V, S0, z0, 1e-6)
    assert np.allclose(O, Op, rtol=1e-12, atol=1e-12)
    assert np.allclose(S, Sp, rtol=1e-12, atol=1e-12) and np.allclose(z, zp, rtol=1e-12)


def pin_stream_equals_prefix():
    """Block calls with the state carried and frame0 advanced by the frames
    of each block equal the whole-sequence prefix route (blocks of whole
    frames: 2 frames of 2 x 3 tokens each), with a non-zero S0, z0."""
    g = np.random.default_rng(17)
    Q, K, V = (g.standard_normal((2, 1, 36, 32)) for _ in range(3))
    S, z = g.standard_normal((2, 1, 32, 32)), g.uniform(1.0, 2.0, (2, 1, 32))
    bounds = [0, 12, 24, 36]
    O_ref, S_pre, z_pre = oracle.rope_prefix_forward(Q, K, V, bounds, 1e-6, 5, 2, 3, 10000.0,
                                                     S, z)
    for c in range(3):
        a, b = bounds[c], bounds[c + 1]
        O, S, z = oracle.rope_chunk_forward(Q[:, :, a:b], K[:, :, a:b], V[:, :, a:b], S, z, 1e-6,
                                            5 + 2 * c, 2, 3, 10000.0)
        assert np.max(np.abs(O - O_ref[:, :, a:b])) / np.max(np.abs(O_ref)) < 1e-12
        assert np.allclose(S, S_pre[c], rtol=1e-12, atol=1e-12)
        assert np.allclose(z, z_pre[c], rtol=1e-12, atol=1e-12)


PINS = [pin_axis_split, pin_theta_one_closed_form, pin_one_dimensional_rope, pin_norm_preserved,
        pin_linear_equals_quadratic, pin_shift_invariance, pin_still_pairs_reduce_to_plain,
        pin_stream_equals_prefix]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_rope_pin(pin):
    pin()


# ---------------------------------------------------------------------------
# Planted mistakes: each replaces one oracle function with a plausible wrong
# version; at least one pin must fail.

_axes, _angles, _rotate = oracle.rope_axes, oracle.rope_angles, oracle.rope_rotate
_chunk, _prefix = oracle.rope_chunk_forward, oracle.rope_prefix_forward


def _mut_rotation_sign(X, ang):
    return _rotate(X, -np.asarray(ang))


def _mut_pairs_split_halves(X, ang):
    # pairs (m, m + d/2) instead of (2m, 2m + 1)
    X = np.asarray(X, dtype=np.float64)
    d = X.shape[-1]
    perm = np.empty(d, dtype=int)
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2
    out = np.empty_like(X)
    out[..., perm] = _rotate(X[..., perm], ang)
    return out


def _mut_freq_whole_d(n, d, frame0, grid_h, grid_w, theta):
    a = _angles(n, d, frame0, grid_h, grid_w, 1.0)  # positions per pair (theta = 1)
    i = np.arange(d // 2)
    return a * float(theta) ** (-2.0 * i / d)[None, :]


def _mut_freq_offset(n, d, frame0, grid_h, grid_w, theta):
    a = _angles(n, d, frame0, grid_h, grid_w, theta)
    return a * float(theta) ** (-2.0 / d)


def _mut_rows_cols_swapped(n, d, frame0, grid_h, grid_w, theta):
    # row = i % grid_w and column = (i // grid_w) % grid_h
    i = np.arange(n)
    dt, dh, dw = _axes(d)
    rows, cols = i % grid_w, (i // grid_w) % grid_h
    out = _angles(n, d, frame0, grid_h, grid_w, theta).copy()
    jh, jw = np.arange(dh // 2), np.arange(dw // 2)
    out[:, dt // 2:dt // 2 + dh // 2] = rows[:, None] * float(theta) ** (-2.0 * jh / dh)
    out[:, (dt + dh) // 2:] = cols[:, None] * float(theta) ** (-2.0 * jw / dw)
    return out


def _mut_no_frame0(n, d, frame0, grid_h, grid_w, theta):
    return _angles(n, d, 0, grid_h, grid_w, theta)


def _mut_axes_remainder_to_width(d):
    dh = 2 * (d // 6)
    return dh, dh, d - 2 * dh


def _mut_rotated_denominator(Q, K, V, S_in, z_in, eps, frame0, grid_h, grid_w, theta):
    fQ, fK, V = oracle.phi(Q), oracle.phi(K), np.asarray(V, dtype=np.float64)
    n, d = fQ.shape[-2], fQ.shape[-1]
    ang = _angles(n, d, frame0, grid_h, grid_w, theta)
    rQ, rK = _rotate(fQ, ang), _rotate(fK, ang)
    S_out = S_in + np.matmul(np.swapaxes(rK, -1, -2), V)
    z_out = z_in + rK.sum(axis=-2)
    return np.matmul(rQ, S_out) / (np.matmul(rQ, z_out[..., :, None]) + eps), S_out, z_out


def _mut_rope_before_phi(Q, K, V, S_in, z_in, eps, frame0, grid_h, grid_w, theta):
    n, d = np.shape(Q)[-2], np.shape(Q)[-1]
    ang = _angles(n, d, frame0, grid_h, grid_w, theta)
    return oracle.chunk_forward(_rotate(Q, ang), _rotate(K, ang), V, S_in, z_in, eps)


def _mut_query_unrotated(Q, K, V, S_in, z_in, eps, frame0, grid_h, grid_w, theta):
    fQ, fK, V = oracle.phi(Q), oracle.phi(K), np.asarray(V, dtype=np.float64)
    n, d = fQ.shape[-2], fQ.shape[-1]
    rK = _rotate(fK, _angles(n, d, frame0, grid_h, grid_w, theta))
    S_out = S_in + np.matmul(np.swapaxes(rK, -1, -2), V)
    z_out = z_in + fK.sum(axis=-2)
    return np.matmul(fQ, S_out) / (np.matmul(fQ, z_out[..., :, None]) + eps), S_out, z_out


MUTANTS = {
    "rotation_sign": ("rope_rotate", _mut_rotation_sign),
    "pairs_split_halves": ("rope_rotate", _mut_pairs_split_halves),
    "freq_whole_d": ("rope_angles", _mut_freq_whole_d),
    "freq_offset": ("rope_angles", _mut_freq_offset),
    "rows_cols_swapped": ("rope_angles", _mut_rows_cols_swapped),
    "no_frame0": ("rope_angles", _mut_no_frame0),
    "axes_remainder_to_width": ("rope_axes", _mut_axes_remainder_to_width),
    "rotated_denominator": ("rope_chunk_forward", _mut_rotated_denominator),
    "rope_before_phi": ("rope_chunk_forward", _mut_rope_before_phi),
    "query_unrotated": ("rope_chunk_forward", _mut_query_unrotated),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_rope_mutants_caught(name, monkeypatch):
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
