"""fp64 CPU oracle for kernelised linear attention, global and block-causal.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this package.  The product path (the HIP library and its Python binding)
never imports, calls or falls back to anything here, and nothing here
imports the product.

Sources (web pages about SANA-Video; cited by title and section):

* [TR] "Nvidia, MIT ve diğerleri video yapay zeka devrimini başlattı"
  (aihaber.org), section "Sabit Bellekli KV önbelleğe alma mekanizması":
  the video is cut into N blocks; later blocks fuse earlier blocks'
  features through linear attention and never the reverse; the attention
  can be split along token order with identical results, every token's
  result coming from KV products plus accumulation; KV1 is cached, KV2 is
  added to give KV1-2, and after block n the global KV matrix results;
  each block's work is the accumulated KVsum plus its own KV.
* [ZH] sd114.wiki article on SANA-Video, section "1. 线性 DiT：用 O(N)
  替代 O(N²)": attention is split into a kernel-function mapping followed
  by a global aggregation, never building the N x N attention matrix;
  section "2. 块线性注意力 + 恒定内存 KV 缓存": each chunk keeps only one
  accumulated state as global context, updated by composition, with no
  stored history of keys and values.
* [EN] "SANA-Video: Efficient Video Generation with Block Linear Diffusion
  Transformer" (chatpaper.ai), abstract, designs (1) Linear DiT and
  (2) Constant-Memory KV cache for Block Linear Attention.

What the pages leave open, and the reading taken here (the same reading
the HIP library implements):

* The kernel-function mapping is phi(x) = max(x, 0) (ReLU), applied to
  queries and keys only, never to values.
* The pages never write a normaliser.  The output is normalised by the
  kernel-weight row sum plus a positive eps:
  o_i = phi(q_i)^T S / (phi(q_i) . z + eps), with S = sum_j phi(k_j) v_j^T
  (d x d) and z = sum_j phi(k_j) (d) over the tokens query i may see.
* Visibility: bidirectional inside a block, causal across blocks
  ([TR]: each block uses KVsum plus its *own* KV).  Token j is visible to
  query i iff block(j) <= block(i).

Gradients (``readout_backward``, ``kv_backward``, ``blockcausal_backward``)
are the chain rule applied to the forward definition above, nothing more:
the pages train the model with the same attention ([EN] abstract; [TR]:
block-causal attention in training) but print no gradient formula.  The
derivative of max(x, 0) is taken as 0 at x = 0.

Layout: every tensor is a numpy array [B, H, T, d]; a state is a pair
(S [B, H, d, d], z [B, H, d]) with S[a, c] = sum_t phi(k_t)[a] v_t[c].
All arithmetic is float64 (or exact rationals in ``quadratic_exact``).
"""

from fractions import Fraction

import numpy as np

__all__ = [
    "phi",
    "kv_of_block",
    "readout",
    "chunk_forward",
    "global_forward",
    "stream_forward",
    "prefix_forward",
    "quadratic_forward",
    "quadratic_exact",
    "zero_state",
    "readout_backward",
    "kv_backward",
    "blockcausal_backward",
    "temporal_conv_chunk",
    "temporal_conv_stream",
    "temporal_conv_blockcausal",
    "rope_axes",
    "rope_angles",
    "rope_rotate",
    "rope_chunk_forward",
    "rope_prefix_forward",
    "rope_quadratic_forward",
    "rope_blockcausal_backward",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def phi(x):
    """Kernel-function mapping ([ZH] section 1): ReLU, elementwise."""
    x = _f64(x)
    return np.where(x > 0.0, x, 0.0)


def zero_state(B, H, d):
    """The state before the first block: S_0 = 0, z_0 = 0 ([TR]: the cache
    starts empty and KV1 is the first thing put in it)."""
    return np.zeros((B, H, d, d)), np.zeros((B, H, d))


def kv_of_block(K, V):
    """One block's KV product ([TR], [ZH] section 2).

    KV = phi(K)^T V  ([B, H, d, d], rows indexed by the key feature a,
    columns by the value feature c) and k = phi(K)^T 1 ([B, H, d]).
    """
    fK = phi(K)
    V = _f64(V)
    KV = np.matmul(np.swapaxes(fK, -1, -2), V)
    k = fK.sum(axis=-2)
    return KV, k


def readout(Q, S, z, eps):
    """Global aggregation for a set of queries against one state.

    o_i = phi(q_i)^T S / (phi(q_i) . z + eps), per (b, h).  Q is [B,H,T,d].
    """
    fQ = phi(Q)
    num = np.matmul(fQ, S)                              # [B,H,T,d]
    den = np.matmul(fQ, z[..., :, None]) + float(eps)   # [B,H,T,1]
    return num / den


def chunk_forward(Q, K, V, S_in, z_in, eps):
    """One block of the block-causal form ([TR]: KVsum plus the current
    block's KV): S_out = S_in + KV_n, z_out = z_in + k_n, and the block's
    queries read S_out / z_out.  Returns (O, S_out, z_out)."""
    KV, k = kv_of_block(K, V)
    S_out = _f64(S_in) + KV
    z_out = _f64(z_in) + k
    return readout(Q, S_out, z_out, eps), S_out, z_out


def global_forward(Q, K, V, eps):
    """Global (non-causal) linear attention ([ZH] section 1; [EN] design
    (1)): one state over every token, read by every query.
    Returns (O, S, z)."""
    B, H, _, d = np.shape(Q)
    S0, z0 = zero_state(B, H, d)
    return chunk_forward(Q, K, V, S0, z0, eps)


def stream_forward(blocks, eps, S0=None, z0=None):
    """Block-wise streaming with a carried state ([TR]; [ZH] section 2).

    ``blocks`` is an iterable of (Q_n, K_n, V_n).  Returns
    (outputs, states) where states[n] = (S_n, z_n) after block n.
    """
    outs, states = [], []
    S, z = S0, z0
    for Qn, Kn, Vn in blocks:
        if S is None:
            B, H, _, d = np.shape(Qn)
            S, z = zero_state(B, H, d)
        O, S, z = chunk_forward(Qn, Kn, Vn, S, z, eps)
        outs.append(O)
        states.append((S, z))
    return outs, states


def prefix_forward(Q, K, V, bounds, eps):
    """The same block-causal result by a separate route: every block's KV
    first, then an inclusive prefix sum over the block axis ([TR]: KV1,
    KV1-2, ..., global KV), then every block's queries against its prefix.

    Q, K, V are the whole sequence [B,H,T,d]; ``bounds`` lists the block
    start offsets (first 0) and ends with T.  Returns (O, S_prefix, z_prefix)
    with S_prefix [C,B,H,d,d] and z_prefix [C,B,H,d].
    """
    C = len(bounds) - 1
    KVs, ks = [], []
    for n in range(C):
        a, b = bounds[n], bounds[n + 1]
        KV, k = kv_of_block(K[:, :, a:b], V[:, :, a:b])
        KVs.append(KV)
        ks.append(k)
    S_pre = np.cumsum(np.stack(KVs), axis=0)
    z_pre = np.cumsum(np.stack(ks), axis=0)
    O = np.empty(np.shape(Q), dtype=np.float64)
    for n in range(C):
        a, b = bounds[n], bounds[n + 1]
        O[:, :, a:b] = readout(Q[:, :, a:b], S_pre[n], z_pre[n], eps)
    return O, S_pre, z_pre


def quadratic_forward(Q, K, V, block_id, eps):
    """Explicit quadratic form under the block-causal mask (tiny inputs).

    W_ij = (phi(q_i) . phi(k_j)) * [block(j) <= block(i)],
    o_i = sum_j W_ij v_j / (sum_j W_ij + eps).  This builds the T x T
    matrix that linear attention avoids ([ZH] section 1), which is why it
    is an independent route to the same numbers.  ``block_id`` is a length
    T integer sequence.
    """
    fQ, fK, V = phi(Q), phi(K), _f64(V)
    bid = np.asarray(block_id)
    mask = (bid[None, :] <= bid[:, None]).astype(np.float64)   # [i, j]
    W = np.matmul(fQ, np.swapaxes(fK, -1, -2)) * mask
    return np.matmul(W, V) / (W.sum(axis=-1, keepdims=True) + float(eps))


def quadratic_exact(q, k, v, block_id, eps):
    """The quadratic form in exact rational arithmetic, pure Python loops.

    q, k, v are nested lists [T][d] of ints or Fractions for one (b, h);
    eps is a Fraction.  Every operation (max, x, +, /) is rational, so the
    result (a [T][d] list of Fractions) is exact.
    """
    T = len(q)
    d = len(q[0])
    eps = Fraction(eps)

    def relu(x):
        x = Fraction(x)
        return x if x > 0 else Fraction(0)

    out = []
    for i in range(T):
        wsum = Fraction(0)
        acc = [Fraction(0)] * d
        for j in range(T):
            if block_id[j] > block_id[i]:
                continue
            w = sum((relu(q[i][a]) * relu(k[j][a]) for a in range(d)), Fraction(0))
            wsum += w
            for c in range(d):
                acc[c] += w * Fraction(v[j][c])
        out.append([acc[c] / (wsum + eps) for c in range(d)])
    return out


# --------------------------------------------------------------------------
# Gradients.  For a loss L with dO = dL/dO and (optionally) dL/dS_n, dL/dz_n
# for the state after every block, the chain rule through the definitions
# above gives everything below; no step is fused or reordered beyond it.


def readout_backward(Q, S, z, dO, eps):
    """Gradients of ``readout`` w.r.t. its queries and its state.

    With num_i = phi(q_i)^T S, den_i = phi(q_i) . z + eps, o_i = num_i / den_i:
      dnum_i = do_i / den_i,   dden_i = -(do_i . o_i) / den_i
      dphi(q_i) = S dnum_i + dden_i z,   dq_i = dphi(q_i) * [q_i > 0]
      dS = sum_i phi(q_i) dnum_i^T,      dz = sum_i dden_i phi(q_i)
    Returns (dQ, dS, dz).
    """
    fQ = phi(Q)
    dO = _f64(dO)
    S = _f64(S)
    z = _f64(z)
    den = np.matmul(fQ, z[..., :, None]) + float(eps)          # [B,H,T,1]
    O = np.matmul(fQ, S) / den
    dnum = dO / den
    dden = -np.sum(dO * O, axis=-1, keepdims=True) / den       # [B,H,T,1]
    dfQ = np.matmul(dnum, np.swapaxes(S, -1, -2)) + dden * z[..., None, :]
    dQ = np.where(_f64(Q) > 0.0, dfQ, 0.0)
    fQt = np.swapaxes(fQ, -1, -2)
    dS = np.matmul(fQt, dnum)
    dz = np.matmul(fQt, dden)[..., 0]
    return dQ, dS, dz


def kv_backward(K, V, dKV, dk):
    """Gradients of ``kv_of_block`` given dL/dKV ([B,H,d,d]) and dL/dk
    ([B,H,d]).  KV = sum_j phi(k_j) v_j^T and k = sum_j phi(k_j), so
      dphi(k_j) = dKV v_j + dk,   dk_j = dphi(k_j) * [k_j > 0],
      dv_j = dKV^T phi(k_j).
    Returns (dK, dV)."""
    fK = phi(K)
    V = _f64(V)
    dKV = _f64(dKV)
    dfK = np.matmul(V, np.swapaxes(dKV, -1, -2)) + _f64(dk)[..., None, :]
    dK = np.where(_f64(K) > 0.0, dfK, 0.0)
    dV = np.matmul(fK, dKV)
    return dK, dV


def _suffix_sums(xs):
    """[x_0, ..., x_{C-1}] -> [sum_{m >= n} x_m for n in 0..C-1]."""
    out = [None] * len(xs)
    acc = None
    for n in range(len(xs) - 1, -1, -1):
        acc = xs[n] if acc is None else acc + xs[n]
        out[n] = acc
    return out


def blockcausal_backward(Q, K, V, bounds, dO, eps, S0=None, z0=None, dS=None, dz=None):
    """Gradients of the block-causal form over a whole sequence.

    The forward: S_n = S0 + KV_1 + ... + KV_n (and z_n likewise) for the
    blocks given by ``bounds`` (as in ``prefix_forward``), and block n's
    queries read (S_n, z_n) ([TR]: KVsum plus the block's own KV).  Since
    KV_m enters S_n for every n >= m, its gradient is the suffix sum
      R_m = sum_{n >= m} (dL/dS_n),
    where dL/dS_n collects block n's readout gradient plus the caller's
    dS[n] (the gradient of the state output after block n, zero if None).
    dL/dS0 = R_1 because S0 enters every S_n.

    Q, K, V, dO: [B,H,T,d].  S0 [B,H,d,d], z0 [B,H,d] (None: zeros).
    dS [C,B,H,d,d], dz [C,B,H,d] or None.
    Returns (dQ, dK, dV, dS0, dz0).
    """
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    B, H, T, d = Q.shape
    C = len(bounds) - 1
    if S0 is None:
        S0, z0 = zero_state(B, H, d)
    S, z = _f64(S0), _f64(z0)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(Q)
    dV = np.zeros_like(Q)
    GS, Gz = [], []
    for n in range(C):
        a, b = bounds[n], bounds[n + 1]
        KV, k = kv_of_block(K[:, :, a:b], V[:, :, a:b])
        S, z = S + KV, z + k
        dQn, dSn, dzn = readout_backward(Q[:, :, a:b], S, z, dO[:, :, a:b], eps)
        dQ[:, :, a:b] = dQn
        if dS is not None:
            dSn = dSn + _f64(dS[n])
            dzn = dzn + _f64(dz[n])
        GS.append(dSn)
        Gz.append(dzn)
    RS, Rz = _suffix_sums(GS), _suffix_sums(Gz)
    for n in range(C):
        a, b = bounds[n], bounds[n + 1]
        dK[:, :, a:b], dV[:, :, a:b] = kv_backward(K[:, :, a:b], V[:, :, a:b], RS[n], Rz[n])
    if C == 0:
        return dQ, dK, dV, np.zeros((B, H, d, d)), np.zeros((B, H, d))
    return dQ, dK, dV, RS[0], Rz[0]


# --------------------------------------------------------------------------
# Temporal convolution of the Spatial-Temporal Mix-FFN and its chunk-boundary
# cache.  [TR] section "Verimli doğrusal DiT": the MLP alternates a 1x3x3
# spatial and a 3x1x1 temporal convolution; [ZH] section 1: a temporal
# convolution module models motion between frames.  What the pages leave
# open, and the reading taken here:
# * the 3x1x1 convolution is depthwise (one 3-tap filter per channel along
#   latent frames, as the Mix-FFN's convolutions are per channel), with an
#   optional per-channel bias;
# * in block-causal streaming it follows the attention's visibility rule
#   ([TR]: later blocks read earlier ones, never the reverse; bidirectional
#   inside a block): frame f of a chunk reads frames f - 1, f, f + 1 of the
#   sequence, except that a frame of a later chunk is never visible (zero),
#   and before the first frame of the video there is nothing (zero).  So a
#   stream needs only the previous chunk's last frame: a one-frame cache,
#   constant in memory like the attention state.
# Layout: x [B, F, P, C] (frames, positions per frame, channels), w [C, 3]
# (taps for f - 1, f, f + 1), b [C], a cache [B, P, C].


def temporal_conv_chunk(x, w, b=None, cache=None):
    """One chunk of F frames: y[f] = w0 x[f-1] + w1 x[f] + w2 x[f+1] + b per
    channel, with x[-1] = cache (zeros if None: the start of a video) and
    x[F] = 0 (the next chunk is not visible).  Returns (y, cache_out) with
    cache_out = x[F-1] (the cache is unchanged when F = 0)."""
    x = _f64(x)
    w = _f64(w)
    B, F, P, C = x.shape
    prev = np.zeros((B, P, C)) if cache is None else _f64(cache)
    if F == 0:
        return np.zeros_like(x), prev
    xp = np.concatenate([prev[:, None], x, np.zeros((B, 1, P, C))], axis=1)  # [B, F+2, P, C]
    y = w[:, 0] * xp[:, 0:F] + w[:, 1] * xp[:, 1:F + 1] + w[:, 2] * xp[:, 2:F + 2]
    if b is not None:
        y = y + _f64(b)
    return y, x[:, F - 1]


def temporal_conv_stream(chunks, w, b=None, cache=None):
    """Chunks in order with the one-frame cache carried between them.
    Returns (outputs, caches)."""
    outs, caches = [], []
    for xc in chunks:
        y, cache = temporal_conv_chunk(xc, w, b, cache)
        outs.append(y)
        caches.append(cache)
    return outs, caches


def temporal_conv_blockcausal(x, w, b, Tf, cache=None):
    """The whole sequence of F frames in chunks of Tf frames, written as an
    explicit visibility-masked sum (a separate route from the carried
    cache): y[f] = sum over taps t in {-1, 0, 1} of w[t + 1] x[f + t] where
    frame g = f + t is used iff 0 <= g < F and chunk(g) <= chunk(f), and
    x[-1] = cache (zeros if None)."""
    x = _f64(x)
    w = _f64(w)
    B, F, P, C = x.shape
    y = np.zeros_like(x)
    for f in range(F):
        acc = np.zeros((B, P, C))
        for t in (-1, 0, 1):
            g = f + t
            if g < 0:
                src = None if cache is None else _f64(cache)
            elif g < F and g // Tf <= f // Tf:
                src = x[:, g]
            else:
                src = None
            if src is not None:
                acc = acc + w[:, t + 1] * src
        y[:, f] = acc if b is None else acc + _f64(b)
    return y


# --------------------------------------------------------------------------
# Rotary position embedding over the latent token grid.  [ZH] section 1: the
# Linear DiT adds rotary position encoding (RoPE) for awareness of relative
# positions in space and time.  The pages say no more, so every step below
# is a reading:
# * 3-D RoPE: token i of a sequence whose frames hold grid_h x grid_w tokens
#   (row-major) sits at frame frame0 + i // (grid_h grid_w), row
#   (i // grid_w) % grid_h, column i % grid_w.  The head dimension is split
#   into a temporal, a row and a column group of d_t, d_h, d_w features,
#   d_h = d_w = 2 floor(d / 6) and d_t = d - d_h - d_w (three even parts as
#   equal as they can be, the remainder to time).
# * Features (2m, 2m + 1) form pair m; pairs [0, d_t/2) rotate with the
#   frame, the next d_h/2 with the row, the last d_w/2 with the column.  Pair
#   j of a group of size d_a turns by the angle p * theta^(-2 j / d_a) for
#   the token's position p on that axis; (x, y) -> (x cos - y sin,
#   x sin + y cos).
# * Placement: the linear-attention form of RoPE of Su et al., "RoFormer:
#   Enhanced Transformer with Rotary Position Embedding" (2021, section
#   3.4.3): the rotation acts on the feature-mapped queries and keys in the
#   numerator only; the denominator keeps the unrotated phi(q) . phi(k), which
#   stays positive.  So the state becomes S = sum_j R_j phi(k_j) v_j^T (keys
#   rotated by their absolute positions) while z = sum_j phi(k_j) is as before,
#   and o_i = (R_i phi(q_i))^T S / (phi(q_i) . z + eps).  Since R_i^T R_j
#   depends only on the position difference, the state carries across blocks
#   as long as every call passes the absolute frame0 of its first token.


def rope_axes(d):
    """(d_t, d_h, d_w): the features given to frame, row and column."""
    dh = 2 * (d // 6)
    return d - 2 * dh, dh, dh


def rope_angles(n, d, frame0, grid_h, grid_w, theta):
    """Rotation angles [n, d/2] of the first n tokens of a sequence whose
    token 0 is at frame frame0 (row 0, column 0)."""
    i = np.arange(n)
    hw = grid_h * grid_w
    pos = (frame0 + i // hw, (i // grid_w) % grid_h, i % grid_w)
    parts = []
    for p, da in zip(pos, rope_axes(d)):
        if da == 0:
            continue
        j = np.arange(da // 2, dtype=np.float64)
        freq = float(theta) ** (-2.0 * j / da)
        parts.append(np.asarray(p, dtype=np.float64)[:, None] * freq[None, :])
    return np.concatenate(parts, axis=1)


def rope_rotate(X, ang):
    """Turn feature pair m of token t of X [..., n, d] by ang[t, m]."""
    X = _f64(X)
    x, y = X[..., 0::2], X[..., 1::2]
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(X)
    out[..., 0::2] = x * c - y * s
    out[..., 1::2] = x * s + y * c
    return out


def rope_chunk_forward(Q, K, V, S_in, z_in, eps, frame0, grid_h, grid_w, theta):
    """One block with RoPE: S_out = S_in + (R phi(K))^T V, z_out = z_in +
    phi(K)^T 1, o_i = (R_i phi(q_i))^T S_out / (phi(q_i) . z_out + eps), the
    block's token 0 at frame frame0.  Returns (O, S_out, z_out)."""
    fQ, fK, V = phi(Q), phi(K), _f64(V)
    n, d = fQ.shape[-2], fQ.shape[-1]
    ang = rope_angles(n, d, frame0, grid_h, grid_w, theta)
    rK = rope_rotate(fK, ang)
    S_out = _f64(S_in) + np.matmul(np.swapaxes(rK, -1, -2), V)
    z_out = _f64(z_in) + fK.sum(axis=-2)
    num = np.matmul(rope_rotate(fQ, ang), S_out)
    den = np.matmul(fQ, z_out[..., :, None]) + float(eps)
    return num / den, S_out, z_out


def rope_prefix_forward(Q, K, V, bounds, eps, frame0, grid_h, grid_w, theta, S0=None, z0=None):
    """The block-causal sequence with RoPE by the prefix route: angles of the
    whole sequence, every block's rotated KV, an inclusive prefix sum over
    blocks (plus S0, z0), then every block's queries.  Returns (O, S_prefix,
    z_prefix) as ``prefix_forward``."""
    fQ, fK, V = phi(Q), phi(K), _f64(V)
    B, H, n, d = fQ.shape
    ang = rope_angles(n, d, frame0, grid_h, grid_w, theta)
    rQ, rK = rope_rotate(fQ, ang), rope_rotate(fK, ang)
    C = len(bounds) - 1
    KVs = [np.matmul(np.swapaxes(rK[:, :, a:b], -1, -2), V[:, :, a:b])
           for a, b in zip(bounds[:-1], bounds[1:])]
    ks = [fK[:, :, a:b].sum(axis=-2) for a, b in zip(bounds[:-1], bounds[1:])]
    S_pre = np.cumsum(np.stack(KVs), axis=0)
    z_pre = np.cumsum(np.stack(ks), axis=0)
    if S0 is not None:
        S_pre = S_pre + _f64(S0)
        z_pre = z_pre + _f64(z0)
    O = np.empty((B, H, n, d))
    for c in range(C):
        a, b = bounds[c], bounds[c + 1]
        num = np.matmul(rQ[:, :, a:b], S_pre[c])
        den = np.matmul(fQ[:, :, a:b], z_pre[c][..., :, None]) + float(eps)
        O[:, :, a:b] = num / den
    return O, S_pre, z_pre


def rope_quadratic_forward(Q, K, V, block_id, eps, frame0, grid_h, grid_w, theta):
    """Explicit quadratic form with RoPE (tiny inputs): W_ij = (R_i phi(q_i))
    . (R_j phi(k_j)) and D_ij = phi(q_i) . phi(k_j), both masked by
    [block(j) <= block(i)]; o_i = sum_j W_ij v_j / (sum_j D_ij + eps)."""
    fQ, fK, V = phi(Q), phi(K), _f64(V)
    n, d = fQ.shape[-2], fQ.shape[-1]
    ang = rope_angles(n, d, frame0, grid_h, grid_w, theta)
    rQ, rK = rope_rotate(fQ, ang), rope_rotate(fK, ang)
    bid = np.asarray(block_id)
    mask = (bid[None, :] <= bid[:, None]).astype(np.float64)
    W = np.matmul(rQ, np.swapaxes(rK, -1, -2)) * mask
    D = np.matmul(fQ, np.swapaxes(fK, -1, -2)) * mask
    return np.matmul(W, V) / (D.sum(axis=-1, keepdims=True) + float(eps))


def rope_blockcausal_backward(Q, K, V, bounds, dO, eps, frame0, grid_h, grid_w, theta,
                              S0=None, z0=None, dS=None, dz=None):
    """Gradients of the RoPE'd block-causal form (``rope_prefix_forward``),
    the chain rule through its definition.  With q~ = R phi(q), k~ = R phi(k)
    (R the token's rotation; its transpose turns by the opposite angles):
      block n, query i:  dnum_i = do_i / den_i,  dden_i = -(do_i . o_i) / den_i
        dphi(q_i) = R_i^T (S_n dnum_i) + dden_i z_n,  dq_i = dphi(q_i) * [q_i > 0]
        dS_n += sum_i q~_i dnum_i^T,  dz_n += sum_i dden_i phi(q_i)
      suffixes G_m = sum_{n >= m} dS_n (with dL/dS_n), g_m likewise
      block m, key j:  dphi(k_j) = R_j^T (G_m v_j) + g_m,  dk_j = dphi(k_j) * [k_j > 0]
        dv_j = G_m^T k~_j
    Arguments as ``rope_prefix_forward`` plus dO [B,H,T,d] and dS [C,B,H,d,d],
    dz [C,B,H,d] (None: zero).  Returns (dQ, dK, dV, dS0, dz0)."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    B, H, n, d = Q.shape
    C = len(bounds) - 1
    fQ, fK = phi(Q), phi(K)
    ang = rope_angles(n, d, frame0, grid_h, grid_w, theta)
    rQ, rK = rope_rotate(fQ, ang), rope_rotate(fK, ang)
    if S0 is None:
        S0, z0 = zero_state(B, H, d)
    S, z = _f64(S0), _f64(z0)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(Q)
    dV = np.zeros_like(Q)
    GS, Gz = [], []
    for c in range(C):
        a, b = bounds[c], bounds[c + 1]
        S = S + np.matmul(np.swapaxes(rK[:, :, a:b], -1, -2), V[:, :, a:b])
        z = z + fK[:, :, a:b].sum(axis=-2)
        den = np.matmul(fQ[:, :, a:b], z[..., :, None]) + float(eps)
        O = np.matmul(rQ[:, :, a:b], S) / den
        dnum = dO[:, :, a:b] / den
        dden = -np.sum(dO[:, :, a:b] * O, axis=-1, keepdims=True) / den
        drq = np.matmul(dnum, np.swapaxes(S, -1, -2))
        dfq = rope_rotate(drq, -ang[a:b]) + dden * z[..., None, :]
        dQ[:, :, a:b] = np.where(Q[:, :, a:b] > 0.0, dfq, 0.0)
        dSn = np.matmul(np.swapaxes(rQ[:, :, a:b], -1, -2), dnum)
        dzn = np.matmul(np.swapaxes(fQ[:, :, a:b], -1, -2), dden)[..., 0]
        if dS is not None:
            dSn = dSn + _f64(dS[c])
            dzn = dzn + _f64(dz[c])
        GS.append(dSn)
        Gz.append(dzn)
    RS, Rz = _suffix_sums(GS), _suffix_sums(Gz)
    for c in range(C):
        a, b = bounds[c], bounds[c + 1]
        drk = np.matmul(V[:, :, a:b], np.swapaxes(RS[c], -1, -2))
        dfk = rope_rotate(drk, -ang[a:b]) + Rz[c][..., None, :]
        dK[:, :, a:b] = np.where(K[:, :, a:b] > 0.0, dfk, 0.0)
        dV[:, :, a:b] = np.matmul(rK[:, :, a:b], RS[c])
    if C == 0:
        return dQ, dK, dV, np.zeros((B, H, d, d)), np.zeros((B, H, d))
    return dQ, dK, dV, RS[0], Rz[0]
