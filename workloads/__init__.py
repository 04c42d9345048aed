"""Seeded synthetic inputs shaped like SANA-Video's latent-token workloads.

This module is shared by the tests, the benchmark and the oracle checks.
It draws random numbers and rounds them to the storage precision; it holds
none of the attention arithmetic.

Token grids.  A 5 s, 81-frame clip becomes 21 latent frames (4x temporal
compression); with the 8x spatial VAE plus a 2x2 patch the grid is the
frame size / 16 per side: 480x832 -> 30x52 = 1,560 tokens per latent
frame, 720x1280 -> 45x80 = 3,600 ("Nvidia, MIT ve diğerleri video yapay
zeka devrimini başlattı", sections on DC-AE-V and the Wan-VAE / F8T4C16
comparison).  The pages' quality benchmark (VBench) is not used; these
seeded normal tensors stand in for real latents.

Every tensor is [B, H, T, d] float32 holding values that are exactly
representable in the configuration's storage type (bfloat16 values are
rounded to nearest-even).  Any (config, tensor, chunk) triple can be
regenerated on its own: the stream is
``np.random.default_rng(np.random.SeedSequence([cfg, tensor, chunk]))``
with tensor 0 = Q, 1 = K, 2 = V, 3 = the outlier-row mask.
"""

from dataclasses import dataclass

import numpy as np

EPS = float(np.float32(1e-6))

Q_ID, K_ID, V_ID, MASK_ID = 0, 1, 2, 3
# upstream gradients for the backward tests: dL/dO, dL/d(block states)
DO_ID, DSTATE_ID = 4, 5
# temporal-convolution inputs: activations, taps and bias, cache
TC_X_ID, TC_W_ID, TC_C_ID = 6, 7, 8


@dataclass(frozen=True)
class Workload:
    cid: int            # seed namespace
    name: str
    form: str           # "global" or "chunk"
    B: int
    H: int
    d: int
    L: int              # tokens per call (per chunk, or the whole sequence)
    chunks: int         # number of calls in sequence
    dtype: str          # "f32" or "bf16"
    scale: float = 1.0
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0

    @property
    def tokens(self):
        return self.L * self.chunks


LAT_480 = 21 * 30 * 52   # 32,760
LAT_720 = 21 * 45 * 80   # 75,600

WORKLOADS = {
    1: Workload(1, "tiny-f32-block-causal", "chunk", 1, 2, 32, 64, 4, "f32"),
    2: Workload(2, "480p-5s-global", "global", 1, 16, 64, LAT_480, 1, "bf16"),
    3: Workload(3, "720p-5s-global", "global", 1, 32, 64, LAT_720, 1, "bf16", scale=0.5),
    4: Workload(4, "480p-1min-stream", "chunk", 1, 16, 64, LAT_480, 12, "bf16"),
    5: Workload(5, "long-horizon-d128", "chunk", 4, 16, 128, 4 * 32 * 32, 40, "bf16",
                outlier_frac=0.01, outlier_scale=8.0),
}

# Latent token grid (rows, columns) of one frame per workload, for the
# rotary-position calls: chunk n of a workload starts at frame
# n * L / (rows * columns).  The tiny block-causal workload (64 tokens per
# chunk) is taken as four 4 x 4 frames and the long-horizon one (4,096 tokens)
# as four 32 x 32 frames; the video workloads use their latent grids.
GRIDS = {1: (4, 4), 2: (30, 52), 3: (45, 80), 4: (30, 52), 5: (32, 32)}
ROPE_THETA = 10000.0


def chunk_frame0(w, chunk):
    """Frame index of the first token of chunk ``chunk`` of workload ``w``."""
    gh, gw = GRIDS[w.cid]
    return chunk * w.L // (gh * gw)


# The timed workload: one block-causal chunk at the 720p latent shape, the
# config-3 distribution, chunk 1 read against the state left by chunk 0.
CHUNK_720P = Workload(3, "720p-chunk", "chunk", 1, 32, 64, LAT_720, 2, "bf16", scale=0.5)


def bf16_round(x):
    """Round float32 values to the nearest bfloat16 (ties to even); the
    result is float32 holding bf16-representable values.  Finite inputs."""
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    u = x.view(np.uint32)
    # finite values: the largest bit pattern plus 0x8000 still fits in 32 bits
    lsb = u >> 16
    lsb &= 1
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return x


def _rng(cid, tensor, chunk):
    return np.random.default_rng(np.random.SeedSequence([int(cid), int(tensor), int(chunk)]))


def draw(cid, tensor, chunk, shape, dtype="bf16", scale=1.0,
         outlier_frac=0.0, outlier_scale=1.0):
    """One seeded tensor of standard normals, scaled, with optional outlier
    rows, rounded to the storage precision."""
    x = _rng(cid, tensor, chunk).standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    if outlier_frac > 0.0:
        B, H, T, _ = shape
        u = _rng(cid, MASK_ID, chunk).random(size=(3, B, H, T))
        rows = u[tensor] < outlier_frac
        x[rows] *= np.float32(outlier_scale)
    if dtype == "bf16":
        x = bf16_round(x)
    return x


def chunk_qkv(w, chunk):
    """(Q, K, V) of chunk ``chunk`` of workload ``w`` as float32 arrays."""
    shape = (w.B, w.H, w.L, w.d)
    kw = dict(dtype=w.dtype, scale=w.scale, outlier_frac=w.outlier_frac,
              outlier_scale=w.outlier_scale)
    return tuple(draw(w.cid, t, chunk, shape, **kw) for t in (Q_ID, K_ID, V_ID))


def random_qkv(seed, B, H, L, d, dtype="bf16", scale=1.0, chunk=0):
    """Ad-hoc test shapes: the same generator under a caller-chosen seed."""
    w = Workload(seed, "adhoc", "chunk", B, H, d, L, 1, dtype, scale=scale)
    return chunk_qkv(w, chunk)


def random_state(seed, B, H, d, tokens=1000):
    """A plausible fp32 carried state (S, z): what ``tokens`` N(0,1) keys
    and values would leave behind, drawn directly (S ~ N(0, tokens/2),
    z ~ |N| * tokens/2.5) without running attention."""
    g = _rng(seed, 7, 0)
    S = (g.standard_normal((B, H, d, d)) * np.sqrt(tokens / 2.0)).astype(np.float32)
    z = (np.abs(g.standard_normal((B, H, d))) * 0.1 + 0.4) * tokens
    return S, z.astype(np.float32)


def random_grads(seed, B, H, N, d, dtype="f32", chunk=0, scale=1.0):
    """An upstream gradient dL/dO [B, H, N, d] ~ N(0, 1) * scale, rounded to
    the gradient's storage precision (tensor id 4 of the seed's streams)."""
    return draw(seed, DO_ID, chunk, (B, H, N, d), dtype=dtype, scale=scale)


def random_state_grads(seed, B, H, C, d, scale=1e-4):
    """Gradients of C block states: (dS [C, B, H, d, d], dz [C, B, H, d]),
    N(0, 1) * scale in float32 (tensor id 5)."""
    g = _rng(seed, DSTATE_ID, 0)
    dS = (g.standard_normal((C, B, H, d, d)) * scale).astype(np.float32)
    dz = (g.standard_normal((C, B, H, d)) * scale).astype(np.float32)
    return dS, dz


def random_tconv(seed, B, F, P, C, dtype="bf16", chunk=0):
    """Inputs of the Mix-FFN temporal convolution: activations x [B, F, P, C]
    ~ N(0, 1) rounded to the storage precision (chunk-addressable: chunk n
    of a stream is its own draw), taps w [C, 3] ~ N(0, 1/3) and bias [C] ~
    N(0, 0.1^2) in float32, and a cache [B, P, C] ~ N(0, 1) at the storage
    precision (the last frame of a preceding chunk)."""
    x = draw(seed, TC_X_ID, chunk, (B, F, P, C), dtype=dtype)
    g = _rng(seed, TC_W_ID, 0)
    w = (g.standard_normal((C, 3)) / np.sqrt(3.0)).astype(np.float32)
    b = (g.standard_normal(C) * 0.1).astype(np.float32)
    cache = draw(seed, TC_C_ID, 0, (B, 1, P, C), dtype=dtype)[:, 0]
    return x, w, b, cache
