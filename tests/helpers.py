"""Comparison and transfer helpers for the GPU parity tests (no attention
arithmetic here)."""

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

TOL = {"f32": 1e-5, "bf16": 2e-3}


def dev(x, dtype):
    """float32 numpy (already representable in `dtype`) -> device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def normwise(got, ref, axes):
    """max over slices of max|got - ref| / max|ref|, the slice being the
    remaining axes after `axes` (e.g. per (b, h))."""
    err = np.abs(got - ref).max(axis=axes)
    scale = np.abs(ref).max(axis=axes)
    return float(np.max(err / np.maximum(scale, 1e-300)))


def out_err(got, ref):
    """normwise error of [B, H, L, d] outputs per (b, h) slice."""
    return normwise(got, ref, axes=(2, 3))


def state_err(got_state, S_ref, z_ref):
    """(S error, z error) of a [B, H, d*d + d] state, normwise per (b, h)."""
    d = S_ref.shape[-1]
    S = got_state[..., : d * d].reshape(S_ref.shape)
    z = got_state[..., d * d:]
    return normwise(S, S_ref, axes=(2, 3)), normwise(z, z_ref, axes=(2,))


def state_np(S, z):
    B, H, d, _ = S.shape
    return np.concatenate([S.reshape(B, H, d * d), z], axis=-1).astype(np.float32)


def report(name, **vals):
    msg = " ".join(f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}" for k, v in vals.items())
    print(f"[parity] {name} {msg}", flush=True)
    sys.stdout.flush()


def bf16_rne(x):
    """float64 values rounded to bfloat16 (ties to even) through float32,
    the way a float32 result is stored as bfloat16; returned as float64."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).copy()
    u = (u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return u.view(np.float32).astype(np.float64)


def bf16_ulp(r):
    """Spacing of bfloat16 at each bfloat16 value r (toward larger magnitude)."""
    f = np.ascontiguousarray(np.asarray(r, dtype=np.float32))
    u = f.view(np.uint32)
    nxt = ((u & np.uint32(0x7FFFFFFF)) + np.uint32(0x10000)).view(np.float32)
    return np.abs(nxt.astype(np.float64)) - np.abs(f.astype(np.float64))


def bf16_rounding(got, ref, axes, rel_err):
    """A bfloat16 result against the fp64 oracle rounded to bfloat16 (ties to
    even).  Each element may differ from the rounded oracle by at most one
    bfloat16 ulp plus the float32 arithmetic error before rounding
    (rel_err x max|ref| over the slice reduced by `axes`): the float32 value
    can sit on the other side of a rounding boundary.  Returns
    (worst excess over that bound in ulps (<= 0 passes), fraction of elements
    not equal to the rounded oracle).  Rounding to nearest even leaves that
    fraction near zero; truncation or another rounding mode makes it about
    one half."""
    got = np.asarray(got, dtype=np.float64)
    r = bf16_rne(ref)
    ulp = bf16_ulp(r)
    abs_err = rel_err * np.abs(ref).max(axis=axes, keepdims=True)
    excess = (np.abs(got - r) - (ulp + abs_err)) / ulp
    return float(excess.max()), float(np.mean(got != r))


# elements of a bfloat16 result that may differ from the rounded oracle
BF16_MISMATCH_MAX = 0.02


def draw_workers():
    """Host threads for drawing test inputs: the cores this process may use,
    at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def drawn_chunks(draw, chunks, ahead=8):
    """Yield (n, draw(n)) for each n of `chunks`, in order, while up to
    `ahead` later draws run on a thread pool.  Every chunk's tensors come
    from generators seeded by the chunk's own index, so the values do not
    depend on the order or thread the draws run in; numpy fills large arrays
    without holding the interpreter lock, so the draws run in parallel."""
    chunks = list(chunks)
    with ThreadPoolExecutor(min(draw_workers(), max(1, ahead))) as ex:
        futs = {}
        nxt = 0
        for i, n in enumerate(chunks):
            while nxt < len(chunks) and nxt < i + max(1, ahead):
                futs[nxt] = ex.submit(draw, chunks[nxt])
                nxt += 1
            yield n, futs.pop(i).result()
