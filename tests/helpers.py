"""Comparison and transfer helpers for the GPU parity tests (no attention
arithmetic here)."""

import sys

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
