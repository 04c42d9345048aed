"""Python binding of liblinattn, the gfx950 linear-attention library.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, output buffers are allocated with torch when the caller does not
pass them, and raw device pointers plus the current HIP stream go to the C
ABI (include/linattn.h).  Every arithmetic step runs in the library's HIP
kernels.  There is no fallback: if liblinattn.so is missing or a call is
rejected, an exception is raised.

Shapes: q, k, v and out are [B, H, L, d]; a state is [B, H, d*d + d] float32
(S[a, c] at a*d + c, then z).  d is 32, 64 or 128; q/k/v are float32 or
bfloat16; out is float32 (default) or bfloat16.  The backward calls take
dO in float32 or bfloat16 and return dq, dk, dv in that type.
"""

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# LINATTN_LIB names another build of the same library (the sanitizer build of
# the host code, for the CPU contract tests); by default the in-tree one.
LIB_PATH = os.environ.get("LINATTN_LIB") or os.path.join(_HERE, "liblinattn.so")

LA_OK, LA_E_INVAL, LA_E_UNSUPPORTED, LA_E_ALIGN, LA_E_ALIAS, LA_E_HIP, LA_E_SCRATCH = range(7)
# static device scratch of la_blockcausal_backward_noalloc
NOALLOC_SCRATCH_BYTES = 32 << 20
LA_F32, LA_BF16 = 0, 1
DEFAULT_EPS = 1e-6
DEFAULT_THETA = 10000.0

_DTYPE = {torch.float32: LA_F32, torch.bfloat16: LA_BF16}


class LinAttnError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {_status_string(status)} (status {status})")


class LaunchOpts(ctypes.Structure):
    _fields_ = [("kv_splits", ctypes.c_int), ("readout_workgroups", ctypes.c_int),
                ("stage_events", ctypes.POINTER(ctypes.c_void_p))]


class BackwardShape(ctypes.Structure):
    _fields_ = [("blocks", ctypes.c_int), ("query_splits", ctypes.c_int),
                ("query_workgroups", ctypes.c_int), ("key_items", ctypes.c_int),
                ("key_workgroups", ctypes.c_int), ("key_sweep_units", ctypes.c_int)]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t

_SIGNATURES = {
    "la_state_reset": [_P, _I, _I, _I, _P],
    "la_chunk_forward": [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P],
    "la_chunk_forward_ex": [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F,
                            ctypes.POINTER(LaunchOpts), _P],
    "la_global_forward": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P],
    "la_global_forward_ex": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F,
                             ctypes.POINTER(LaunchOpts), _P],
    "la_blockcausal_forward": [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P],
    "la_blockcausal_forward_ex": [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F,
                                  ctypes.POINTER(LaunchOpts), _P],
    "la_chunk_forward_rope": [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _F,
                              _P],
    "la_blockcausal_forward_rope": [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I,
                                    _I, _I, _F, _P],
    "la_global_forward_rope": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _F,
                               _P],
    "la_blockcausal_forward_rope_ex": [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F,
                                       _I, _I, _I, _F, ctypes.POINTER(LaunchOpts), _P],
    "la_backward_workspace_size": [_I, _I, _I, _I, _I, _I, ctypes.POINTER(_Z)],
    "la_backward_stream_count": [_I, _I, _I, _I, _I, _I, _I, ctypes.POINTER(_I)],
    "la_backward_plan": [_I, _I, _I, _I, _I, _I, _I, _I, _I, _Z, ctypes.POINTER(BackwardShape)],
    "la_blockcausal_backward": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                _I, _I, _F, _P, _Z, _P],
    "la_blockcausal_backward_ex": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I,
                                   _I, _I, _I, _F, _P, _Z, ctypes.POINTER(LaunchOpts), _P],
    "la_blockcausal_backward_noalloc": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I,
                                        _I, _I, _I, _I, _F, _P],
    "la_blockcausal_backward_rope": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                     _I, _I, _F, _P, _Z, _I, _I, _I, _F, _P],
    "la_blockcausal_backward_rope_ex": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I,
                                        _I, _I, _I, _F, _P, _Z, _I, _I, _I, _F,
                                        ctypes.POINTER(LaunchOpts), _P],
    "la_chunk_backward": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F,
                          _P, _Z, _P],
    "la_chunk_backward_rope": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                               _F, _P, _Z, _I, _I, _I, _F, _P],
    "la_global_backward": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _Z,
                           _P],
    "la_global_backward_rope": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P,
                                _Z, _I, _I, _I, _F, _P],
    "la_temporal_conv_chunk": [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P],
    "la_temporal_conv_blockcausal": [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P],
    "la_plan": [_I, _I, _I, _I, _I, _I, _I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I)],
    "la_status_string": [_I],
    "la_abi_version": [],
}
EXPORTS = tuple(_SIGNATURES)


def lib():
    """The loaded liblinattn (ctypes.CDLL); raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m block_causal_linear_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, argtypes in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = argtypes
            fn.restype = ctypes.c_char_p if name == "la_status_string" else ctypes.c_int
        _lib = handle
    return _lib


def _status_string(status):
    try:
        return lib().la_status_string(int(status)).decode()
    except Exception:  # pragma: no cover - only when the library itself is missing
        return "unknown"


def _check(status, what):
    if status != LA_OK:
        raise LinAttnError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def head_dim_of_state(state):
    """d from a state's last dimension d*d + d."""
    e = state.shape[-1]
    d = (math.isqrt(4 * e + 1) - 1) // 2
    if d * d + d != e:
        raise ValueError(f"state last dimension {e} is not d*d + d")
    return d


def new_state(B, H, d, device="cuda"):
    """A zero state [B, H, d*d + d] float32 (allocated by torch, cleared by
    the library's fill kernel)."""
    st = torch.empty((B, H, d * d + d), dtype=torch.float32, device=device)
    state_reset(st)
    return st


def state_reset(state):
    B, H, _ = state.shape
    d = head_dim_of_state(state)
    _need(state, "state", torch.float32)
    _check(lib().la_state_reset(_ptr(state), B, H, d, _stream(state.device)), "la_state_reset")
    return state


def split_state(state):
    """Views (S [B, H, d, d], z [B, H, d]) of a state tensor."""
    d = head_dim_of_state(state)
    return state[..., : d * d].unflatten(-1, (d, d)), state[..., d * d:]


def _need(t, name, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _prepare_out(q, k, v, out, out_dtype):
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name)
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, L, d]")
    if not (q.shape == k.shape == v.shape):
        raise ValueError(f"q, k, v shapes differ: {tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPE:
        raise TypeError("q, k, v must share one dtype, float32 or bfloat16")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _need(out, "out")
    if out.shape != q.shape or out.dtype not in _DTYPE or out.device != q.device:
        raise ValueError("out must be [B, H, L, d], float32 or bfloat16, on q's device")
    return out


def _prepare(q, k, v, out, out_dtype, state_out):
    out = _prepare_out(q, k, v, out, out_dtype)
    B, H, L, d = q.shape
    if state_out is None:
        state_out = torch.empty((B, H, d * d + d), dtype=torch.float32, device=q.device)
    _need(state_out, "state_out", torch.float32)
    if tuple(state_out.shape) != (B, H, d * d + d) or state_out.device != q.device:
        raise ValueError(f"state_out must be [{B}, {H}, {d * d + d}] on q's device")
    return out, state_out


def _opts(kv_splits, readout_workgroups, stage_events):
    if not kv_splits and not readout_workgroups and stage_events is None:
        return None
    o = LaunchOpts()
    o.kv_splits = int(kv_splits or 0)
    o.readout_workgroups = int(readout_workgroups or 0)
    if stage_events is not None:
        o.stage_events = stage_events.as_ctypes()
    return o


def chunk_forward(q, k, v, state_in, out=None, state_out=None, eps=DEFAULT_EPS,
                  out_dtype=torch.float32, kv_splits=0, readout_workgroups=0, stage_events=None):
    """One block of the block-causal form: returns (out, state_out) with
    state_out = state_in + phi(K)^T V (and + phi(K)^T 1 for z) and every query
    of the block read against state_out.  state_out may be state_in."""
    out, state_out = _prepare(q, k, v, out, out_dtype, state_out)
    _need(state_in, "state_in", torch.float32)
    if state_in.shape != state_out.shape or state_in.device != q.device:
        raise ValueError("state_in must match state_out's shape and device")
    B, H, L, d = q.shape
    o = _opts(kv_splits, readout_workgroups, stage_events)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(state_in), _ptr(out), _ptr(state_out),
            B, H, L, d, _DTYPE[q.dtype], _DTYPE[out.dtype], float(eps))
    L_ = lib()
    if o is None:
        rc = L_.la_chunk_forward(*args, _stream(q.device))
    else:
        rc = L_.la_chunk_forward_ex(*args, ctypes.byref(o), _stream(q.device))
    _check(rc, "la_chunk_forward")
    return out, state_out


def global_forward(q, k, v, out=None, state_out=None, eps=DEFAULT_EPS,
                   out_dtype=torch.float32, kv_splits=0, readout_workgroups=0, stage_events=None):
    """Global (non-causal) linear attention: returns (out, state_out) where
    state_out holds the global (S, z)."""
    out, state_out = _prepare(q, k, v, out, out_dtype, state_out)
    B, H, L, d = q.shape
    o = _opts(kv_splits, readout_workgroups, stage_events)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(state_out),
            B, H, L, d, _DTYPE[q.dtype], _DTYPE[out.dtype], float(eps))
    L_ = lib()
    if o is None:
        rc = L_.la_global_forward(*args, _stream(q.device))
    else:
        rc = L_.la_global_forward_ex(*args, ctypes.byref(o), _stream(q.device))
    _check(rc, "la_global_forward")
    return out, state_out


def global_forward_rope(q, k, v, frame0, grid_h, grid_w, theta=DEFAULT_THETA, out=None,
                        state_out=None, eps=DEFAULT_EPS, out_dtype=torch.float32):
    """global_forward with rotary position embedding on the numerator
    (token 0 at frame frame0 of grid_h x grid_w tokens); state_out holds S
    with every key turned by its position, and z."""
    out, state_out = _prepare(q, k, v, out, out_dtype, state_out)
    B, H, L, d = q.shape
    _check(lib().la_global_forward_rope(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(state_out), B, H, L, d, _DTYPE[q.dtype],
        _DTYPE[out.dtype], float(eps), int(frame0), int(grid_h), int(grid_w), float(theta),
        _stream(q.device)), "la_global_forward_rope")
    return out, state_out


def _prepare_blockcausal(q, k, v, T, state_in, out, states, out_dtype):
    _need(q, "q")
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    T = int(T)
    if T < 1:
        raise ValueError("T must be >= 1")
    C = -(-N // T) if N > 0 else 0
    if states is None:
        states = torch.empty((B, H, C, d * d + d), dtype=torch.float32, device=q.device)
    _need(states, "states", torch.float32)
    if tuple(states.shape) != (B, H, C, d * d + d) or states.device != q.device:
        raise ValueError(f"states must be [{B}, {H}, {C}, {d * d + d}] on q's device")
    out = _prepare_out(q, k, v, out, out_dtype)
    if state_in is not None:
        _need(state_in, "state_in", torch.float32)
        if tuple(state_in.shape) != (B, H, d * d + d) or state_in.device != q.device:
            raise ValueError("state_in must be [B, H, d*d + d] on q's device")
    return T, out, states


def blockcausal_forward(q, k, v, T, state_in=None, out=None, states=None, eps=DEFAULT_EPS,
                        out_dtype=torch.float32, kv_splits=0, readout_workgroups=0,
                        stage_events=None):
    """A whole sequence in the block-causal form: the N tokens of every (b, h)
    cut into C = ceil(N / T) blocks of T tokens; block n's queries read
    state_in + KV_1 + ... + KV_n.  Returns (out, states) with states
    [B, H, C, d*d + d] the state after every block (states[:, :, -1] is the
    state after the sequence).  state_in None means zeros."""
    T, out, states = _prepare_blockcausal(q, k, v, T, state_in, out, states, out_dtype)
    B, H, N, d = q.shape
    o = _opts(kv_splits, readout_workgroups, stage_events)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(state_in), _ptr(out), _ptr(states),
            B, H, N, T, d, _DTYPE[q.dtype], _DTYPE[out.dtype], float(eps))
    L_ = lib()
    if o is None:
        rc = L_.la_blockcausal_forward(*args, _stream(q.device))
    else:
        rc = L_.la_blockcausal_forward_ex(*args, ctypes.byref(o), _stream(q.device))
    _check(rc, "la_blockcausal_forward")
    return out, states


def chunk_forward_rope(q, k, v, state_in, frame0, grid_h, grid_w, theta=DEFAULT_THETA, out=None,
                       state_out=None, eps=DEFAULT_EPS, out_dtype=torch.float32):
    """chunk_forward with rotary position embedding on the numerator: token i
    of the block sits at frame frame0 + i // (grid_h grid_w), row
    (i // grid_w) % grid_h, column i % grid_w; the state's S holds keys
    turned by their absolute positions.  Returns (out, state_out)."""
    out, state_out = _prepare(q, k, v, out, out_dtype, state_out)
    _need(state_in, "state_in", torch.float32)
    if state_in.shape != state_out.shape or state_in.device != q.device:
        raise ValueError("state_in must match state_out's shape and device")
    B, H, L, d = q.shape
    rc = lib().la_chunk_forward_rope(
        _ptr(q), _ptr(k), _ptr(v), _ptr(state_in), _ptr(out), _ptr(state_out), B, H, L, d,
        _DTYPE[q.dtype], _DTYPE[out.dtype], float(eps), int(frame0), int(grid_h), int(grid_w),
        float(theta), _stream(q.device))
    _check(rc, "la_chunk_forward_rope")
    return out, state_out


def blockcausal_forward_rope(q, k, v, T, frame0, grid_h, grid_w, theta=DEFAULT_THETA,
                             state_in=None, out=None, states=None, eps=DEFAULT_EPS,
                             out_dtype=torch.float32, kv_splits=0, readout_workgroups=0,
                             stage_events=None):
    """blockcausal_forward with rotary position embedding on the numerator
    (positions as in chunk_forward_rope, counted over the whole sequence).
    With T >= N it is the global form (state_in None) or one block."""
    T, out, states = _prepare_blockcausal(q, k, v, T, state_in, out, states, out_dtype)
    B, H, N, d = q.shape
    o = _opts(kv_splits, readout_workgroups, stage_events)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(state_in), _ptr(out), _ptr(states),
            B, H, N, T, d, _DTYPE[q.dtype], _DTYPE[out.dtype], float(eps), int(frame0),
            int(grid_h), int(grid_w), float(theta))
    L_ = lib()
    if o is None:
        rc = L_.la_blockcausal_forward_rope(*args, _stream(q.device))
    else:
        rc = L_.la_blockcausal_forward_rope_ex(*args, ctypes.byref(o), _stream(q.device))
    _check(rc, "la_blockcausal_forward_rope")
    return out, states


def backward_workspace_size(B, H, N, T, d, in_dtype=torch.bfloat16):
    """Bytes of workspace a backward call needs (T = N for the chunk and
    global calls)."""
    z = ctypes.c_size_t()
    _check(lib().la_backward_workspace_size(B, H, N, max(int(T), 1), d, _DTYPE[in_dtype],
                                            ctypes.byref(z)), "la_backward_workspace_size")
    return z.value


def _prepare_grads(q, k, v, dout, dq, dk, dv):
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name)
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d]")
    _need(dout, "dout")
    if not (q.shape == k.shape == v.shape == dout.shape):
        raise ValueError("q, k, v, dout shapes differ")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPE:
        raise TypeError("q, k, v must share one dtype, float32 or bfloat16")
    if dout.dtype not in _DTYPE or dout.device != q.device:
        raise TypeError("dout must be float32 or bfloat16 on q's device")
    grads = []
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is None:
            t = torch.empty(q.shape, dtype=dout.dtype, device=q.device)
        _need(t, name, dout.dtype)
        if t.shape != q.shape or t.device != q.device:
            raise ValueError(f"{name} must be [B, H, N, d] on q's device")
        grads.append(t)
    return grads


def backward_stream_count(B, H, N, T, d, in_dtype=torch.bfloat16, rope=False):
    """Streams (1 or 2) a backward call of this shape (rope: the rotary
    backward) runs on when it may use two: the second half of its (b, h)
    pairs goes to the library's second stream, joined back before the call's
    work completes on the caller's."""
    c = ctypes.c_int()
    _check(lib().la_backward_stream_count(B, H, N, max(int(T), 1), d, _DTYPE[in_dtype],
                                          int(bool(rope)), ctypes.byref(c)),
           "la_backward_stream_count")
    return c.value


def backward_plan(B, H, N, T, d, in_dtype=torch.bfloat16, rope=False, query_splits=0,
                  key_workgroups=0, workspace_bytes=0):
    """The launch shape (a dict of la_backward_shape's fields) a backward call
    of this shape would use on one stream; query_splits and key_workgroups
    are the launch requests (0: the library's choice), workspace_bytes the
    workspace it is given (0: as much as it needs)."""
    sh = BackwardShape()
    _check(lib().la_backward_plan(B, H, N, max(int(T), 1), d, _DTYPE[in_dtype], int(bool(rope)),
                                  int(query_splits), int(key_workgroups), int(workspace_bytes),
                                  ctypes.byref(sh)), "la_backward_plan")
    return {name: getattr(sh, name) for name, _ in BackwardShape._fields_}


def _workspace(workspace, need, device):
    if workspace is None:
        return torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    _need(workspace, "workspace")
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds fewer than {need} bytes")
    return workspace


def _state_like(t, shape, name, device):
    _need(t, name, torch.float32)
    if tuple(t.shape) != tuple(shape) or t.device != device:
        raise ValueError(f"{name} must be {list(shape)} on q's device")


def blockcausal_backward(q, k, v, states, dout, T, dstates=None, want_dstate_in=False,
                         eps=DEFAULT_EPS, dq=None, dk=None, dv=None, dstate_in=None,
                         workspace=None, kv_splits=0, readout_workgroups=0,
                         stage_events=None):
    """Gradients of blockcausal_forward(q, k, v, T, ...) for the upstream
    gradient dout (and dstates, the gradient of the returned states, or
    None).  `states` is what the forward returned.  Returns
    (dq, dk, dv, dstate_in) with dstate_in the gradient of the forward's
    state_in ([B, H, d*d + d], or None unless asked for)."""
    dq, dk, dv = _prepare_grads(q, k, v, dout, dq, dk, dv)
    B, H, N, d = q.shape
    T = int(T)
    if T < 1:
        raise ValueError("T must be >= 1")
    C = -(-N // T) if N > 0 else 0
    _state_like(states, (B, H, C, d * d + d), "states", q.device)
    if dstates is not None:
        _state_like(dstates, (B, H, C, d * d + d), "dstates", q.device)
    if want_dstate_in and dstate_in is None:
        dstate_in = torch.empty((B, H, d * d + d), dtype=torch.float32, device=q.device)
    if dstate_in is not None:
        _state_like(dstate_in, (B, H, d * d + d), "dstate_in", q.device)
    need = backward_workspace_size(B, H, N, T, d, q.dtype)
    workspace = _workspace(workspace, need, q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    o = _opts(kv_splits, readout_workgroups, stage_events)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(states), _ptr(dout), _ptr(dstates), _ptr(dq),
            _ptr(dk), _ptr(dv), _ptr(dstate_in), B, H, N, T, d, _DTYPE[q.dtype],
            _DTYPE[dout.dtype], float(eps), _ptr(workspace), ws_bytes)
    L_ = lib()
    if o is None:
        rc = L_.la_blockcausal_backward(*args, _stream(q.device))
    else:
        rc = L_.la_blockcausal_backward_ex(*args, ctypes.byref(o), _stream(q.device))
    _check(rc, "la_blockcausal_backward")
    return dq, dk, dv, dstate_in


def blockcausal_backward_noalloc(q, k, v, states, dout, T, dstates=None, want_dstate_in=False,
                                 eps=DEFAULT_EPS, dq=None, dk=None, dv=None, dstate_in=None):
    """blockcausal_backward through la_blockcausal_backward_noalloc: the
    library's static device scratch instead of a workspace (the library
    allocates nothing; pass dq, dk, dv (and dstate_in) to allocate nothing
    here either).  Calls that overlap in time on one GPU race."""
    dq, dk, dv = _prepare_grads(q, k, v, dout, dq, dk, dv)
    B, H, N, d = q.shape
    T = int(T)
    if T < 1:
        raise ValueError("T must be >= 1")
    C = -(-N // T) if N > 0 else 0
    _state_like(states, (B, H, C, d * d + d), "states", q.device)
    if dstates is not None:
        _state_like(dstates, (B, H, C, d * d + d), "dstates", q.device)
    if want_dstate_in and dstate_in is None:
        dstate_in = torch.empty((B, H, d * d + d), dtype=torch.float32, device=q.device)
    if dstate_in is not None:
        _state_like(dstate_in, (B, H, d * d + d), "dstate_in", q.device)
    rc = lib().la_blockcausal_backward_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(states), _ptr(dout), _ptr(dstates), _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(dstate_in), B, H, N, T, d, _DTYPE[q.dtype], _DTYPE[dout.dtype], float(eps),
        _stream(q.device))
    _check(rc, "la_blockcausal_backward_noalloc")
    return dq, dk, dv, dstate_in


def blockcausal_backward_rope(q, k, v, states, dout, T, frame0, grid_h, grid_w,
                              theta=DEFAULT_THETA, dstates=None, want_dstate_in=False,
                              eps=DEFAULT_EPS, dq=None, dk=None, dv=None, dstate_in=None,
                              workspace=None, kv_splits=0, readout_workgroups=0,
                              stage_events=None):
    """Gradients of blockcausal_forward_rope(q, k, v, T, frame0, grid_h,
    grid_w, theta, ...) for the upstream gradient dout (and dstates, the
    gradient of the returned states, or None).  Returns (dq, dk, dv,
    dstate_in) as blockcausal_backward; launch options as there."""
    dq, dk, dv = _prepare_grads(q, k, v, dout, dq, dk, dv)
    B, H, N, d = q.shape
    T = int(T)
    if T < 1:
        raise ValueError("T must be >= 1")
    C = -(-N // T) if N > 0 else 0
    _state_like(states, (B, H, C, d * d + d), "states", q.device)
    if dstates is not None:
        _state_like(dstates, (B, H, C, d * d + d), "dstates", q.device)
    if want_dstate_in and dstate_in is None:
        dstate_in = torch.empty((B, H, d * d + d), dtype=torch.float32, device=q.device)
    if dstate_in is not None:
        _state_like(dstate_in, (B, H, d * d + d), "dstate_in", q.device)
    need = backward_workspace_size(B, H, N, T, d, q.dtype)
    workspace = _workspace(workspace, need, q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    o = _opts(kv_splits, readout_workgroups, stage_events)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(states), _ptr(dout), _ptr(dstates), _ptr(dq),
            _ptr(dk), _ptr(dv), _ptr(dstate_in), B, H, N, T, d, _DTYPE[q.dtype],
            _DTYPE[dout.dtype], float(eps), _ptr(workspace), ws_bytes, int(frame0), int(grid_h),
            int(grid_w), float(theta))
    L_ = lib()
    if o is None:
        rc = L_.la_blockcausal_backward_rope(*args, _stream(q.device))
    else:
        rc = L_.la_blockcausal_backward_rope_ex(*args, ctypes.byref(o), _stream(q.device))
    _check(rc, "la_blockcausal_backward_rope")
    return dq, dk, dv, dstate_in


def chunk_backward(q, k, v, state_out, dout, dstate_out=None, want_dstate_in=True,
                   eps=DEFAULT_EPS, dq=None, dk=None, dv=None, dstate_in=None, workspace=None):
    """Gradients of chunk_forward(q, k, v, state_in) -> (out, state_out) for
    the upstream gradients dout and dstate_out (None: zero).  Returns
    (dq, dk, dv, dstate_in)."""
    dq, dk, dv = _prepare_grads(q, k, v, dout, dq, dk, dv)
    B, H, L, d = q.shape
    _state_like(state_out, (B, H, d * d + d), "state_out", q.device)
    if dstate_out is not None:
        _state_like(dstate_out, (B, H, d * d + d), "dstate_out", q.device)
    if want_dstate_in and dstate_in is None:
        dstate_in = torch.empty((B, H, d * d + d), dtype=torch.float32, device=q.device)
    if dstate_in is not None:
        _state_like(dstate_in, (B, H, d * d + d), "dstate_in", q.device)
    need = backward_workspace_size(B, H, L, L, d, q.dtype)
    workspace = _workspace(workspace, need, q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().la_chunk_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(state_out), _ptr(dout), _ptr(dstate_out), _ptr(dq),
        _ptr(dk), _ptr(dv), _ptr(dstate_in), B, H, L, d, _DTYPE[q.dtype], _DTYPE[dout.dtype],
        float(eps), _ptr(workspace), ws_bytes, _stream(q.device)), "la_chunk_backward")
    return dq, dk, dv, dstate_in


def chunk_backward_rope(q, k, v, state_out, dout, frame0, grid_h, grid_w, theta=DEFAULT_THETA,
                        dstate_out=None, want_dstate_in=True, eps=DEFAULT_EPS, dq=None, dk=None,
                        dv=None, dstate_in=None, workspace=None):
    """Gradients of chunk_forward_rope(q, k, v, state_in, frame0, grid_h,
    grid_w, theta) -> (out, state_out) for the upstream gradients dout and
    dstate_out (None: zero).  Returns (dq, dk, dv, dstate_in)."""
    dq, dk, dv = _prepare_grads(q, k, v, dout, dq, dk, dv)
    B, H, L, d = q.shape
    _state_like(state_out, (B, H, d * d + d), "state_out", q.device)
    if dstate_out is not None:
        _state_like(dstate_out, (B, H, d * d + d), "dstate_out", q.device)
    if want_dstate_in and dstate_in is None:
        dstate_in = torch.empty((B, H, d * d + d), dtype=torch.float32, device=q.device)
    if dstate_in is not None:
        _state_like(dstate_in, (B, H, d * d + d), "dstate_in", q.device)
    need = backward_workspace_size(B, H, L, L, d, q.dtype)
    workspace = _workspace(workspace, need, q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().la_chunk_backward_rope(
        _ptr(q), _ptr(k), _ptr(v), _ptr(state_out), _ptr(dout), _ptr(dstate_out), _ptr(dq),
        _ptr(dk), _ptr(dv), _ptr(dstate_in), B, H, L, d, _DTYPE[q.dtype], _DTYPE[dout.dtype],
        float(eps), _ptr(workspace), ws_bytes, int(frame0), int(grid_h), int(grid_w),
        float(theta), _stream(q.device)), "la_chunk_backward_rope")
    return dq, dk, dv, dstate_in


def global_backward_rope(q, k, v, state, dout, frame0, grid_h, grid_w, theta=DEFAULT_THETA,
                         eps=DEFAULT_EPS, dq=None, dk=None, dv=None, workspace=None):
    """Gradients of global_forward_rope(q, k, v, frame0, grid_h, grid_w,
    theta) -> (out, state) for the upstream gradient dout.  Returns
    (dq, dk, dv)."""
    dq, dk, dv = _prepare_grads(q, k, v, dout, dq, dk, dv)
    B, H, N, d = q.shape
    _state_like(state, (B, H, d * d + d), "state", q.device)
    need = backward_workspace_size(B, H, N, N, d, q.dtype)
    workspace = _workspace(workspace, need, q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().la_global_backward_rope(
        _ptr(q), _ptr(k), _ptr(v), _ptr(state), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        B, H, N, d, _DTYPE[q.dtype], _DTYPE[dout.dtype], float(eps), _ptr(workspace), ws_bytes,
        int(frame0), int(grid_h), int(grid_w), float(theta), _stream(q.device)),
        "la_global_backward_rope")
    return dq, dk, dv


def global_backward(q, k, v, state, dout, eps=DEFAULT_EPS, dq=None, dk=None, dv=None,
                    workspace=None):
    """Gradients of global_forward(q, k, v) -> (out, state) for the upstream
    gradient dout.  Returns (dq, dk, dv)."""
    dq, dk, dv = _prepare_grads(q, k, v, dout, dq, dk, dv)
    B, H, N, d = q.shape
    _state_like(state, (B, H, d * d + d), "state", q.device)
    need = backward_workspace_size(B, H, N, N, d, q.dtype)
    workspace = _workspace(workspace, need, q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().la_global_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(state), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        B, H, N, d, _DTYPE[q.dtype], _DTYPE[dout.dtype], float(eps), _ptr(workspace), ws_bytes,
        _stream(q.device)), "la_global_backward")
    return dq, dk, dv


class _BlockCausalFunction(torch.autograd.Function):
    """Autograd glue: the forward is blockcausal_forward (or
    blockcausal_forward_rope), the backward blockcausal_backward (or
    blockcausal_backward_rope), all library calls; nothing is computed
    here."""

    @staticmethod
    def forward(ctx, q, k, v, state_in, T, eps, rope):
        if rope is None:
            out, states = blockcausal_forward(q, k, v, T, state_in=state_in, eps=eps)
        else:
            out, states = blockcausal_forward_rope(q, k, v, T, *rope, state_in=state_in, eps=eps)
        ctx.save_for_backward(q, k, v, states)
        ctx.T, ctx.eps, ctx.rope, ctx.has_state_in = T, eps, rope, state_in is not None
        return out, states

    @staticmethod
    def backward(ctx, dout, dstates):
        q, k, v, states = ctx.saved_tensors
        if dout is None:
            dout = torch.zeros(q.shape, dtype=torch.float32, device=q.device)
        dout = dout.contiguous()
        if dout.dtype not in _DTYPE:
            dout = dout.float()
        if dstates is not None:
            dstates = dstates.contiguous().float()
        if ctx.rope is None:
            dq, dk, dv, dsi = blockcausal_backward(q, k, v, states, dout, ctx.T,
                                                   dstates=dstates,
                                                   want_dstate_in=ctx.has_state_in, eps=ctx.eps)
        else:
            dq, dk, dv, dsi = blockcausal_backward_rope(q, k, v, states, dout, ctx.T, *ctx.rope,
                                                        dstates=dstates,
                                                        want_dstate_in=ctx.has_state_in,
                                                        eps=ctx.eps)
        return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), dsi, None, None, None


def linear_attention(q, k, v, T=None, state_in=None, eps=DEFAULT_EPS, rope=None):
    """Differentiable block-causal linear attention (torch autograd).

    q, k, v [B, H, N, d] (float32 or bfloat16, contiguous, on one GPU); the N
    tokens of every (b, h) are cut into blocks of T tokens (None: one block,
    the global form).  state_in [B, H, d*d + d] float32 or None.  rope: None,
    or (frame0, grid_h, grid_w) or (frame0, grid_h, grid_w, theta) for the
    rotary form (blockcausal_forward_rope).  Returns (out [B, H, N, d]
    float32, states [B, H, C, d*d + d]); gradients flow to q, k, v and
    state_in through la_blockcausal_backward (la_blockcausal_backward_rope),
    including gradients that reach the returned states."""
    N = q.shape[2]
    T = max(int(T if T is not None else N), 1)
    if rope is not None:
        rope = tuple(rope)
        if len(rope) not in (3, 4):
            raise ValueError("rope must be (frame0, grid_h, grid_w[, theta])")
        theta = float(rope[3]) if len(rope) == 4 else DEFAULT_THETA
        rope = (int(rope[0]), int(rope[1]), int(rope[2]), theta)
    return _BlockCausalFunction.apply(q, k, v, state_in, T, float(eps), rope)


def _prepare_tconv(x, weight, bias, cache_in, y, cache_out, out_dtype, want_cache):
    _need(x, "x")
    if x.dim() != 4 or x.dtype not in _DTYPE:
        raise ValueError("x must be [B, F, P, C], float32 or bfloat16")
    B, F, P, C = x.shape
    _need(weight, "weight", torch.float32)
    if tuple(weight.shape) != (C, 3) or weight.device != x.device:
        raise ValueError(f"weight must be [{C}, 3] float32 on x's device")
    if bias is not None:
        _need(bias, "bias", torch.float32)
        if tuple(bias.shape) != (C,) or bias.device != x.device:
            raise ValueError(f"bias must be [{C}] float32 on x's device")
    for name, t in (("cache_in", cache_in), ("cache_out", cache_out)):
        if t is not None:
            _need(t, name, x.dtype)
            if tuple(t.shape) != (B, P, C) or t.device != x.device:
                raise ValueError(f"{name} must be [{B}, {P}, {C}] {x.dtype} on x's device")
    if y is None:
        y = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    _need(y, "y")
    if y.shape != x.shape or y.dtype not in _DTYPE or y.device != x.device:
        raise ValueError("y must be [B, F, P, C], float32 or bfloat16, on x's device")
    if cache_out is None and want_cache:
        cache_out = torch.empty((B, P, C), dtype=x.dtype, device=x.device)
    return y, cache_out


def temporal_conv_chunk(x, weight, bias=None, cache_in=None, y=None, cache_out=None,
                        out_dtype=None, want_cache=True):
    """One chunk of the Mix-FFN's depthwise 3x1x1 temporal convolution with
    its one-frame cache: x [B, F, P, C], weight [C, 3] (taps f-1, f, f+1),
    bias [C] or None, cache_in [B, P, C] (None: zeros).  Returns
    (y, cache_out) with cache_out the chunk's last frame; cache_out may be
    cache_in."""
    y, cache_out = _prepare_tconv(x, weight, bias, cache_in, y, cache_out, out_dtype, want_cache)
    B, F, P, C = x.shape
    _check(lib().la_temporal_conv_chunk(
        _ptr(x), _ptr(cache_in), _ptr(weight), _ptr(bias), _ptr(y), _ptr(cache_out), B, F, P, C,
        _DTYPE[x.dtype], _DTYPE[y.dtype], _stream(x.device)), "la_temporal_conv_chunk")
    return y, cache_out


def temporal_conv_blockcausal(x, weight, Tf, bias=None, cache_in=None, y=None, cache_out=None,
                              out_dtype=None, want_cache=True):
    """A whole sequence of F frames in chunks of Tf frames: the chunk call
    over the chunks in order with the cache carried.  Returns
    (y, cache_out)."""
    y, cache_out = _prepare_tconv(x, weight, bias, cache_in, y, cache_out, out_dtype, want_cache)
    B, F, P, C = x.shape
    _check(lib().la_temporal_conv_blockcausal(
        _ptr(x), _ptr(cache_in), _ptr(weight), _ptr(bias), _ptr(y), _ptr(cache_out), B, F,
        int(Tf), P, C, _DTYPE[x.dtype], _DTYPE[y.dtype], _stream(x.device)),
        "la_temporal_conv_blockcausal")
    return y, cache_out


def plan(B, H, L, d, in_dtype=torch.bfloat16, out_dtype=torch.float32, kv_splits=0,
         readout_workgroups=0):
    """(kv_splits, readout_workgroups) the library would use."""
    s, t = ctypes.c_int(), ctypes.c_int()
    _check(lib().la_plan(B, H, L, d, _DTYPE[in_dtype], _DTYPE[out_dtype], int(kv_splits),
                         int(readout_workgroups), ctypes.byref(s), ctypes.byref(t)), "la_plan")
    return s.value, t.value


def abi_version():
    return lib().la_abi_version()


# ---------------------------------------------------------------------------
# HIP events for per-stage timing (plumbing over libamdhip64).

_hip = None


def _hiplib():
    global _hip
    if _hip is None:
        h = ctypes.CDLL("libamdhip64.so")
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                          ctypes.c_void_p]
        h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        _hip = h
    return _hip


# hipEventDisableSystemFence from HIP's runtime header: the event takes its time stamp without
# the system-scope cache write-back and invalidate of a default event, which would otherwise
# lengthen the interval of the kernel after it.  These events only time; they order nothing.
_HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class StageEvents:
    """Four HIP events that a forward call records around its stages:
    [before KV reduction, before split reduce, before readout, after]."""

    def __init__(self):
        h = _hiplib()
        self._arr = (ctypes.c_void_p * 4)()
        for i in range(4):
            ev = ctypes.c_void_p()
            if h.hipEventCreateWithFlags(ctypes.byref(ev), _HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self._arr[i] = ev.value

    def as_ctypes(self):
        return ctypes.cast(self._arr, ctypes.POINTER(ctypes.c_void_p))

    def elapsed_ms(self):
        """(kv, reduce, readout) milliseconds of the last recorded call."""
        h = _hiplib()
        if h.hipEventSynchronize(self._arr[3]) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        out = []
        for i in range(3):
            ms = ctypes.c_float()
            if h.hipEventElapsedTime(ctypes.byref(ms), self._arr[i], self._arr[i + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append(ms.value)
        return tuple(out)

    def close(self):
        h = _hiplib()
        for i in range(4):
            if self._arr[i]:
                h.hipEventDestroy(self._arr[i])
                self._arr[i] = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
