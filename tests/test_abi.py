"""C-ABI contract tests that need no GPU: the library loads, exports every
function include/linattn.h declares, and rejects bad arguments before it
enqueues anything (every call here fails validation, so no HIP call is
made and the fake pointers are never dereferenced)."""

import ctypes
import os
import re

import pytest
import torch

import block_causal_linear_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linattn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(la.LIB_PATH),
                                reason="liblinattn.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(la_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"la_state_reset", "la_chunk_forward", "la_global_forward"} <= set(names)
    lib = ctypes.CDLL(la.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(la.EXPORTS)


def test_version_and_status_strings():
    assert la.abi_version() == 13
    for code in range(7):
        assert la._status_string(code) != "unknown status"
    assert la._status_string(99) == "unknown status"


A = 1 << 20  # fake, 16-byte aligned addresses; never dereferenced
BF16, F32 = la.LA_BF16, la.LA_F32


def chunk(q=A, k=2 * A, v=3 * A, si=4 * A, out=5 * A, so=6 * A, B=1, H=2, L=64, d=64,
          idt=BF16, odt=F32, eps=1e-6):
    return la.lib().la_chunk_forward(q, k, v, si, out, so, B, H, L, d, idt, odt, eps, None)


def glob(q=A, k=2 * A, v=3 * A, out=5 * A, so=6 * A, B=1, H=2, N=64, d=64, idt=BF16, odt=F32,
         eps=1e-6):
    return la.lib().la_global_forward(q, k, v, out, so, B, H, N, d, idt, odt, eps, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), la.LA_E_INVAL),
    (dict(H=-1), la.LA_E_INVAL),
    (dict(L=-5), la.LA_E_INVAL),
    (dict(B=70000), la.LA_E_INVAL),
    (dict(L=1 << 26, d=64), la.LA_E_INVAL),
    (dict(d=48), la.LA_E_UNSUPPORTED),
    (dict(d=256), la.LA_E_UNSUPPORTED),
    (dict(idt=7), la.LA_E_UNSUPPORTED),
    (dict(odt=3), la.LA_E_UNSUPPORTED),
    (dict(eps=-1.0), la.LA_E_INVAL),
    (dict(eps=float("nan")), la.LA_E_INVAL),
    (dict(eps=float("inf")), la.LA_E_INVAL),
    (dict(q=None), la.LA_E_INVAL),
    (dict(v=None), la.LA_E_INVAL),
    (dict(out=None), la.LA_E_INVAL),
    (dict(si=None), la.LA_E_INVAL),
    (dict(so=None), la.LA_E_INVAL),
    (dict(q=A + 8), la.LA_E_ALIGN),
    (dict(out=5 * A + 4), la.LA_E_ALIGN),
    (dict(so=6 * A + 2), la.LA_E_ALIGN),
    (dict(out=A), la.LA_E_ALIAS),                 # out == q
    (dict(out=2 * A + 4096), la.LA_E_ALIAS),      # out overlaps k
    (dict(so=3 * A + 256), la.LA_E_ALIAS),        # state_out inside v
    (dict(so=5 * A + 1024), la.LA_E_ALIAS),       # state_out inside out
    (dict(si=5 * A), la.LA_E_ALIAS),              # state_in inside out
    (dict(si=6 * A + 16), la.LA_E_ALIAS),         # partial state overlap
])
def test_chunk_rejects(kw, code):
    assert chunk(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(N=-1), la.LA_E_INVAL),
    (dict(d=16), la.LA_E_UNSUPPORTED),
    (dict(k=None), la.LA_E_INVAL),
    (dict(so=None), la.LA_E_INVAL),
    (dict(k=2 * A + 4), la.LA_E_ALIGN),
    (dict(out=3 * A), la.LA_E_ALIAS),
])
def test_global_rejects(kw, code):
    assert glob(**kw) == code


def rope_chunk(q=A, k=2 * A, v=3 * A, si=4 * A, out=5 * A, so=6 * A, B=1, H=2, L=64, d=64,
               idt=BF16, odt=F32, eps=1e-6, f0=0, gh=4, gw=4, theta=10000.0):
    return la.lib().la_chunk_forward_rope(q, k, v, si, out, so, B, H, L, d, idt, odt, eps, f0,
                                          gh, gw, theta, None)


def rope_bc(q=A, k=2 * A, v=3 * A, si=4 * A, out=5 * A, sts=6 * A, B=1, H=2, N=640, T=64, d=64,
            idt=BF16, odt=F32, eps=1e-6, f0=0, gh=4, gw=4, theta=10000.0):
    return la.lib().la_blockcausal_forward_rope(q, k, v, si, out, sts, B, H, N, T, d, idt, odt,
                                                eps, f0, gh, gw, theta, None)


@pytest.mark.parametrize("kw,code", [
    (dict(gh=0), la.LA_E_INVAL),
    (dict(gw=-2), la.LA_E_INVAL),
    (dict(gh=4096, gw=1024), la.LA_E_INVAL),        # 2^22 tokens per frame
    (dict(theta=0.0), la.LA_E_INVAL),
    (dict(theta=-1.0), la.LA_E_INVAL),
    (dict(theta=float("nan")), la.LA_E_INVAL),
    (dict(theta=float("inf")), la.LA_E_INVAL),
    (dict(f0=1 << 22), la.LA_E_INVAL),
    (dict(f0=-(1 << 22)), la.LA_E_INVAL),
    (dict(L=(1 << 22) - 64), la.LA_E_INVAL),
    (dict(d=48), la.LA_E_UNSUPPORTED),
    (dict(si=None), la.LA_E_INVAL),
    (dict(q=A + 8), la.LA_E_ALIGN),
    (dict(out=A), la.LA_E_ALIAS),
    (dict(eps=-1.0), la.LA_E_INVAL),
])
def test_rope_chunk_rejects(kw, code):
    assert rope_chunk(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(T=0), la.LA_E_INVAL),
    (dict(gw=0), la.LA_E_INVAL),
    (dict(theta=float("nan")), la.LA_E_INVAL),
    (dict(N=1 << 22), la.LA_E_INVAL),
    (dict(si=6 * A), la.LA_E_ALIAS),
    (dict(idt=5), la.LA_E_UNSUPPORTED),
])
def test_rope_blockcausal_rejects(kw, code):
    assert rope_bc(**kw) == code


def bc(q=A, k=2 * A, v=3 * A, si=4 * A, out=5 * A, sts=6 * A, B=1, H=2, N=640, T=64, d=64,
       idt=BF16, odt=F32, eps=1e-6):
    return la.lib().la_blockcausal_forward(q, k, v, si, out, sts, B, H, N, T, d, idt, odt, eps,
                                           None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=0), la.LA_E_INVAL),
    (dict(T=-3), la.LA_E_INVAL),
    (dict(N=-1), la.LA_E_INVAL),
    (dict(sts=None), la.LA_E_INVAL),
    (dict(d=96), la.LA_E_UNSUPPORTED),
    (dict(si=4 * A + 8), la.LA_E_ALIGN),
    (dict(si=6 * A + 16640 * 3), la.LA_E_ALIAS),   # state_in inside states (block 3 of head 0)
    (dict(si=6 * A), la.LA_E_ALIAS),               # with several blocks even equal is illegal
    (dict(out=6 * A + 64), la.LA_E_ALIAS),         # out overlaps states
    (dict(sts=3 * A + 1024), la.LA_E_ALIAS),       # states inside v
])
def test_blockcausal_rejects(kw, code):
    assert bc(**kw) == code


def test_blockcausal_empty_is_a_no_op():
    # N = 0: no blocks, nothing is written or launched (fake pointers are fine)
    assert bc(N=0, q=None, k=None, v=None, out=None) == la.LA_OK


def test_state_reset_rejects():
    f = la.lib().la_state_reset
    assert f(None, 1, 1, 64, None) == la.LA_E_INVAL
    assert f(A, 0, 1, 64, None) == la.LA_E_INVAL
    assert f(A, 1, 1, 40, None) == la.LA_E_UNSUPPORTED
    assert f(A + 4, 1, 1, 64, None) == la.LA_E_ALIGN


def test_plan_shapes():
    # the 720p chunk: 32 heads -> 16 splits of 4736 tokens
    s, t = la.plan(1, 32, 75600, 64)
    assert s == 16
    # tiny chunks write the state directly from the KV kernel
    assert la.plan(1, 2, 64, 32, in_dtype=la.torch.float32)[0] == 1
    # requests are clamped to the tile count and to the scratch in `out`
    assert la.plan(1, 1, 100, 64, kv_splits=50)[0] == 1
    assert la.plan(1, 1, 6400, 64, kv_splits=7)[0] == 7
    assert la.plan(1, 1, 0, 64)[0] == 0
    # readout: the sweep grid (512 workgroups) at 720p; a request is honoured
    # up to one workgroup per 128-token unit
    assert la.plan(1, 32, 75600, 64)[1] == 512
    assert la.plan(1, 32, 75600, 64, readout_workgroups=300)[1] == 300
    assert la.plan(1, 1, 100, 64, readout_workgroups=300)[1] == 1
    # d = 128 reads out over persistent work items of at least 1,024 tokens:
    # 64 heads x 4 items = 256 workgroups; a request sets the item count (up
    # to the resident grid of 512); float32 inputs keep per-head workgroups
    # (512 at d = 128: 8 per head here).  One chunk at d = 128 over 64 heads
    # takes the quadrant KV kernel: one "split".
    assert la.plan(4, 16, 4096, 128) == (1, 256)
    assert la.plan(4, 16, 4096, 128, readout_workgroups=2048)[1] == 512
    assert la.plan(4, 16, 4096, 128, kv_splits=4)[0] == 4  # a request keeps the splits
    assert la.plan(2, 16, 4096, 128)[0] > 1                # 32 heads: token splits
    assert la.plan(4, 16, 40 * 4096, 128)[1] == 512
    assert la.plan(4, 16, 4096, 128, in_dtype=la.torch.float32)[1] == 4 * 16 * 8
    with pytest.raises(la.LinAttnError):
        la.plan(1, 1, 10, 48)


def bwd(q=A, k=2 * A, v=3 * A, sts=4 * A, do=5 * A, dsts=None, dq=6 * A, dk=7 * A, dv=8 * A,
        dsi=None, B=1, H=2, N=640, T=64, d=64, idt=BF16, gdt=F32, eps=1e-6, ws=9 * A,
        wsb=1 << 20):
    return la.lib().la_blockcausal_backward(q, k, v, sts, do, dsts, dq, dk, dv, dsi, B, H, N, T,
                                            d, idt, gdt, eps, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=0), la.LA_E_INVAL),
    (dict(N=-2), la.LA_E_INVAL),
    (dict(eps=-1e-3), la.LA_E_INVAL),
    (dict(d=48), la.LA_E_UNSUPPORTED),
    (dict(gdt=5), la.LA_E_UNSUPPORTED),
    (dict(idt=2), la.LA_E_UNSUPPORTED),
    (dict(q=None), la.LA_E_INVAL),
    (dict(do=None), la.LA_E_INVAL),
    (dict(sts=None), la.LA_E_INVAL),
    (dict(dv=None), la.LA_E_INVAL),
    (dict(ws=None), la.LA_E_INVAL),                # workspace needed
    (dict(wsb=1024), la.LA_E_INVAL),               # workspace too small
    (dict(dq=6 * A + 8), la.LA_E_ALIGN),
    (dict(ws=9 * A + 4), la.LA_E_ALIGN),
    (dict(dq=A), la.LA_E_ALIAS),                   # dq == q
    (dict(dk=5 * A + 512), la.LA_E_ALIAS),         # dk inside dout
    (dict(dv=7 * A + 64), la.LA_E_ALIAS),          # dv overlaps dk
    (dict(ws=8 * A + 4096), la.LA_E_ALIAS),        # workspace overlaps dv
    (dict(dsi=4 * A + 16640), la.LA_E_ALIAS),      # dstate_in inside states
    (dict(dsi=9 * A), la.LA_E_ALIAS),              # dstate_in inside the workspace
])
def test_backward_rejects(kw, code):
    assert bwd(**kw) == code


def rope_bwd(q=A, k=2 * A, v=3 * A, sts=4 * A, do=5 * A, dsts=None, dq=6 * A, dk=7 * A,
             dv=8 * A, dsi=None, B=1, H=2, N=640, T=64, d=64, idt=BF16, gdt=F32, eps=1e-6,
             ws=9 * A, wsb=1 << 20, f0=0, gh=4, gw=4, theta=10000.0, ex=False):
    args = (q, k, v, sts, do, dsts, dq, dk, dv, dsi, B, H, N, T, d, idt, gdt, eps, ws, wsb, f0,
            gh, gw, theta)
    if ex:
        return la.lib().la_blockcausal_backward_rope_ex(*args, None, None)
    return la.lib().la_blockcausal_backward_rope(*args, None)


@pytest.mark.parametrize("ex", [False, True])
@pytest.mark.parametrize("kw,code", [
    (dict(gh=0), la.LA_E_INVAL),
    (dict(gw=-1), la.LA_E_INVAL),
    (dict(theta=0.0), la.LA_E_INVAL),
    (dict(theta=float("nan")), la.LA_E_INVAL),
    (dict(f0=1 << 22), la.LA_E_INVAL),
    (dict(N=1 << 22), la.LA_E_INVAL),
    (dict(T=0), la.LA_E_INVAL),
    (dict(d=48), la.LA_E_UNSUPPORTED),
    (dict(ws=None), la.LA_E_INVAL),
    (dict(dq=6 * A + 8), la.LA_E_ALIGN),
    (dict(dk=5 * A + 512), la.LA_E_ALIAS),
])
def test_rope_backward_rejects(kw, code, ex):
    assert rope_bwd(ex=ex, **kw) == code


def test_rope_global_rejects():
    L_ = la.lib()

    def call(out=5 * A, so=6 * A, gh=4, N=640, d=64, f0=0):
        return L_.la_global_forward_rope(A, 2 * A, 3 * A, out, so, 1, 2, N, d, BF16, F32, 1e-6,
                                         f0, gh, 4, 10000.0, None)
    assert call(so=None) == la.LA_E_INVAL
    assert call(gh=0) == la.LA_E_INVAL
    assert call(f0=1 << 22) == la.LA_E_INVAL
    assert call(d=96) == la.LA_E_UNSUPPORTED
    assert call(out=A) == la.LA_E_ALIAS


def test_rope_global_backward_rejects():
    L_ = la.lib()

    def call(st=4 * A, gh=4, N=640, d=64):
        return L_.la_global_backward_rope(A, 2 * A, 3 * A, st, 5 * A, 6 * A, 7 * A, 8 * A, 1, 2,
                                          N, d, BF16, F32, 1e-6, 9 * A, 1 << 20, 0, gh, 4,
                                          10000.0, None)
    assert call(st=None) == la.LA_E_INVAL
    assert call(gh=-1) == la.LA_E_INVAL
    assert call(d=48) == la.LA_E_UNSUPPORTED


def test_rope_chunk_backward_rejects():
    L_ = la.lib()

    def call(so=4 * A, gh=4, theta=10000.0, L=64, d=64):
        return L_.la_chunk_backward_rope(A, 2 * A, 3 * A, so, 5 * A, None, 6 * A, 7 * A, 8 * A,
                                         None, 1, 2, L, d, BF16, F32, 1e-6, 9 * A, 1 << 20, 0,
                                         gh, 4, theta, None)
    assert call(so=None) == la.LA_E_INVAL          # the chunk call needs state_out
    assert call(gh=0) == la.LA_E_INVAL
    assert call(theta=float("nan")) == la.LA_E_INVAL
    assert call(L=-1) == la.LA_E_INVAL
    assert call(d=40) == la.LA_E_UNSUPPORTED


def test_sizes_beyond_one_gpu_rejected():
    """Shapes whose tensors reach 2^40 bytes are rejected before anything is
    enqueued (the pointers here are not device memory)."""
    L_ = la.lib()
    # 65535 x 65535 heads of 64 tokens: 2^44 bytes of q alone
    assert chunk(B=65535, H=65535, L=64) == la.LA_E_INVAL
    assert bc(B=65535, H=2, N=1 << 24, T=1 << 20) == la.LA_E_INVAL
    # one-token blocks: the states of 2^23 blocks x 16 heads at d = 128 are 8.9e12 bytes
    assert bc(B=1, H=16, N=1 << 23, T=1, d=128) == la.LA_E_INVAL
    assert bwd(B=65535, H=65535, N=64) == la.LA_E_INVAL
    assert rope_bwd(B=65535, H=65535, N=64) == la.LA_E_INVAL
    z = ctypes.c_size_t()
    assert L_.la_backward_workspace_size(65535, 65535, 64, 64, 64, BF16,
                                         ctypes.byref(z)) == la.LA_E_INVAL
    k = ctypes.c_int()
    assert L_.la_plan(65535, 65535, 64, 64, BF16, F32, 0, 0, ctypes.byref(k),
                      ctypes.byref(k)) == la.LA_E_INVAL
    assert L_.la_state_reset(A, 70000, 1, 64, None) == la.LA_E_INVAL
    assert L_.la_temporal_conv_chunk(A, None, 2 * A, None, 3 * A, None, 1, 1 << 20, 1 << 20,
                                     1024, BF16, BF16, None) == la.LA_E_INVAL
    # below the limit (states 5.5e11 bytes) the call gets past the size check
    # to the alignment check
    assert bc(B=1, H=8, N=1 << 20, T=1, d=128, q=A + 8) == la.LA_E_ALIGN


def test_backward_entry_points_reject():
    L_ = la.lib()
    # the chunk call needs state_out; the global call rejects a bad d
    assert L_.la_chunk_backward(A, 2 * A, 3 * A, None, 5 * A, None, 6 * A, 7 * A, 8 * A, None,
                                1, 2, 64, 64, BF16, F32, 1e-6, 9 * A, 1 << 20, None) == la.LA_E_INVAL
    assert L_.la_global_backward(A, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A, 7 * A, 8 * A, 1, 2, 64,
                                 40, BF16, F32, 1e-6, 9 * A, 1 << 20, None) == la.LA_E_UNSUPPORTED
    # no tokens and no state gradient wanted: nothing to do, nothing launched
    assert bwd(N=0, q=None, k=None, v=None, do=None, dq=None, dk=None, dv=None, ws=None,
               wsb=0) == la.LA_OK


def test_backward_workspace_size():
    E = 64 * 64 + 64
    # one short block: one query split, the workspace holds R only
    assert la.backward_workspace_size(1, 1, 100, 100, 64) == E * 4
    # the 720p chunk: 16 query items per head (512 = one round of the
    # persistent grid) -> R plus 16 partials per head
    assert la.backward_workspace_size(1, 32, 75600, 75600, 64) == 32 * E * 4 * 17
    # config-5 shape in one call: 40 blocks x 64 heads, one split each
    E2 = 128 * 128 + 128
    assert la.backward_workspace_size(4, 16, 40 * 4096, 4096, 128) == 4 * 16 * 40 * E2 * 4


def tconv(x=A, ci=2 * A, w=3 * A, b=4 * A, y=5 * A, co=6 * A, B=1, F=21, P=36, C=64,
          xdt=BF16, ydt=BF16, Tf=None):
    if Tf is None:
        return la.lib().la_temporal_conv_chunk(x, ci, w, b, y, co, B, F, P, C, xdt, ydt, None)
    return la.lib().la_temporal_conv_blockcausal(x, ci, w, b, y, co, B, F, Tf, P, C, xdt, ydt,
                                                 None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), la.LA_E_INVAL),
    (dict(F=-1), la.LA_E_INVAL),
    (dict(P=0), la.LA_E_INVAL),
    (dict(C=12), la.LA_E_UNSUPPORTED),
    (dict(xdt=4), la.LA_E_UNSUPPORTED),
    (dict(w=None), la.LA_E_INVAL),
    (dict(x=None), la.LA_E_INVAL),
    (dict(Tf=0), la.LA_E_INVAL),
    (dict(F=70000, Tf=1), la.LA_E_INVAL),          # more chunks than the grid allows
    (dict(x=A + 2), la.LA_E_ALIGN),
    (dict(co=6 * A + 8), la.LA_E_ALIGN),
    (dict(y=A + 1024), la.LA_E_ALIAS),             # y overlaps x
    (dict(co=A), la.LA_E_ALIAS),                   # cache_out inside x
    (dict(co=2 * A + 64), la.LA_E_ALIAS),          # partial overlap with cache_in
    (dict(co=2 * A, Tf=7), la.LA_E_ALIAS),         # in place with three chunks
])
def test_temporal_conv_rejects(kw, code):
    assert tconv(**kw) == code


def bwd_noalloc(q=A, k=2 * A, v=3 * A, sts=4 * A, do=5 * A, dsts=None, dq=6 * A, dk=7 * A,
                dv=8 * A, dsi=None, B=1, H=2, N=640, T=64, d=64, idt=BF16, gdt=F32, eps=1e-6):
    return la.lib().la_blockcausal_backward_noalloc(q, k, v, sts, do, dsts, dq, dk, dv, dsi, B, H,
                                                    N, T, d, idt, gdt, eps, None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=0), la.LA_E_INVAL),
    (dict(N=-2), la.LA_E_INVAL),
    (dict(d=48), la.LA_E_UNSUPPORTED),
    (dict(q=None), la.LA_E_INVAL),
    (dict(dq=6 * A + 8), la.LA_E_ALIGN),
    (dict(dk=5 * A + 512), la.LA_E_ALIAS),
    # the suffix states of 64 heads x 40 blocks at d = 128 (169 MB) do not fit
    (dict(B=4, H=16, N=40 * 4096, T=4096, d=128), la.LA_E_SCRATCH),
    # one state slot per (b, h, block) over the 32 MiB: 2,017 heads x 1 block at d = 64
    (dict(B=1, H=2017, N=64, T=64), la.LA_E_SCRATCH),
])
def test_backward_noalloc_rejects(kw, code):
    """The allocation-free backward: argument errors as the workspace call,
    and a clear LA_E_SCRATCH (before any HIP call) when even its smallest plan
    does not fit the static scratch."""
    assert bwd_noalloc(**kw) == code


def test_backward_noalloc_scratch_limit():
    # the largest head count whose suffix states fit one 32 MiB scratch
    E = 64 * 64 + 64
    assert la.NOALLOC_SCRATCH_BYTES // (E * 4) == 2016


def test_backward_stream_count():
    """Two streams for large bfloat16 calls whose key-gradient kernel works on
    items (d = 128, rotary), one otherwise (the key-gradient sweep at d <= 64
    fills the GPU by itself); shape errors as for the workspace size."""
    assert la.backward_stream_count(1, 32, 75600, 75600, 64) == 1        # the 720p chunk: sweep
    assert la.backward_stream_count(1, 32, 75600, 75600, 32) == 1
    assert la.backward_stream_count(1, 32, 75600, 75600, 64, rope=True) == 2
    assert la.backward_stream_count(1, 32, 75600, 75600, 32, rope=True) == 2
    assert la.backward_stream_count(1, 16, 12 * 32760, 32760, 64, rope=True) == 2
    assert la.backward_stream_count(4, 16, 40 * 4096, 4096, 128) == 2    # the long-horizon stream
    assert la.backward_stream_count(4, 16, 40 * 4096, 4096, 128, torch.float32) == 1
    assert la.backward_stream_count(1, 1, 1 << 22, 1 << 22, 128) == 1    # one (b, h) pair
    assert la.backward_stream_count(1, 2, (1 << 19) - 1, 1000, 128) == 1  # below 2^20 token-heads
    assert la.backward_stream_count(1, 2, 1 << 19, 1000, 128) == 2
    assert la.backward_stream_count(1, 8, 0, 1, 128) == 1                 # no tokens
    L_ = la.lib()
    c = ctypes.c_int(-1)
    assert L_.la_backward_stream_count(1, 2, 100, 0, 64, BF16, 0, ctypes.byref(c)) == \
        la.LA_E_INVAL
    assert L_.la_backward_stream_count(1, 2, 100, 100, 48, BF16, 0, ctypes.byref(c)) == \
        la.LA_E_UNSUPPORTED
    assert L_.la_backward_stream_count(1, 2, 100, 100, 64, BF16, 0, None) == la.LA_E_INVAL
    assert c.value == -1
