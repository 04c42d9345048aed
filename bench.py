"""Benchmark: block-causal linear attention on one 720p latent chunk.

One step is one la_chunk_forward call (KV reduction, split reduce + state
add, readout) over a 720p 5 s latent chunk: B=1, H=32, d=64, L=75,600
tokens (21 latent frames of 45 x 80), bfloat16 q/k/v, float32 output and
state, read against the state left by the previous chunk.  Inputs are
seeded synthetic normals x 0.5, resident in HBM before timing; two input
sets alternate so consecutive steps never reuse cached inputs.

Prints one JSON line.  `value` is latent tokens per second of the whole
call; `roofline` covers the dominant kernel (the readout) with algorithmic
bytes per launch over its average launch time from HIP events recorded on
the library's stream inside the timed region; `cpu_baseline` times the fp64
oracle on the same workload on the host; `per_call_us` gives the median and
10th/90th percentiles of further calls (--spread-calls, default 60), each
bracketed by its own events after the timed region (not part of `value`).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --workload {chunk720p,global480p,global720p,stream480p,longhorizon}
    python bench.py --copy-calibration     # plain copy kernel for counter scaling

The other workloads (one JSON line each, same fields) time the global form at
the 480p and 720p latents, the 12-chunk 1-minute 480p stream and the 40-chunk
d = 128 long-horizon stream (one step = the whole stream, state resident);
their inputs are seeded normals drawn on the GPU.
"""

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "latent tokens/sec + % peak HBM BW, block-causal linear attn, 720p chunk"
# the other forward workloads (the workload itself is named in `config`)
METRIC_OTHER = "latent tokens/sec + % peak HBM BW, block-causal linear attn"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "readout_720p_chunk_traffic.json")
# What defines the readout kernel's HBM traffic at the 720p chunk: its
# sources, and the planner constants that set its grid.
KERNEL_SOURCES = ["la_common.h", "row_tiles.h", "readout.h"]
PLAN_CONSTANTS = ("kSweepWorkgroups", "LA_READOUT_ROWS", "LA_READOUT_STREAM", "LA_READOUT_RUN")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def spread_us(ms):
    """Median, 10th and 90th percentile (us) of per-call times in ms."""
    x = np.asarray(ms, dtype=np.float64) * 1e3
    return {"median": float(np.median(x)), "p10": float(np.percentile(x, 10)),
            "p90": float(np.percentile(x, 90)), "samples": int(x.size)}


def _code_only(text):
    """Source text without comments and blank space, so that a comment edit
    does not count as a kernel change."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_causal_linear_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name)) as f:
            h.update(_code_only(f.read()).encode())
    with open(os.path.join(csrc, "linattn.hip")) as f:
        for line in f:
            if any(c in line for c in PLAN_CONSTANTS):
                h.update(_code_only(line).encode())
    return h.hexdigest()[:16]


def bytes_alg(B, H, L, d, s_in=2, s_out=4, with_state_in=True):
    """Algorithmic HBM bytes of one call and of its KV and readout stages."""
    tok = B * H * L * d
    st = B * H * (d * d + d) * 4
    kv = 2 * tok * s_in                  # read K, V once
    readout = tok * (s_in + s_out) + st  # read Q, write O, read the updated state
    call = 3 * tok * s_in + tok * s_out + (2 if with_state_in else 1) * st
    return call, kv, readout


def flops(B, H, L, d):
    return 4 * B * H * L * d * d + 4 * B * H * L * d


def stored_traffic(launch_bytes_alg):
    """HBM bytes per readout launch from committed rocprofv3 counters, if they
    were taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, seconds_min=10.0):
    """The fp64 oracle on the same 720p chunk, on the host cores."""
    import oracle
    import workloads

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    Q, K, V = workloads.chunk_qkv(w, 1)
    B, H, L, d = w.B, w.H, w.L, w.d
    S0 = np.random.default_rng(0).standard_normal((B, H, d, d)) * 100.0
    z0 = np.full((B, H, d), 1e4)
    runs, t_total = 0, 0.0
    while t_total < seconds_min and runs < 12:
        t0 = time.perf_counter()
        oracle.chunk_forward(Q, K, V, S0, z0, workloads.EPS)
        t_total += time.perf_counter() - t0
        runs += 1
    per = t_total / runs
    return {"value": B * L / per, "unit": "latent tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"the full 720p chunk (B=1, H=32, d=64, L=75,600), fp64 numpy "
                      f"{np.__version__} ({threads} BLAS threads), {runs} run(s), {per:.2f} s "
                      f"each; host cpus visible: {len(os.sched_getaffinity(0))}"}


def copy_calibration(steps):
    """A plain device copy of known size, for scaling FETCH_SIZE/WRITE_SIZE."""
    import torch

    n = 1 << 28  # 256 Mi floats = 1 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "launches": steps}))


OTHER = {
    "global480p": 2,
    "global720p": 3,
    "stream480p": 4,
    "longhorizon": 5,
    "stream480p_onecall": 4,
    "longhorizon_onecall": 5,
}


def bench_other(args):
    """One step = one global call, or one whole stream of chunk calls with the
    state resident and reset at the start of the step."""
    import torch

    import block_causal_linear_amd as la
    import workloads

    w = workloads.WORKLOADS[OTHER[args.workload]]
    B, H, L, d, C = w.B, w.H, w.L, w.d, w.chunks
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(1000 + w.cid)
    log(f"drawing inputs on the GPU for {w.name} (B={B} H={H} L={L} d={d} chunks={C})")

    def draw():
        x = torch.randn((B, H, L, d), generator=gen, device=dev)
        if w.scale != 1.0:
            x.mul_(w.scale)
        if w.outlier_frac > 0:
            rows = torch.rand((B, H, L, 1), generator=gen, device=dev) < w.outlier_frac
            x = torch.where(rows, x * w.outlier_scale, x)
        return x.to(torch.bfloat16)

    onecall = args.workload.endswith("_onecall")
    if onecall:
        # the whole stream as one sequence of C blocks, one la_blockcausal_forward per step
        seq = tuple(torch.cat([draw() for _ in range(C)], dim=2) for _ in range(3))
        out_seq = torch.empty((B, H, L * C, d), dtype=torch.float32, device=dev)
        states = torch.empty((B, H, C, d * d + d), dtype=torch.float32, device=dev)
        chunks = []
    else:
        chunks = [tuple(draw() for _ in range(3)) for _ in range(C)]
    out = torch.empty((B, H, L, d), dtype=torch.float32, device=dev)
    state = torch.empty((B, H, d * d + d), dtype=torch.float32, device=dev)
    splits, rwg = la.plan(B, H, L, d, kv_splits=args.kv_splits)
    log(f"plan (per chunk call): kv_splits={splits} readout_workgroups={rwg}")

    # stage events on every `event_every`-th call (counted over all calls)
    every = max(1, args.event_every)
    steps = max(1, args.steps // C) if C > 1 else args.steps
    calls = 1 if onecall else C
    evs = {c: la.StageEvents() for c in range(0, steps * calls, max(1, every // (C // calls)))}

    def step(i=None):
        if onecall:
            ev = None if i is None else evs.get(i)
            la.blockcausal_forward(seq[0], seq[1], seq[2], L, out=out_seq, states=states,
                                   eps=workloads.EPS, kv_splits=args.kv_splits, stage_events=ev)
            return
        base = None if i is None else i * C
        if w.form == "global":
            q, k, v = chunks[0]
            la.global_forward(q, k, v, out=out, state_out=state, eps=workloads.EPS,
                              kv_splits=args.kv_splits,
                              stage_events=None if base is None else evs.get(base))
            return
        la.state_reset(state)
        for n, (q, k, v) in enumerate(chunks):
            la.chunk_forward(q, k, v, state, out=out, state_out=state, eps=workloads.EPS,
                             kv_splits=args.kv_splits,
                             stage_events=None if base is None else evs.get(base + n))

    for _ in range(max(1, args.warmup // C)):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    stages = np.array([e.elapsed_ms() for e in evs.values()])
    for e in evs.values():
        e.close()
    kv_ms, red_ms, ro_ms = (float(x) for x in stages.mean(axis=0))
    call_b, kv_b, ro_b = bytes_alg(B, H, L, d, with_state_in=(w.form != "global"))
    if onecall:  # stage times cover all C blocks
        kv_b, ro_b = kv_b * C, ro_b * C
    tokens = B * L * C
    ro_kernel = f"readout_items_bf16<{d}>" if d == 128 else f"readout_sweep_bf16<{d}>"
    result = {
        "metric": METRIC_OTHER, "value": tokens / (ms * 1e-3), "unit": "latent tokens/s",
        "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name + ("-one-call" if onecall else ""), "form": w.form,
                   "B": B, "H": H, "d": d, "L": L, "blocks_per_step": C,
                   "calls_per_step": calls, "q_k_v": "bf16", "out": "f32", "state": "f32",
                   "kv_splits": splits, "readout_workgroups": rwg},
        "hbm_frac": call_b * C / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "us_per_call": ms * 1e3 / calls,
        "us_per_block": ms * 1e3 / C,
        "roofline": {"bound": "hbm", "kernel": ro_kernel,
                     "achieved": ro_b / (ro_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": ro_b / (ro_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "traffic": None, "bytes_alg_per_launch": ro_b, "launch_us": ro_ms * 1e3},
        "stages_us": {"kv_partial": kv_ms * 1e3, "state_reduce": red_ms * 1e3,
                      "readout": ro_ms * 1e3, "event_samples": int(stages.shape[0])},
        "kv_partial_GBs": kv_b / (kv_ms * 1e-3) / 1e9,
    }
    print(json.dumps(result), flush=True)


ROPE = {
    "rope_chunk720p": 3,
    "rope_stream480p_onecall": 4,
    "rope_longhorizon_onecall": 5,
}


def bench_rope(args):
    """The rotary-position forward (la_blockcausal_forward_rope).  One step:
    the 720p chunk read against the state of the chunk before it (one block,
    frame0 = 21), or a whole stream of blocks in one call."""
    import torch

    import block_causal_linear_amd as la
    import workloads

    chunk = args.workload == "rope_chunk720p"
    w = workloads.CHUNK_720P if chunk else workloads.WORKLOADS[ROPE[args.workload]]
    gh, gw = workloads.GRIDS[w.cid]
    B, H, L, d = w.B, w.H, w.L, w.d
    C = 1 if chunk else w.chunks
    N = L * C
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(2000 + w.cid)
    log(f"drawing inputs on the GPU for rotary {w.name} (B={B} H={H} N={N} d={d} blocks={C}, "
        f"frames of {gh} x {gw})")

    def draw(n):
        x = torch.randn((B, H, n, d), generator=gen, device=dev)
        if w.scale != 1.0:
            x.mul_(w.scale)
        if w.outlier_frac > 0:
            rows = torch.rand((B, H, n, 1), generator=gen, device=dev) < w.outlier_frac
            x = torch.where(rows, x * w.outlier_scale, x)
        return x.to(torch.bfloat16)

    sets = [tuple(draw(N) for _ in range(3)) for _ in range(2 if chunk else 1)]
    out = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    states = torch.empty((B, H, C, d * d + d), dtype=torch.float32, device=dev)
    state0, f0 = None, 0
    if chunk:
        q0, k0, v0 = (draw(N) for _ in range(3))
        _, st = la.blockcausal_forward_rope(q0, k0, v0, N, 0, gh, gw, workloads.ROPE_THETA,
                                            eps=workloads.EPS)
        state0, f0 = st[:, :, 0].contiguous(), workloads.chunk_frame0(w, 1)
        del q0, k0, v0
    torch.cuda.synchronize()

    every = max(1, args.event_every)
    evs = {i: la.StageEvents() for i in range(0, args.steps, every)}

    def step(i, ev=None):
        q, k, v = sets[i % len(sets)]
        la.blockcausal_forward_rope(q, k, v, L, f0, gh, gw, workloads.ROPE_THETA,
                                    state_in=state0, out=out, states=states, eps=workloads.EPS,
                                    kv_splits=args.kv_splits, stage_events=ev)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        step(i, evs.get(i))
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    stages = np.array([e.elapsed_ms() for e in evs.values()])
    for e in evs.values():
        e.close()
    kv_ms, red_ms, ro_ms = (float(x) for x in stages.mean(axis=0))
    call_b, kv_b, ro_b = bytes_alg(B, H, L, d, with_state_in=chunk)
    call_b, kv_b, ro_b = call_b * C, kv_b * C, ro_b * C
    result = {
        "metric": METRIC_OTHER + " (rotary)", "value": B * N / (ms * 1e-3),
        "unit": "latent tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "rotary " + w.name + ("" if chunk else "-one-call"),
                   "B": B, "H": H, "d": d, "L": L, "blocks_per_step": C, "grid": [gh, gw],
                   "theta": workloads.ROPE_THETA, "q_k_v": "bf16", "out": "f32",
                   "state": "f32"},
        "hbm_frac": call_b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "us_per_block": ms * 1e3 / C,
        "roofline": {"bound": "hbm", "kernel": f"readout_rope_bf16<{d}>",
                     "achieved": ro_b / (ro_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": ro_b / (ro_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "traffic": None, "bytes_alg_per_launch": ro_b, "launch_us": ro_ms * 1e3},
        "stages_us": {"kv_partial_rope": kv_ms * 1e3, "state_reduce_or_scan": red_ms * 1e3,
                      "readout": ro_ms * 1e3, "event_samples": int(stages.shape[0])},
        "kv_partial_GBs": kv_b / (kv_ms * 1e-3) / 1e9,
    }
    print(json.dumps(result), flush=True)


BACKWARD = {
    "bwd_chunk720p": 3,
    "bwd_stream480p_onecall": 4,
    "bwd_longhorizon_onecall": 5,
    "rope_bwd_chunk720p": 3,
    "rope_bwd_stream480p_onecall": 4,
}


def bwd_bytes(B, H, N, d, C, s_in=2, s_g=4):
    """Algorithmic bytes of one backward call (float32 gradients):
    query kernel: read Q, dO and the C block states, write dQ;
    key kernel: read K, V and the C suffix states, write dK, dV;
    the whole call: Q, K, V, dO, states (+ one state gradient) in, dQ, dK,
    dV (+ one state gradient) out."""
    th = B * H * N * d
    st = B * H * C * (d * d + d) * 4
    query = th * (s_in + 2 * s_g) + st
    key = th * (2 * s_in + 2 * s_g) + st
    call = th * (3 * s_in + 4 * s_g) + st + 2 * B * H * (d * d + d) * 4
    return call, query, key


def bench_backward(args):
    """One step = one backward call over resident inputs and forward states
    (the 720p chunk with gradients on its state, or a whole stream in one
    la_blockcausal_backward), plain or rotary (la_blockcausal_backward_rope,
    the chunk at frame0 = 21 against the rotated state of frames 0..20)."""
    import torch

    import block_causal_linear_amd as la
    import workloads

    chunked = args.workload in ("bwd_chunk720p", "rope_bwd_chunk720p")
    rope = args.workload.startswith("rope_")
    w = workloads.CHUNK_720P if chunked else workloads.WORKLOADS[BACKWARD[args.workload]]
    gh, gw = workloads.GRIDS[w.cid]
    f0 = workloads.chunk_frame0(w, 1) if chunked and rope else 0
    B, H, d = w.B, w.H, w.d
    C = 1 if chunked else w.chunks
    T = w.L
    N = T * C
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(2000 + w.cid)
    log(f"drawing inputs on the GPU for the backward of {w.name} (B={B} H={H} N={N} T={T} d={d})")

    def draw(dtype=torch.bfloat16, scale=w.scale):
        x = torch.randn((B, H, N, d), generator=gen, device=dev)
        if scale != 1.0:
            x.mul_(scale)
        return x.to(dtype)

    q, k, v = draw(), draw(), draw()
    dout = draw(torch.float32, 1.0)
    state_in = None
    if chunked and rope:
        _, st = la.blockcausal_forward_rope(draw(), draw(), draw(), N, 0, gh, gw,
                                            workloads.ROPE_THETA, eps=workloads.EPS)
        state_in = st[:, :, 0].contiguous()
    elif chunked:
        _, state_in = la.global_forward(draw(), draw(), draw(), eps=workloads.EPS)
    if rope:
        _, states = la.blockcausal_forward_rope(q, k, v, T, f0, gh, gw, workloads.ROPE_THETA,
                                                state_in=state_in, eps=workloads.EPS)
    else:
        _, states = la.blockcausal_forward(q, k, v, T, state_in=state_in, eps=workloads.EPS)
    dstates = torch.randn(states.shape, generator=gen, device=dev).mul_(1e-5) if chunked else None
    dq, dk, dv = (torch.empty((B, H, N, d), dtype=torch.float32, device=dev) for _ in range(3))
    dsi = torch.empty((B, H, d * d + d), dtype=torch.float32, device=dev) if chunked else None
    ws = torch.empty(la.backward_workspace_size(B, H, N, T, d), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        if rope:
            la.blockcausal_backward_rope(q, k, v, states, dout, T, f0, gh, gw,
                                         workloads.ROPE_THETA, dstates=dstates,
                                         eps=workloads.EPS, dq=dq, dk=dk, dv=dv, dstate_in=dsi,
                                         workspace=ws, kv_splits=args.kv_splits,
                                         stage_events=ev)
        else:
            la.blockcausal_backward(q, k, v, states, dout, T, dstates=dstates, eps=workloads.EPS,
                                    dq=dq, dk=dk, dv=dv, dstate_in=dsi, workspace=ws,
                                    kv_splits=args.kv_splits, stage_events=ev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    every = max(1, args.event_every)
    evs = {i: la.StageEvents() for i in range(0, args.steps, every)}
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(evs.get(i))
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    stages = np.array([e.elapsed_ms() for e in evs.values()])
    for e in evs.values():
        e.close()
    q_ms, scan_ms, k_ms = (float(x) for x in stages.mean(axis=0))
    call_b, q_b, k_b = bwd_bytes(B, H, N, d, C)
    result = {
        "metric": "latent tokens/sec + % peak HBM BW, block-causal linear attn backward",
        "value": B * N / (ms * 1e-3), "unit": "latent tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": ("rotary " if rope else "") + w.name
                   + (" backward" if chunked else "-one-call backward"),
                   "B": B, "H": H, "d": d, "N": N, "T": T, "blocks": C, "q_k_v": "bf16",
                   "grads": "f32", "state_grads": chunked,
                   **({"frame0": f0, "grid": [gh, gw]} if rope else {})},
        "hbm_frac": call_b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "us_per_block": ms * 1e3 / C,
        "roofline": {"bound": "hbm",
                     "kernel": f"bwd_key_{'rope_' if rope else ''}bf16<{d}>",
                     "achieved": k_b / (k_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": k_b / (k_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "traffic": None, "bytes_alg_per_launch": k_b, "launch_us": k_ms * 1e3},
        "stages_us": {"bwd_query": q_ms * 1e3, "suffix_scan": scan_ms * 1e3,
                      "bwd_key": k_ms * 1e3, "event_samples": int(stages.shape[0])},
        "bwd_query_GBs": q_b / (q_ms * 1e-3) / 1e9,
        "bwd_key_GBs": k_b / (k_ms * 1e-3) / 1e9,
    }
    print(json.dumps(result), flush=True)


TCONV = {
    # name: (B, frames per chunk, chunks, positions per frame, channels)
    "tconv720p": (1, 21, 1, 3600, 2048),
    "tconv480p_onecall": (1, 21, 12, 1560, 1024),
}


def bench_tconv(args):
    """One step = one temporal-convolution call (bf16 activations in and
    out, float32 taps and bias, the one-frame cache read and written) over
    resident inputs: the 720p chunk, or the 1-minute 480p stream in one
    block-causal call."""
    import torch

    import block_causal_linear_amd as la

    B, T, n, P, C = TCONV[args.workload]
    F = T * n
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(3000)
    log(f"drawing inputs on the GPU for {args.workload} (B={B} F={F} T={T} P={P} C={C})")
    x = torch.randn((B, F, P, C), generator=gen, device=dev).to(torch.bfloat16)
    w = torch.randn((C, 3), generator=gen, device=dev).div_(3 ** 0.5)
    b = torch.randn((C,), generator=gen, device=dev).mul_(0.1)
    cache = torch.randn((B, P, C), generator=gen, device=dev).to(torch.bfloat16)
    y = torch.empty_like(x)
    cache_out = torch.empty_like(cache)

    def step():
        la.temporal_conv_blockcausal(x, w, T, b, cache_in=cache, y=y, cache_out=cache_out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    # x read once, y written once, the cache read and written (taps and bias
    # are a few KB)
    nbytes = 2 * B * F * P * C * 2 + 2 * B * P * C * 2
    result = {
        "metric": "latent tokens/sec + % peak HBM BW, Mix-FFN temporal conv with chunk cache",
        "value": B * F * P / (ms * 1e-3), "unit": "latent tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "frames": F, "frames_per_chunk": T,
                   "positions_per_frame": P, "channels": C, "x_y": "bf16"},
        "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "roofline": {"bound": "hbm", "kernel": "temporal_conv<true, true>",
                     "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "traffic": None,
                     "bytes_alg_per_launch": nbytes, "launch_us": ms * 1e3},
    }
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--kv-splits", type=int, default=0)
    ap.add_argument("--workload", default="chunk720p",
                    choices=["chunk720p", "global480p", "global720p", "stream480p", "longhorizon",
                             "stream480p_onecall", "longhorizon_onecall"] + list(BACKWARD)
                    + list(TCONV) + list(ROPE))
    ap.add_argument("--event-every", type=int, default=10,
                    help="record per-stage HIP events on every N-th timed step")
    ap.add_argument("--plain-steps", type=int, default=0,
                    help="also time this many steps without stage events (for comparison)")
    ap.add_argument("--spread-calls", type=int, default=60,
                    help="after the timed region, bracket this many calls each with events "
                         "for the per-call median and 10th/90th percentiles")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path.  The "
              "(b, h) pairs are independent, so heads shard across GPUs with no exchange and "
              "each GPU runs this same call on its share.  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_causal_linear_amd as la
    import workloads

    if args.copy_calibration:
        copy_calibration(max(args.steps, 1))
        return
    if args.workload in BACKWARD:
        bench_backward(args)
        return
    if args.workload in TCONV:
        bench_tconv(args)
        return
    if args.workload in ROPE:
        bench_rope(args)
        return
    if args.workload != "chunk720p":
        bench_other(args)
        return

    w = workloads.CHUNK_720P
    B, H, L, d = w.B, w.H, w.L, w.d
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"generating inputs for {w.name} (B={B} H={H} L={L} d={d})")

    def upload(x):
        return torch.from_numpy(x).to(dev).to(torch.bfloat16)

    q0, k0, v0 = (upload(x) for x in workloads.chunk_qkv(w, 0))
    sets = []
    for chunk in (1, 2):
        q, k, v = (upload(x) for x in workloads.chunk_qkv(w, chunk))
        out = torch.empty((B, H, L, d), dtype=torch.float32, device=dev)
        st = torch.empty((B, H, d * d + d), dtype=torch.float32, device=dev)
        sets.append((q, k, v, out, st))
    # the committed state after chunk 0
    _, state0 = la.global_forward(q0, k0, v0, eps=workloads.EPS)
    del q0, k0, v0
    torch.cuda.synchronize()
    splits, rtok = la.plan(B, H, L, d, kv_splits=args.kv_splits)
    log(f"plan: kv_splits={splits} readout_workgroups={rtok}")

    def step(i, ev=None):
        q, k, v, out, st = sets[i & 1]
        la.chunk_forward(q, k, v, state0, out=out, state_out=st, eps=workloads.EPS,
                         kv_splits=args.kv_splits, stage_events=ev)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps); timing {args.steps} steps")

    # Timed region.  Every N-th call records four HIP events on the library's
    # stream around its three kernels (an event record costs a few us of GPU
    # time, so sampling keeps `value` close to the plain call rate).
    every = max(1, args.event_every)
    evs = {i: la.StageEvents() for i in range(0, args.steps, every)}
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(i, evs.get(i))
    end.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    stages = np.array([e.elapsed_ms() for e in evs.values()])  # [samples, 3] ms
    for e in evs.values():
        e.close()
    ms = ms_total / args.steps
    log(f"timed: {ms * 1e3:.1f} us/step")

    plain_ms = None
    if args.plain_steps > 0:
        torch.cuda.synchronize()
        start.record()
        for i in range(args.plain_steps):
            step(i)
        end.record()
        torch.cuda.synchronize()
        plain_ms = start.elapsed_time(end) / args.plain_steps
        log(f"without stage events: {plain_ms * 1e3:.1f} us/step")

    spread = None
    if args.spread_calls > 0:
        # not part of `value`: every call bracketed by its own events
        sp = [la.StageEvents() for _ in range(args.spread_calls)]
        torch.cuda.synchronize()
        for i, e in enumerate(sp):
            step(i, e)
        torch.cuda.synchronize()
        per = np.array([e.elapsed_ms() for e in sp])  # [calls, 3] ms
        for e in sp:
            e.close()
        spread = {"call": spread_us(per.sum(axis=1)), "readout": spread_us(per[:, 2])}

    call_b, kv_b, ro_b = bytes_alg(B, H, L, d)
    kv_ms, red_ms, ro_ms = (float(x) for x in stages.mean(axis=0))
    tokens_per_s = B * L / (ms * 1e-3)
    ro_gbs = ro_b / (ro_ms * 1e-3) / 1e9
    kv_gbs = kv_b / (kv_ms * 1e-3) / 1e9
    call_gbs = call_b / (ms * 1e-3) / 1e9
    traffic = stored_traffic(ro_b)

    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "latent tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "720p-chunk block-causal la_chunk_forward", "B": B, "H": H,
                   "d": d, "L": L, "q_k_v": "bf16", "out": "f32", "state": "f32",
                   "kv_splits": splits, "readout_workgroups": rtok},
        "hbm_frac": call_gbs / PEAK_HBM_GBS,
        "achieved_GBs": call_gbs,
        "roofline": {"bound": "hbm", "kernel": "readout_sweep_bf16<64>", "achieved": ro_gbs,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ro_gbs / PEAK_HBM_GBS,
                     "traffic": traffic, "bytes_alg_per_launch": ro_b,
                     "launch_us": ro_ms * 1e3},
        "stages_us": {"kv_partial": kv_ms * 1e3, "state_reduce": red_ms * 1e3,
                      "readout": ro_ms * 1e3, "event_samples": int(stages.shape[0])},
        "kv_partial_GBs": kv_gbs,
        "mfma_frac_call": flops(B, H, L, d) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
    }
    if spread is not None:
        result["per_call_us"] = spread
    if plain_ms is not None:
        result["ms_per_step_without_stage_events"] = plain_ms
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host")
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
