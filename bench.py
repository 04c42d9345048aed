"""Benchmark: block-causal linear attention on one 720p latent chunk.

One step is one la_chunk_forward call (KV reduction, split reduce + state
add, readout) over a 720p 5 s latent chunk: B=1, H=32, d=64, L=75,600
tokens (21 latent frames of 45 x 80), bfloat16 q/k/v, float32 output and
state, read against the state left by the previous chunk.  Inputs are
seeded synthetic normals x 0.5, resident in HBM before timing; two input
sets alternate so consecutive steps never reuse cached inputs.

Prints one JSON line.  The run has four parts:

* warm-up: the W steps asked for, continued until at least --min-warmup-s
  seconds of back-to-back calls have run (clocks and caches settle); the
  number of warm-up calls made is in the line;
* the timed region: exactly K plain calls between two synchronised events.
  `value` (latent tokens per second) and `hbm_frac` come from it alone;
* the sampled pass: max(K, --sample-calls) further calls, each recording four
  HIP events on the library's stream around its three kernels.  `roofline`
  (the dominant kernel, the readout: algorithmic bytes per launch over its
  mean launch interval), `stages_us` and `per_call_us` come from it;
* `cpu_baseline`: the fp64 oracle timed on the host on the same inputs (the
  chunk-0 and chunk-1 tensors; each side derives the chunk-0 state itself),
  with the normwise error of the GPU's output and state against it.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --workload W       # another configuration (see OTHER etc.)
    python bench.py --workload ceiling # HBM stream ceilings of the kernels' access mixes
    python bench.py --copy-calibration # plain copy kernel for counter scaling

Every other workload prints one line of the same form: the timed region, a
sampled pass with stage events, and an oracle leg on a bounded sample of
the same workload (seeded host inputs of the workload's distribution, run
through the GPU call and the oracle, timed on the oracle side).
"""

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
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
PARITY_BOUND_BF16 = 2e-3       # normwise, bf16 inputs
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "readout_720p_chunk_traffic.json")
PROBE_LIB = os.path.join(ROOT, "block_causal_linear_amd", "libla_probes.so")
# What defines the readout kernel's HBM traffic at the 720p chunk: its
# sources, and the planner constants that set its grid.
KERNEL_SOURCES = ["la_common.h", "row_tiles.h", "readout.h"]
PLAN_CONSTANTS = ("kSweepWorkgroups", "LA_READOUT_ROWS", "LA_READOUT_STREAM", "run_log2")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def spread_us(ms):
    """Mean, median, 10th and 90th percentile (us) of per-call times in ms."""
    x = np.asarray(ms, dtype=np.float64) * 1e3
    return {"mean": float(x.mean()), "median": float(np.median(x)),
            "p10": float(np.percentile(x, 10)), "p90": float(np.percentile(x, 90)),
            "samples": int(x.size)}


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


def stored_traffic():
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


# ---------------------------------------------------------------------------
# timing helpers

def warm_up(step, warmup, min_s):
    """`warmup` calls, then more until `min_s` seconds have passed since the
    first; returns the number of calls made."""
    import torch

    t0 = time.perf_counter()
    calls = 0
    for _ in range(warmup):
        step(calls)
        calls += 1
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < min_s:
        for _ in range(8):
            step(calls)
            calls += 1
        torch.cuda.synchronize()
    return calls


def timed_region(step, steps):
    """Exactly `steps` calls between two synchronised events: ms per call."""
    import torch

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def sampled_pass(step_ev, calls):
    """`calls` further calls, each bracketed by its own stage events:
    an array [calls, 3] of (stage 1, stage 2, stage 3) milliseconds."""
    import torch

    import block_causal_linear_amd as la

    evs = [la.StageEvents() for _ in range(calls)]
    torch.cuda.synchronize()
    for i, e in enumerate(evs):
        step_ev(i, e)
    torch.cuda.synchronize()
    per = np.array([e.elapsed_ms() for e in evs])
    for e in evs:
        e.close()
    return per


def stage_summary(per, names):
    out = {name: spread_us(per[:, i]) for i, name in enumerate(names)}
    out["call"] = spread_us(per.sum(axis=1))
    return out


def roofline(kernel, nbytes, launch_ms, traffic=None):
    """Algorithmic bytes per launch over the mean launch interval of the
    sampled pass."""
    x = np.asarray(launch_ms, dtype=np.float64)
    mean_s = float(x.mean()) * 1e-3
    achieved = nbytes / mean_s / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": achieved, "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
            "bytes_alg_per_launch": nbytes, "launch_us": mean_s * 1e6,
            "launch_us_median": float(np.median(x)) * 1e3, "samples": int(x.size),
            "source": "mean of the sampled pass's stage-event intervals (each also holds "
                      "the dispatch gap before the kernel)"}


# ---------------------------------------------------------------------------
# the oracle leg

def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        return int(os.environ.get("OMP_NUM_THREADS", "1"))


def time_oracle(fn, seconds_min=10.0, max_runs=12):
    """Runs fn until `seconds_min` seconds have passed (at most max_runs
    runs); returns (its last result, seconds per run, runs)."""
    runs, total, res = 0, 0.0, None
    while True:
        t0 = time.perf_counter()
        res = fn()
        total += time.perf_counter() - t0
        runs += 1
        if total >= seconds_min or runs >= max_runs:
            return res, total / runs, runs


def normwise(got, ref, slice_axes):
    """max over slices of max|got - ref| / max|ref|, slices being the indices
    of the leading axes not in `slice_axes` (those are reduced)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(got - ref).max(axis=slice_axes)
    den = np.abs(ref).max(axis=slice_axes)
    return float(np.max(num / np.where(den > 0, den, 1.0)))


def state_parts(st, d):
    """(S [..., d, d], z [..., d]) float64 from a float32 state tensor."""
    x = st.double().cpu().numpy()
    return x[..., : d * d].reshape(x.shape[:-1] + (d, d)), x[..., d * d:]


def cpu_leg(tokens, per_s, runs, sample, errors):
    threads = blas_threads()
    return {"value": tokens / per_s, "unit": "latent tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{sample}; fp64 numpy {np.__version__} ({threads} BLAS threads), "
                      f"{runs} run(s) of {per_s:.2f} s; host cpus visible: "
                      f"{len(os.sched_getaffinity(0))}",
            "parity": dict(errors, bound=PARITY_BOUND_BF16,
                           metric="max over (b, h[, block]) slices of max|gpu - oracle| / "
                                  "max|oracle|")}


def to_dev(x, dev, dtype=None):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    return t.to(dtype if dtype is not None else torch.bfloat16)


def oracle_stream(w, chunks, blocks_gpu):
    """Oracle leg of a chunk stream or a whole-sequence call: the first
    `chunks` chunks of workload w from the seeded host generator, carried
    through `blocks_gpu` (a function of the list of (Q, K, V) arrays that
    returns the GPU outputs [chunks] and states [chunks] as tensors)."""
    import oracle
    import workloads

    blocks = [workloads.chunk_qkv(w, c) for c in range(chunks)]
    outs_g, states_g = blocks_gpu(blocks)
    (outs, states), per, runs = time_oracle(lambda: oracle.stream_forward(blocks, workloads.EPS),
                                            seconds_min=8.0)
    d = w.d
    eo = max(normwise(o.double().cpu().numpy(), r, (2, 3)) for o, r in zip(outs_g, outs))
    es = 0.0
    for sg, (S, z) in zip(states_g, states):
        Sg, zg = state_parts(sg, d)
        es = max(es, normwise(Sg, S, (2, 3)), normwise(zg, z, (2,)))
    return per, runs, {"out": eo, "state": es}


# ---------------------------------------------------------------------------
# the HBM ceiling probes

def bench_ceiling(args):
    """Times the stream probes (libla_probes.so) at the byte counts of the
    720p chunk: read-only (the KV reduction's 619.3 MB of K and V), write-only
    (the readout's 619.3 MB of float32 rows), copy (309.7 MB each way) and the
    readout's mix (309.7 MB of bfloat16 in, 619.3 MB of float32 out), over
    schedules, grid sizes and cache policies.  Prints one JSON line with the
    best rate of each mix and the whole table."""
    import torch

    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is not built; run `python -m block_causal_linear_amd.build`")
    pl = ctypes.CDLL(PROBE_LIB)
    pl.lap_stream.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p, ctypes.c_void_p,
                                                    ctypes.c_longlong, ctypes.c_void_p,
                                                    ctypes.c_void_p]
    pl.lap_stream.restype = ctypes.c_int
    pl.lap_chunk_bytes.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_longlong),
                                   ctypes.POINTER(ctypes.c_longlong)]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    big = 32 * 75600 * 64 * 4  # 619,315,200 B
    src = torch.randint(0, 256, (big,), dtype=torch.uint8, device=dev)
    dst = torch.empty(big, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4096, dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    mixes = {  # mode, bytes read per launch, label
        "read": (0, big, "read-only: the KV reduction's mix"),
        "write": (1, 0, "write-only"),
        "copy": (2, big // 2, "1 read : 1 write: the temporal convolution's mix"),
        "widen": (3, big // 2, "1 read : 2 writes (bf16 in, fp32 out): the readout's mix"),
    }
    scheds = {"sweep": 0, "range": 1, "oneshot": 2}
    grids = [256, 512, 1024, 2048, 4096]
    reps = max(5, args.steps // 10)
    table = []
    best = {}
    for name, (mode, rbytes, label) in mixes.items():
        rb, wb = ctypes.c_longlong(), ctypes.c_longlong()
        pl.lap_chunk_bytes(mode, ctypes.byref(rb), ctypes.byref(wb))
        unit = rb.value if mode != 1 else wb.value
        nchunks = (rbytes if mode != 1 else big) // unit
        nbytes = nchunks * (rb.value + wb.value)
        nts = [0] if mode == 0 else [0, 1]
        ntl = [0, 1] if mode == 0 else [0]
        for sname, sched in scheds.items():
            for wgs in (grids if sched != 2 else [0]):
                for a in ntl:
                    for b in nts:
                        def launch():
                            rc = pl.lap_stream(mode, sched, wgs, a, b,
                                               ctypes.c_void_p(src.data_ptr()),
                                               ctypes.c_void_p(dst.data_ptr()), nchunks,
                                               ctypes.c_void_p(sink.data_ptr()), stream)
                            if rc != 0:
                                raise RuntimeError(f"lap_stream failed with {rc}")
                        launch()
                        launch()
                        ms = timed_region(lambda i: launch(), reps)
                        gbs = nbytes / (ms * 1e-3) / 1e9
                        row = {"mix": name, "schedule": sname, "workgroups": wgs or nchunks,
                               "nt_loads": a, "nt_stores": b, "GBs": gbs, "us": ms * 1e3}
                        table.append(row)
                        if name not in best or gbs > best[name]["GBs"]:
                            best[name] = dict(row, bytes_per_launch=nbytes, what=label)
        log(f"{name}: best {best[name]['GBs']:.0f} GB/s ({best[name]['schedule']}, "
            f"{best[name]['workgroups']} workgroups)")
    result = {
        "metric": "HBM stream ceilings of the kernels' access mixes (probe kernels)",
        "value": best["widen"]["GBs"], "unit": "GB/s", "n_gpus": 1, "steps": reps,
        "warmup": 2, "higher_is_better": True, "dtype": "u8", "data": "synthetic",
        "config": {"workload": "hbm-ceiling probes at the 720p chunk's byte counts"},
        "peak": PEAK_HBM_GBS,
        "ceilings": {k: {"GBs": v["GBs"], "frac_of_peak": v["GBs"] / PEAK_HBM_GBS,
                         "schedule": v["schedule"], "workgroups": v["workgroups"],
                         "nt_loads": v["nt_loads"], "nt_stores": v["nt_stores"],
                         "bytes_per_launch": v["bytes_per_launch"], "what": v["what"]}
                     for k, v in best.items()},
        "table": table,
    }
    print(json.dumps(result), flush=True)


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


# ---------------------------------------------------------------------------
# the other forward workloads

OTHER = {
    "global480p": 2,
    "global720p": 3,
    "stream480p": 4,
    "longhorizon": 5,
    "stream480p_onecall": 4,
    "longhorizon_onecall": 5,
}
# chunks (or blocks) of the oracle leg's sample
SAMPLE_CHUNKS = {2: 1, 3: 1, 4: 2, 5: 3}


def bench_other(args):
    """One step = one global call, or one whole stream of chunk calls with the
    state resident and reset at the start of the step, or the whole stream as
    one la_blockcausal_forward call."""
    import torch

    import block_causal_linear_amd as la
    import workloads

    w = workloads.WORKLOADS[OTHER[args.workload]]
    B, H, L, d, C = w.B, w.H, w.L, w.d, w.chunks
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
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
    splits, rwg = la.plan(B, H, L, d, kv_splits=args.kv_splits,
                          readout_workgroups=args.readout_workgroups)
    log(f"plan (per chunk call): kv_splits={splits} readout_workgroups={rwg}")

    calls = 1 if (onecall or w.form == "global") else C

    def step(i, evs=None):
        """One step; evs: a list of `calls` StageEvents (or None)."""
        if onecall:
            la.blockcausal_forward(seq[0], seq[1], seq[2], L, out=out_seq, states=states,
                                   eps=workloads.EPS, kv_splits=args.kv_splits,
                                   readout_workgroups=args.readout_workgroups,
                                   stage_events=None if evs is None else evs[0])
            return
        if w.form == "global":
            q, k, v = chunks[0]
            la.global_forward(q, k, v, out=out, state_out=state, eps=workloads.EPS,
                              kv_splits=args.kv_splits,
                              readout_workgroups=args.readout_workgroups,
                              stage_events=None if evs is None else evs[0])
            return
        la.state_reset(state)
        for n, (q, k, v) in enumerate(chunks):
            la.chunk_forward(q, k, v, state, out=out, state_out=state, eps=workloads.EPS,
                             kv_splits=args.kv_splits,
                             readout_workgroups=args.readout_workgroups,
                             stage_events=None if evs is None else evs[n])

    steps = max(1, args.steps // calls) if calls > 1 else args.steps
    wcalls = warm_up(step, max(1, args.warmup // calls), args.min_warmup_s)
    ms = timed_region(step, steps)
    log(f"timed: {ms * 1e3:.1f} us/step")

    # sampled pass: whole steps, every call with stage events
    nsteps = max(1, math.ceil(max(args.sample_calls, args.steps) / calls))
    per = []
    for s in range(nsteps):
        evs = [la.StageEvents() for _ in range(calls)]
        torch.cuda.synchronize()
        step(s, evs)
        torch.cuda.synchronize()
        per.extend(e.elapsed_ms() for e in evs)
        for e in evs:
            e.close()
    per = np.array(per)
    call_b, kv_b, ro_b = bytes_alg(B, H, L, d, with_state_in=(w.form != "global"))
    if onecall:  # stage times cover all C blocks
        kv_b, ro_b = kv_b * C, ro_b * C
    tokens = B * L * C
    ro_kernel = f"readout_items_bf16<{d}>" if d == 128 else f"readout_sweep_bf16<{d}>"
    stage_names = ["kv_partial", "state_reduce" if not onecall else "state_scan", "readout"]
    result = {
        "metric": METRIC_OTHER, "value": tokens / (ms * 1e-3), "unit": "latent tokens/s",
        "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "warmup_calls": wcalls * calls,
        "min_warmup_s": args.min_warmup_s, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name + ("-one-call" if onecall else ""), "form": w.form,
                   "B": B, "H": H, "d": d, "L": L, "blocks_per_step": C,
                   "calls_per_step": calls, "q_k_v": "bf16", "out": "f32", "state": "f32",
                   "kv_splits": splits, "readout_workgroups": rwg},
        "hbm_frac": call_b * C / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "us_per_call": ms * 1e3 / calls,
        "us_per_block": ms * 1e3 / C,
        "roofline": roofline(ro_kernel, ro_b, per[:, 2]),
        "stages_us": stage_summary(per, stage_names),
        "kv_partial_GBs": kv_b / (float(per[:, 0].mean()) * 1e-3) / 1e9,
    }
    del chunks
    if onecall:
        del seq, out_seq, states
    torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        nc = SAMPLE_CHUNKS[w.cid]
        log(f"oracle leg: {nc} chunk(s) of {w.name} from the seeded host generator")

        def gpu_blocks(blocks):
            if w.form == "global":
                q, k, v = (to_dev(x, dev) for x in blocks[0])
                o, st = la.global_forward(q, k, v, eps=workloads.EPS)
                return [o], [st]
            if onecall:
                q, k, v = (to_dev(np.concatenate([b[i] for b in blocks], axis=2), dev)
                           for i in range(3))
                o, sts = la.blockcausal_forward(q, k, v, L, eps=workloads.EPS)
                return ([o[:, :, c * L:(c + 1) * L] for c in range(len(blocks))],
                        [sts[:, :, c] for c in range(len(blocks))])
            st = la.new_state(B, H, d, device=dev)
            outs, sts = [], []
            for Qn, Kn, Vn in blocks:
                o, st2 = la.chunk_forward(to_dev(Qn, dev), to_dev(Kn, dev), to_dev(Vn, dev), st,
                                          eps=workloads.EPS)
                outs.append(o)
                sts.append(st2)
                st = st2
            return outs, sts

        per_s, runs, errs = oracle_stream(w, nc, gpu_blocks)
        what = ("the whole global call" if w.form == "global"
                else f"the first {nc} chunks of the stream"
                + (" as one whole-sequence call on the GPU" if onecall else ""))
        result["cpu_baseline"] = cpu_leg(B * L * nc, per_s, runs,
                                         f"{what} ({w.name}: B={B}, H={H}, d={d}, L={L} per "
                                         f"chunk), seeded host inputs", errs)
    print(json.dumps(result), flush=True)


# ---------------------------------------------------------------------------
# the rotary forward

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
    import oracle
    import workloads

    chunk = args.workload == "rope_chunk720p"
    w = workloads.CHUNK_720P if chunk else workloads.WORKLOADS[ROPE[args.workload]]
    gh, gw = workloads.GRIDS[w.cid]
    B, H, L, d = w.B, w.H, w.L, w.d
    C = 1 if chunk else w.chunks
    N = L * C
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
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

    def step(i, ev=None):
        q, k, v = sets[i % len(sets)]
        la.blockcausal_forward_rope(q, k, v, L, f0, gh, gw, workloads.ROPE_THETA,
                                    state_in=state0, out=out, states=states, eps=workloads.EPS,
                                    kv_splits=args.kv_splits,
                                    readout_workgroups=args.readout_workgroups, stage_events=ev)

    wcalls = warm_up(step, args.warmup, args.min_warmup_s)
    ms = timed_region(step, args.steps)
    per = sampled_pass(step, max(args.steps, args.sample_calls))
    call_b, kv_b, ro_b = bytes_alg(B, H, L, d, with_state_in=chunk)
    call_b, kv_b, ro_b = call_b * C, kv_b * C, ro_b * C
    result = {
        "metric": METRIC_OTHER + " (rotary)", "value": B * N / (ms * 1e-3),
        "unit": "latent tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_calls": wcalls,
        "min_warmup_s": args.min_warmup_s, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "rotary " + w.name + ("" if chunk else "-one-call"),
                   "B": B, "H": H, "d": d, "L": L, "blocks_per_step": C, "grid": [gh, gw],
                   "theta": workloads.ROPE_THETA, "q_k_v": "bf16", "out": "f32",
                   "state": "f32"},
        "hbm_frac": call_b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "us_per_block": ms * 1e3 / C,
        "roofline": roofline(f"readout_rope_bf16<{d}>", ro_b, per[:, 2]),
        "stages_us": stage_summary(per, ["kv_partial_rope", "state_reduce_or_scan", "readout"]),
        "kv_partial_GBs": kv_b / (float(per[:, 0].mean()) * 1e-3) / 1e9,
    }
    del sets, out, states
    torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        # chunk: the chunk-1 tensors read against the state of the chunk-0
        # tensors (each side derives that state itself); streams: the first
        # two blocks in one call
        nb = 1 if chunk else 2
        log(f"oracle leg: rotary {w.name}, {'chunk 1 after chunk 0' if chunk else '2 blocks'}")
        if chunk:
            Q0, K0, V0 = workloads.chunk_qkv(w, 0)
            Q, K, V = workloads.chunk_qkv(w, 1)
            _, S0p, z0p = oracle.rope_prefix_forward(Q0, K0, V0, [0, L], workloads.EPS, 0, gh,
                                                     gw, workloads.ROPE_THETA)
            S0, z0 = S0p[0], z0p[0]
            _, st0 = la.blockcausal_forward_rope(to_dev(Q0, dev), to_dev(K0, dev),
                                                 to_dev(V0, dev), L, 0, gh, gw,
                                                 workloads.ROPE_THETA, eps=workloads.EPS)
            og, sg = la.blockcausal_forward_rope(to_dev(Q, dev), to_dev(K, dev), to_dev(V, dev),
                                                 L, f0, gh, gw, workloads.ROPE_THETA,
                                                 state_in=st0[:, :, 0].contiguous(),
                                                 eps=workloads.EPS)
            del Q0, K0, V0
        else:
            blocks = [workloads.chunk_qkv(w, c) for c in range(nb)]
            Q, K, V = (np.concatenate([b[i] for b in blocks], axis=2) for i in range(3))
            S0 = z0 = None
            og, sg = la.blockcausal_forward_rope(to_dev(Q, dev), to_dev(K, dev), to_dev(V, dev),
                                                 L, 0, gh, gw, workloads.ROPE_THETA,
                                                 eps=workloads.EPS)
        bounds = [L * c for c in range(nb + 1)]
        (O, Sp, zp), per_s, runs = time_oracle(
            lambda: oracle.rope_prefix_forward(Q, K, V, bounds, workloads.EPS, f0, gh, gw,
                                               workloads.ROPE_THETA, S0=S0, z0=z0),
            seconds_min=8.0)
        ogn = og.double().cpu().numpy()
        eo = max(normwise(ogn[:, :, a:b], O[:, :, a:b], (2, 3))
                 for a, b in zip(bounds[:-1], bounds[1:]))
        Sg, zg = state_parts(sg, d)
        es = max(max(normwise(Sg[:, :, c], Sp[c], (2, 3)), normwise(zg[:, :, c], zp[c], (2,)))
                 for c in range(nb))
        result["cpu_baseline"] = cpu_leg(
            B * L * nb, per_s, runs,
            f"rotary {w.name}: " + ("chunk 1 (frames 21-41) against the state of chunk 0"
                                     if chunk else "the first 2 blocks of the stream in one call")
            + ", seeded host inputs", {"out": eo, "state": es})
    print(json.dumps(result), flush=True)


# ---------------------------------------------------------------------------
# the backward

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
    import oracle
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
    torch.cuda.set_device(dev)
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

    def step(i, ev=None):
        if rope:
            la.blockcausal_backward_rope(q, k, v, states, dout, T, f0, gh, gw,
                                         workloads.ROPE_THETA, dstates=dstates,
                                         eps=workloads.EPS, dq=dq, dk=dk, dv=dv, dstate_in=dsi,
                                         workspace=ws, kv_splits=args.kv_splits,
                                         readout_workgroups=args.readout_workgroups,
                                         stage_events=ev)
        else:
            la.blockcausal_backward(q, k, v, states, dout, T, dstates=dstates, eps=workloads.EPS,
                                    dq=dq, dk=dk, dv=dv, dstate_in=dsi, workspace=ws,
                                    kv_splits=args.kv_splits,
                                    readout_workgroups=args.readout_workgroups, stage_events=ev)

    wcalls = warm_up(step, args.warmup, args.min_warmup_s)
    ms = timed_region(step, args.steps)
    per = sampled_pass(step, max(args.steps, args.sample_calls))
    call_b, q_b, k_b = bwd_bytes(B, H, N, d, C)
    streams = la.backward_stream_count(B, H, N, T, d, rope=rope)
    # bf16 at d <= 64 without a key-workgroup request: the sweep kernel
    key_kernel = ("bwd_key_rope_bf16" if rope
                  else "bwd_key_sweep_bf16" if d <= 64 and args.readout_workgroups <= 0
                  else "bwd_key_bf16")
    rf = roofline(f"{key_kernel}<{d}>", k_b, per[:, 2])
    if streams == 2:
        rf["source"] += ("; stage events keep a call on one stream, so this is the kernel of "
                         "a one-stream call, while the timed calls run the two halves of the "
                         "(b, h) pairs on two streams")
    result = {
        "metric": "latent tokens/sec + % peak HBM BW, block-causal linear attn backward",
        "value": B * N / (ms * 1e-3), "unit": "latent tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_calls": wcalls,
        "min_warmup_s": args.min_warmup_s, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": ("rotary " if rope else "") + w.name
                   + (" backward" if chunked else "-one-call backward"),
                   "B": B, "H": H, "d": d, "N": N, "T": T, "blocks": C, "q_k_v": "bf16",
                   "grads": "f32", "state_grads": chunked,
                   **({"frame0": f0, "grid": [gh, gw]} if rope else {})},
        "hbm_frac": call_b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "us_per_block": ms * 1e3 / C,
        "roofline": rf,
        "streams": streams,
        "stages_us": stage_summary(per, ["bwd_query", "suffix_scan", "bwd_key"]),
        "bwd_query_GBs": q_b / (float(per[:, 0].mean()) * 1e-3) / 1e9,
        "bwd_key_GBs": k_b / (float(per[:, 2].mean()) * 1e-3) / 1e9,
    }
    del q, k, v, dout, states, dstates, dq, dk, dv, dsi, ws
    torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        # a bounded sample of the same shape: the first Hs heads (chunk
        # workloads) or the first two blocks (streams), seeded host inputs,
        # a state input and state gradients on the chunk workloads
        Hs = min(H, 4) if chunked else H
        Cs = 1 if chunked else 2
        Ns = T * Cs
        ws_ = workloads.Workload(w.cid, w.name, "chunk", B, Hs, d, Ns, 1, "bf16", scale=w.scale,
                                 outlier_frac=w.outlier_frac, outlier_scale=w.outlier_scale)
        Q, K, V = workloads.chunk_qkv(ws_, 1)
        dO = workloads.random_grads(500 + w.cid, B, Hs, Ns, d)
        bounds = [T * c for c in range(Cs + 1)]
        S0 = z0 = dS = dz = None
        if chunked:
            S0, z0 = workloads.random_state(600 + w.cid, B, Hs, d, tokens=T)
            dS, dz = workloads.random_state_grads(700 + w.cid, B, Hs, Cs, d, scale=1e-5)
        log(f"oracle leg: backward of {w.name}, {Hs} heads x {Cs} block(s)")
        qd, kd, vd = (to_dev(x, dev) for x in (Q, K, V))
        dOd = to_dev(dO, dev, torch.float32)
        si = dsts = None
        if chunked:
            si = to_dev(np.concatenate([S0.reshape(B, Hs, d * d), z0], axis=-1), dev,
                        torch.float32)
            dsts = to_dev(np.concatenate([np.moveaxis(dS, 0, 2).reshape(B, Hs, Cs, d * d),
                                          np.moveaxis(dz, 0, 2)], axis=-1), dev, torch.float32)
        if rope:
            _, sts = la.blockcausal_forward_rope(qd, kd, vd, T, f0, gh, gw, workloads.ROPE_THETA,
                                                 state_in=si, eps=workloads.EPS)
            g = la.blockcausal_backward_rope(qd, kd, vd, sts, dOd, T, f0, gh, gw,
                                             workloads.ROPE_THETA, dstates=dsts,
                                             want_dstate_in=chunked, eps=workloads.EPS)

            def run():
                return oracle.rope_blockcausal_backward(Q, K, V, bounds, dO, workloads.EPS, f0,
                                                        gh, gw, workloads.ROPE_THETA, S0=S0,
                                                        z0=z0, dS=dS, dz=dz)
        else:
            _, sts = la.blockcausal_forward(qd, kd, vd, T, state_in=si, eps=workloads.EPS)
            g = la.blockcausal_backward(qd, kd, vd, sts, dOd, T, dstates=dsts,
                                        want_dstate_in=chunked, eps=workloads.EPS)

            def run():
                return oracle.blockcausal_backward(Q, K, V, bounds, dO, workloads.EPS, S0=S0,
                                                   z0=z0, dS=dS, dz=dz)
        ref, per_s, runs = time_oracle(run, seconds_min=8.0)
        errs = {}
        for name, gt, r in zip(("dq", "dk", "dv"), g[:3], ref[:3]):
            gn = gt.double().cpu().numpy()
            errs[name] = max(normwise(gn[:, :, a:b], r[:, :, a:b], (2, 3))
                             for a, b in zip(bounds[:-1], bounds[1:]))
        if chunked:
            Sg, zg = state_parts(g[3], d)
            errs["dstate_in"] = max(normwise(Sg, ref[3], (2, 3)), normwise(zg, ref[4], (2,)))
        result["cpu_baseline"] = cpu_leg(
            B * Ns * Hs / H, per_s, runs,
            f"{'rotary ' if rope else ''}backward of {w.name}: the first {Hs} of {H} heads, "
            f"{Cs} block(s) of {T} tokens, seeded host inputs (tokens/s scaled to all {H} heads)",
            errs)
    print(json.dumps(result), flush=True)


# ---------------------------------------------------------------------------
# the temporal convolution

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
    import oracle
    import workloads

    B, T, n, P, C = TCONV[args.workload]
    F = T * n
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev).manual_seed(3000)
    log(f"drawing inputs on the GPU for {args.workload} (B={B} F={F} T={T} P={P} C={C})")
    x = torch.randn((B, F, P, C), generator=gen, device=dev).to(torch.bfloat16)
    w = torch.randn((C, 3), generator=gen, device=dev).div_(3 ** 0.5)
    b = torch.randn((C,), generator=gen, device=dev).mul_(0.1)
    cache = torch.randn((B, P, C), generator=gen, device=dev).to(torch.bfloat16)
    y = torch.empty_like(x)
    cache_out = torch.empty_like(cache)

    def step(i):
        la.temporal_conv_blockcausal(x, w, T, b, cache_in=cache, y=y, cache_out=cache_out)

    wcalls = warm_up(step, args.warmup, args.min_warmup_s)
    ms = timed_region(step, args.steps)
    # x read once, y written once, the cache read and written (taps and bias
    # are a few KB)
    nbytes = 2 * B * F * P * C * 2 + 2 * B * P * C * 2
    result = {
        "metric": "latent tokens/sec + % peak HBM BW, Mix-FFN temporal conv with chunk cache",
        "value": B * F * P / (ms * 1e-3), "unit": "latent tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_calls": wcalls,
        "min_warmup_s": args.min_warmup_s, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "frames": F, "frames_per_chunk": T,
                   "positions_per_frame": P, "channels": C, "x_y": "bf16"},
        "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "roofline": {"bound": "hbm", "kernel": "temporal_conv<true, true>",
                     "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "traffic": None,
                     "bytes_alg_per_launch": nbytes, "launch_us": ms * 1e3,
                     "source": "the timed region (one kernel per call)"},
    }
    del x, y, cache, cache_out
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        # one chunk of 21 frames at the workload's positions, the first 256
        # channels, seeded host inputs
        Cs = 256
        Fs = T
        xs, ws_, bs, cs = workloads.random_tconv(800, B, Fs, P, Cs)
        log(f"oracle leg: temporal conv, {Fs} frames x {P} positions x {Cs} channels")
        yg, cg = la.temporal_conv_chunk(to_dev(xs, dev), to_dev(ws_, dev, torch.float32),
                                        bias=to_dev(bs, dev, torch.float32),
                                        cache_in=to_dev(cs, dev))
        (yr, cr), per_s, runs = time_oracle(lambda: oracle.temporal_conv_chunk(xs, ws_, bs, cs),
                                            seconds_min=8.0)
        eo = normwise(yg.double().cpu().numpy(), yr, (2, 3))
        ec = float(np.abs(cg.double().cpu().numpy() - cr).max())
        leg = cpu_leg(B * Fs * P * Cs / C, per_s, runs,
                      f"one chunk of {Fs} frames x {P} positions, the first {Cs} of {C} channels, "
                      f"seeded host inputs (tokens/s scaled to all {C} channels)",
                      {"out": eo, "cache_abs": ec})
        leg["parity"]["bound"] = 2.0 ** -8
        leg["parity"]["metric"] = "max over (b, frame) of max|gpu - oracle| / max|oracle| (bf16 out)"
        result["cpu_baseline"] = leg
    print(json.dumps(result), flush=True)


# ---------------------------------------------------------------------------
# the headline: the 720p chunk

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--min-warmup-s", type=float, default=1.0,
                    help="continue the warm-up until this many seconds have passed")
    ap.add_argument("--sample-calls", type=int, default=60,
                    help="calls of the sampled pass with stage events (at least --steps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--kv-splits", type=int, default=0)
    ap.add_argument("--readout-workgroups", type=int, default=0,
                    help="launch option: the readout grid of the forward calls, the "
                         "key-gradient workgroups of the backward calls (0: the planner's "
                         "choice)")
    ap.add_argument("--workload", default="chunk720p",
                    choices=["chunk720p", "ceiling"] + list(OTHER) + list(BACKWARD)
                    + list(TCONV) + list(ROPE))
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
    if args.workload == "ceiling":
        bench_ceiling(args)
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
    host = {c: workloads.chunk_qkv(w, c) for c in (0, 1, 2)}

    def upload(x):
        return torch.from_numpy(x).to(dev).to(torch.bfloat16)

    q0, k0, v0 = (upload(x) for x in host[0])
    sets = []
    for chunk in (1, 2):
        q, k, v = (upload(x) for x in host[chunk])
        out = torch.empty((B, H, L, d), dtype=torch.float32, device=dev)
        st = torch.empty((B, H, d * d + d), dtype=torch.float32, device=dev)
        sets.append((q, k, v, out, st))
    del host[2]
    # the committed state after chunk 0
    _, state0 = la.global_forward(q0, k0, v0, eps=workloads.EPS)
    del q0, k0, v0
    torch.cuda.synchronize()
    splits, rtok = la.plan(B, H, L, d, kv_splits=args.kv_splits,
                           readout_workgroups=args.readout_workgroups)
    log(f"plan: kv_splits={splits} readout_workgroups={rtok}")

    def step(i, ev=None):
        q, k, v, out, st = sets[i & 1]
        la.chunk_forward(q, k, v, state0, out=out, state_out=st, eps=workloads.EPS,
                         kv_splits=args.kv_splits, readout_workgroups=args.readout_workgroups,
                         stage_events=ev)

    wcalls = warm_up(step, args.warmup, args.min_warmup_s)
    log(f"warm-up done ({wcalls} calls); timing {args.steps} steps")
    # the timed region: plain calls only
    ms = timed_region(step, args.steps)
    log(f"timed: {ms * 1e3:.1f} us/step")
    # the sampled pass: every call with stage events
    per = sampled_pass(step, max(args.steps, args.sample_calls))
    # leave sets[0] holding chunk 1's output and state
    step(0)
    torch.cuda.synchronize()

    call_b, kv_b, ro_b = bytes_alg(B, H, L, d)
    kv_ms = float(per[:, 0].mean())
    call_gbs = call_b / (ms * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": B * L / (ms * 1e-3),
        "unit": "latent tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_calls": wcalls,
        "min_warmup_s": args.min_warmup_s,
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
        "roofline": roofline("readout_sweep_bf16<64>", ro_b, per[:, 2], stored_traffic()),
        "stages_us": stage_summary(per, ["kv_partial", "state_reduce", "readout"]),
        "kv_partial_GBs": kv_b / (kv_ms * 1e-3) / 1e9,
        "mfma_frac_call": flops(B, H, L, d) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
    }
    if not args.no_cpu_baseline:
        import oracle

        log("oracle leg: the chunk-0 state, then chunk 1 against it (timed)")
        Q0, K0, V0 = host[0]
        _, S0, z0 = oracle.global_forward(Q0, K0, V0, workloads.EPS)
        del host[0], Q0, K0, V0
        Q, K, V = host[1]
        (O, S1, z1), per_s, runs = time_oracle(
            lambda: oracle.chunk_forward(Q, K, V, S0, z0, workloads.EPS))
        out, st = sets[0][3], sets[0][4]
        Sg, zg = state_parts(st, d)
        errs = {"out": normwise(out.double().cpu().numpy(), O, (2, 3)),
                "state": max(normwise(Sg, S1, (2, 3)), normwise(zg, z1, (2,)))}
        result["cpu_baseline"] = cpu_leg(
            B * L, per_s, runs,
            "the full 720p chunk (B=1, H=32, d=64, L=75,600): chunk 1 against the state the "
            "oracle derives from chunk 0, the same seeded bf16 tensors the GPU reads", errs)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
