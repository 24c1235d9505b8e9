#!/usr/bin/env python3
"""Benchmark of the MXFP4 grouped-expert MoE layer on one MI355X (gfx950).

One step is one full layer call (router logits, top-k, softmax, tile table,
gate/up + SwiGLU, down, combine) over one batch of synthetic gpt-oss-shaped
input already resident in HBM: moe_route (or, up to 16 tokens,
moe_route_tiles) + moe_build_tiles + moe_forward, and for one token the
single-launch moe_layer_one_token.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1]

Method (the SimpleLLM README, "How we measured": three runs per point, each
in a process of its own, the median reported):
  * this process never touches the GPU.  For the headline workload (default:
    the gpt-oss-20b-shaped decode layer at T=1) and for each of the other
    gpt-oss workloads (20b T=64 with a skewed router, 120b T=64, 120b
    T=4096) it starts `--runs` fresh child processes (`bench.py --child`),
    each of which measures the workload once and prints one JSON record; the
    record with the median µs/call is kept, with every run's value beside
    it.  The headline child times exactly K steps after W warmup steps (and,
    before those, 0.1 s of untimed replays that bring the GPU's clocks to
    their steady state).
  * within a child: HIP graphs, each holding one call per rotating weight
    copy, replayed back to back; exactly K steps between two events on the
    replay stream, synchronised on both sides.  R copies of the expert
    weights rotate so that R x (bytes one call touches) >= 3 x the 256 MB
    Infinity Cache (R = 1 is also timed and reported as the cache-inflated
    figure), and eager calls are timed as the stream-enqueue figure.
  * per-kernel durations: for each entry point a HIP graph of back-to-back
    launches of it alone, timed with HIP events on the launch stream; the
    dominant kernel's average launch duration gives the roofline fraction
    (for one token the whole step is one kernel, timed by the headline loop
    itself; the separate entry points are then reported as components);
  * cpu_baseline: the float64 oracle on this host's cores, on a bounded
    sample of each workload, run by this (GPU-free) process.
Prints one JSON line.  Under a profiler (or with --child) the measurement
runs in this process instead, once, with no child processes.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer µs/call + HBM GB/s at T=1,64; TFLOP/s (MFMA util) at T=4096"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
INFINITY_CACHE = 256 << 20
GPTOSS_WORKLOADS = (1, 2, 3, 4)
CHILD_TIMEOUT_S = 300
BURN_IN_S = 0.1              # untimed replays before the warmup steps (see measure)


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", type=int, default=1, choices=range(7))
    ap.add_argument("--others", default=None,
                    help="comma-separated workload ids measured beside the headline "
                         "(default: the other gpt-oss workloads; 'none' for none)")
    ap.add_argument("--runs", type=int, default=3, help="child processes per workload")
    ap.add_argument("--rotations", type=int, default=0, help="weight copies (0 = auto)")
    ap.add_argument("--bm", type=int, default=None, choices=(16, 32, 64, 128),
                    help="token tile (default: the library's moe_pick_bm rule)")
    ap.add_argument("--layout", default="blocked", choices=("canonical", "blocked"),
                    help="byte layout of the packed expert codes (blocked: repacked at load)")
    ap.add_argument("--no-graph", action="store_true", help="time eager calls instead of graphs")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (known bytes) for counter scaling")
    ap.add_argument("--child", action="store_true",
                    help="measure in this process (one run, no CPU baseline unless asked)")
    return ap.parse_args(argv)


def expert_bytes(H, I):
    return 2 * I * H // 2 + 2 * I * H // 32 + H * I // 2 + H * I // 32


def gateup_bytes(H, I):
    return 2 * I * H // 2 + 2 * I * H // 32


# ------------------------------------------------------------ CPU baseline --

def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, seconds):
    """The float64 oracle, as it stands, on this host.  Up to 64 tokens: whole
    layer calls, repeated for about `seconds`.  Above that the oracle's own
    steps are timed on a sample: routing and the tile table for every token,
    the expert FFN (decode + matmuls) of a sample of the touched experts with
    all their rows, scaled by touched / sampled, and the combine."""
    import numpy as np
    import oracle
    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = affinity
    T, k = inp["T"], inp["k"]
    if T <= 64:
        calls, t0 = 0, time.perf_counter()
        while True:
            oracle.moe_layer(inp, BM=16)
            calls += 1
            el = time.perf_counter() - t0
            if el >= seconds or calls >= 50:
                break
        per_call = el / calls
        what = f"full layer (all {T} tokens); {calls} call(s) in {el:.1f} s"
    else:
        t0 = time.perf_counter()
        ids, w, _ = oracle.route(inp["x"], inp["w_router"], inp.get("bias"), k,
                                 inp.get("gating", "softmax"))
        E = inp["w13_q"].shape[0]
        off, srt, _, _ = oracle.build_tiles(ids, E, 128)
        x64 = oracle.bf16_to_f64(inp["x"])
        t_route = time.perf_counter() - t0
        touched = [e for e in range(E) if off[e + 1] > off[e]]
        y = np.zeros((T * k, inp["H"]))
        t1, done = time.perf_counter(), 0
        for e in touched[:: max(1, len(touched) // 64)]:
            slots = srt[off[e]:off[e + 1]].astype(np.int64)
            y[slots] = oracle.expert_ffn(x64[slots // k], inp["w13_q"][e], inp["w13_s"][e],
                                         inp["w2_q"][e], inp["w2_s"][e])
            done += 1
            if time.perf_counter() - t1 >= seconds:
                break
        t_ffn = time.perf_counter() - t1
        t2 = time.perf_counter()
        oracle.combine(y, w)
        t_comb = time.perf_counter() - t2
        per_call = t_route + t_ffn * len(touched) / done + t_comb
        what = (f"routing + tile table for all {T} tokens ({t_route:.2f} s), expert FFN of "
                f"{done} of the {len(touched)} touched experts with all their rows "
                f"({t_ffn:.1f} s, scaled by {len(touched)}/{done}), combine ({t_comb:.2f} s)")
    return {"value": round(per_call * 1e6, 1), "unit": "us/call", "cores": int(threads),
            "kind": "oracle", "sample": f"{what}; float64 numpy",
            "affinity_cores": affinity, "blas_threads": int(threads), "cpu_model": cpu_model()}


# ---------------------------------------------------- counter cross-check --

def _source_hash(src_rel: str) -> str:
    """sha256 prefix of a kernel source together with every local header it
    includes (recursively), so an edit to any of them invalidates counters."""
    import hashlib
    seen, order = set(), []

    def visit(path):
        path = os.path.normpath(path)
        if path in seen or not os.path.exists(path):
            return
        seen.add(path)
        order.append(path)
        for m in re.finditer(r'#include\s+"([^"]+)"', open(path, encoding="utf-8").read()):
            visit(os.path.join(os.path.dirname(path), m.group(1)))

    visit(os.path.join(ROOT, src_rel))
    h = hashlib.sha256()
    for path in order:
        h.update(os.path.relpath(path, ROOT).encode())
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` at `workload` from the rocprofv3
    FETCH_SIZE/WRITE_SIZE summary in profiles/, or None when there is no row
    or the kernel source (or a header it includes) changed since the
    counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic_counters.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) != 9 or cells[0] != workload or cells[1] != kernel:
            continue
        if not os.path.exists(os.path.join(ROOT, cells[7])) or _source_hash(cells[7]) != cells[8]:
            return None
        return int(cells[6])
    return None


# ------------------------------------------------ one measurement (child) --

def measure(args) -> dict:
    """Measures one workload in this process (the GPU is used here)."""
    import numpy as np
    import torch

    import mxfp4_grouped_expert_amd as moe
    from moe_inputs import make_workload

    wid = args.workload
    inp = make_workload(wid)
    T, H, E, k, I = inp["T"], inp["H"], inp["E"], inp["k"], inp["I"]
    steps = args.steps if args.steps is not None else (400 if T <= 64 else 20)
    warmup = args.warmup if args.warmup is not None else (32 if T <= 64 else 3)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    moe.load()

    x = torch.from_numpy(inp["x"].view(np.int16)).to(dev)
    wr = torch.from_numpy(inp["w_router"]).to(dev)
    bias = None if inp["bias"] is None else torch.from_numpy(inp["bias"]).to(dev)
    w0 = [torch.from_numpy(inp[key]).to(dev) for key in ("w13_q", "w13_s", "w2_q", "w2_s")]

    ids, _, _ = moe.moe_route(x, wr, bias, k)
    n_touched = int(torch.unique(ids).numel())
    touched = n_touched * expert_bytes(H, I) + E * H * 4 + (E * 4 if bias is not None else 0) \
        + 2 * T * H * 2
    layer_flops = 2 * T * k * 3 * I * H + 2 * T * E * H
    R = args.rotations or max(1, min(32, math.ceil(3 * INFINITY_CACHE / touched)))
    layer = moe.MoeLayer(wr, bias, *w0, k, gating=inp["gating"], layout=args.layout).plan(T, BM=args.bm)
    w0 = [layer.w13_q, layer.w13_s, layer.w2_q, layer.w2_s]  # in the layer's layout
    copies = [w0] + [[w.clone() for w in w0] for _ in range(R - 1)]
    BM = layer.BM
    del inp["w13_q"], inp["w13_s"], inp["w2_q"], inp["w2_s"]

    def step(r):
        layer.set_weights(*copies[r])
        return layer(x)

    for i in range(max(warmup, R)):
        step(i % R)
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()

    def capture(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for r in range(n):
                    fn(r)
        torch.cuda.synchronize()
        return g

    def time_graph(g, reps, per):
        """µs per call of `reps` replays of a graph holding `per` calls."""
        with torch.cuda.stream(stream):
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * per)

    mode = "hip_graph"
    graphs = []
    # calls per graph: a multiple of the R weight copies and at least 8, so
    # that one replay's fixed cost is spread over several calls
    G = R * max(1, math.ceil(8 / R))
    if not args.no_graph:
        try:
            graphs.append(capture(lambda r: step(r % R), G))
            if steps % G:
                graphs.append(capture(lambda r: step(r % R), steps % G))
        except Exception as exc:  # graph capture unavailable: time eagerly
            print(f"graph capture failed ({exc}); timing eager calls", file=sys.stderr)
            graphs = []
    if not graphs:
        mode = "eager"

    # Burn-in: after idling, the GPU runs at lower clocks for the first few
    # tens of milliseconds of sustained work (µs per call over consecutive
    # 16-call windows from a cold start: 1,154, 1,035, then 1,000-1,007 at
    # the 4k-token prefill; 18.6, then 18.15 at one token), so every run
    # replays its workload for BURN_IN_S of wall time, untimed, before the W
    # warmup steps, and the K timed steps measure the steady state that a
    # serving loop runs in.
    with torch.cuda.stream(stream):
        t_burn = time.perf_counter()
        i = 0
        while time.perf_counter() - t_burn < BURN_IN_S:
            if graphs:
                graphs[0].replay()
            else:
                step(i % R)
                i += 1
            torch.cuda.synchronize()

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        if graphs:
            for _ in range(max(1, warmup // G)):
                graphs[0].replay()
            torch.cuda.synchronize()
            start.record(stream)
            for _ in range(steps // G):
                graphs[0].replay()
            if steps % G:
                graphs[1].replay()
            end.record(stream)
        else:
            for i in range(warmup):
                step(i % R)
            torch.cuda.synchronize()
            start.record(stream)
            for i in range(steps):
                step(i % R)
            end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / steps
    us = ms_per_step * 1e3

    # stream-enqueue figure: the same K steps as eager calls from the host
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            step(i % R)
        e1.record(stream)
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) * 1e3 / steps
    # cache-inflated figure: one weight copy, so repeated calls may hit the
    # Infinity Cache
    r1_us = None
    if graphs:
        L1 = 16
        g1 = capture(lambda r: step(0), L1)
        r1_us = time_graph(g1, max(1, min(steps, 256) // L1), L1)
        del g1

    # ---- per-kernel durations: for each entry point, a HIP graph of max(R, 16)
    # back-to-back launches of it alone (weights rotating as in the headline
    # loop), replayed between two events on the launch stream.  The layer
    # buffers hold a valid routing and tile table from the calls above.
    parts = {
        ("route_tiles" if layer.fused else "route"): lambda r: layer.route_only(x),
        **({} if layer.fused else {"tiles": lambda r: layer.tiles_only()}),
        "gateup": lambda r: (layer.set_weights(*copies[r]), layer.gateup_only(x)),
        "down": lambda r: (layer.set_weights(*copies[r]), layer.down_only()),
        "combine": lambda r: layer.combine_only(),
    }
    kernel_us = {}
    # at least 16 launches per graph, so one replay's fixed cost does not
    # land on a short kernel (weights still rotate over the R copies)
    L = max(R, 16)
    reps = max(1, min(steps, 256) // L)
    for name, fn in parts.items():
        if graphs:
            g = capture(lambda r, fn=fn: fn(r % R), L)
            kernel_us[name] = time_graph(g, reps, L)
            del g
        else:
            with torch.cuda.stream(stream):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    for r in range(L):
                        fn(r % R)
                e1.record(stream)
            torch.cuda.synchronize()
            kernel_us[name] = e0.elapsed_time(e1) * 1e3 / (reps * L)

    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    gu_us = kernel_us["gateup"]
    # the gate/up GEMM runs on the 128-row matrix-core kernel when the library
    # picks it (expert_mma_ok: 128-row tiles, >= 32 slots per expert, the
    # scale slab of K = H in its 48 KB: K <= 3072, or K = 4096)
    KB = H // 32
    slab = 2 * (((15 if KB % 16 else 0) + 192 * KB + 15) // 16)
    uses_mma = BM == 128 and T * k >= 32 * E and slab <= 6 * 512
    traffic_key = inp["name"] + ("" if args.layout == "canonical" else "/" + args.layout)
    gu_bytes = n_touched * gateup_bytes(H, I) + T * H * 2 + T * k * I * 2
    gu_flops = 2 * T * k * 2 * I * H
    if layer.one_launch:
        # the step is one launch: every byte the layer touches, per launch of it
        achieved = touched / (us * 1e-6) / 1e9
        kname = "moe_layer_one_token_kernel"
        roof = {"kernel": kname, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(traffic_key, kname),
                "algorithmic_bytes_per_launch": touched, "avg_launch_us": round(us, 2)}
    elif T <= 64 or not uses_mma or gu_flops < gu_bytes * BF16_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3:
        # weight streaming: fewer flops per byte than the MFMA/HBM peak ratio
        achieved = gu_bytes / (gu_us * 1e-6) / 1e9
        kname = "expert_mma_kernel<gate/up>" if uses_mma else "expert_gemm_kernel<gate/up>"
        roof = {"kernel": kname, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(traffic_key, kname),
                "algorithmic_bytes_per_launch": gu_bytes, "avg_launch_us": round(gu_us, 2)}
    else:
        achieved = gu_flops / (gu_us * 1e-6) / 1e12
        kname = "expert_mma_kernel<gate/up>"
        roof = {"kernel": kname, "bound": "mfma", "achieved": round(achieved, 1),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(traffic_key, kname),
                "algorithmic_flops_per_launch": gu_flops, "avg_launch_us": round(gu_us, 2)}

    gbps = touched / (us * 1e-6) / 1e9
    tflops = layer_flops / (us * 1e-6) / 1e12
    return {
        "metric": METRIC,
        "value": round(us, 2),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded MXFP4 layer of the workload's shape, no checkpoint)",
        "config": {"workload": inp["name"], "T": T, "H": H, "E": E, "k": k, "I": I, "BM": BM,
                   "experts_touched": n_touched, "weight_rotations": R, "timing": mode,
                   "calls_per_graph": G if graphs else None,
                   "gating": inp["gating"], "weight_layout": args.layout,
                   "routing": ("moe_layer_one_token" if layer.one_launch else
                               "moe_route_tiles" if layer.fused else
                               "moe_route+moe_build_tiles")},
        "tokens_per_s": round(T / (us * 1e-6), 1),
        "hbm_gbps": round(gbps, 1),
        "hbm_frac": round(gbps / HBM_PEAK_GBS, 4),
        "tflops": round(tflops, 3),
        "tflops_frac": round(tflops / BF16_PEAK_TFLOPS, 4),
        "algorithmic_bytes_per_call": touched,
        "algorithmic_flops_per_call": layer_flops,
        "stream_enqueue_us": round(eager_us, 2),
        "cache_inflated_r1_us": None if r1_us is None else round(r1_us, 2),
        "kernel_us": {n: round(v, 2) for n, v in kernel_us.items()},
        "roofline": roof,
    }


# --------------------------------------------------- orchestration (parent) --

def _under_profiler() -> bool:
    return any(key.startswith("ROCPROF") for key in os.environ)


def run_children(args, wid, steps, warmup):
    """`args.runs` fresh processes measuring workload `wid`; returns their
    records sorted by value (µs/call)."""
    cmd = [sys.executable, os.path.abspath(__file__), "--child", "--no-cpu-baseline",
           "--workload", str(wid), "--layout", args.layout]
    if steps is not None:
        cmd += ["--steps", str(steps)]
    if warmup is not None:
        cmd += ["--warmup", str(warmup)]
    if args.rotations:
        cmd += ["--rotations", str(args.rotations)]
    if args.bm is not None:
        cmd += ["--bm", str(args.bm)]
    if args.no_graph:
        cmd += ["--no-graph"]
    recs = []
    for run in range(args.runs):
        t0 = time.perf_counter()
        p = subprocess.run(cmd, stdout=subprocess.PIPE, text=True, timeout=CHILD_TIMEOUT_S)
        if p.returncode != 0:
            print(f"bench child (workload {wid}, run {run}) failed with status {p.returncode}",
                  file=sys.stderr)
            sys.exit(p.returncode if p.returncode > 0 else 1)
        line = [ln for ln in p.stdout.splitlines() if ln.startswith("{")][-1]
        recs.append(json.loads(line))
        print(f"[bench] workload {wid} run {run}: {recs[-1]['value']} us/call "
              f"({time.perf_counter() - t0:.1f} s)", file=sys.stderr, flush=True)
    return sorted(recs, key=lambda r: r["value"])


def median_record(recs):
    rec = dict(recs[(len(recs) - 1) // 2])  # recs are sorted: the (lower) middle run
    vals = [r["value"] for r in recs]
    rec["runs_us"] = vals
    rec["value"] = round(statistics.median(vals), 2)
    rec["method"] = f"median of {len(recs)} processes"
    return rec


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.child or _under_profiler():
        result = measure(args)
        if not args.no_cpu_baseline and not args.child:
            from moe_inputs import make_workload
            result["cpu_baseline"] = cpu_baseline(make_workload(args.workload), args.cpu_seconds)
        print(json.dumps(result), flush=True)
        return

    # this process only starts children and runs the CPU oracle
    from moe_inputs import make_workload
    others = ([w for w in GPTOSS_WORKLOADS if w != args.workload] if args.others is None
              else [] if args.others == "none" else [int(w) for w in args.others.split(",")])
    result = median_record(run_children(args, args.workload, args.steps, args.warmup))
    subs = {}
    for wid in others:
        subs[wid] = median_record(run_children(args, wid, None, None))
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(make_workload(args.workload), args.cpu_seconds)
        for wid in others:
            subs[wid]["cpu_baseline"] = cpu_baseline(make_workload(wid), args.cpu_seconds)
    keep = ("value", "unit", "method", "runs_us", "steps", "warmup", "ms_per_step", "config",
            "tokens_per_s", "hbm_gbps", "hbm_frac", "tflops", "tflops_frac",
            "algorithmic_bytes_per_call", "algorithmic_flops_per_call", "stream_enqueue_us",
            "cache_inflated_r1_us", "kernel_us", "roofline", "cpu_baseline")
    result["workloads"] = {subs[w]["config"]["workload"]: {key: subs[w][key] for key in keep
                                                            if key in subs[w]}
                           for w in others}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
