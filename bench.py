#!/usr/bin/env python3
"""Benchmark of the MXFP4 grouped-expert MoE layer on one MI355X (gfx950).

One step is one full layer call (router logits, top-k, softmax, tile table,
gate/up + SwiGLU, down, combine) over one batch of synthetic gpt-oss-shaped
input already resident in HBM: moe_route (or, up to 16 tokens,
moe_route_tiles) + moe_build_tiles + moe_forward, and for one token the
single-launch moe_layer_one_token.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1]

Default workload: the gpt-oss-20b-shaped decode layer at T=1 (H=2880, E=32,
k=4, I=2880).  Timing:
  * headline: HIP graphs, each holding one call per rotating weight copy,
    replayed back to back; exactly K steps between two events on the replay
    stream, synchronised on both sides.  R copies of the expert weights are
    rotated so that R x (bytes one call touches) >= 3 x the 256 MB Infinity
    Cache, which keeps repeated calls from being served by it;
  * per-kernel durations: for each entry point a HIP graph of back-to-back
    launches of it alone, timed with HIP events on the launch stream; the
    dominant kernel's average launch duration gives the roofline fraction
    (for one token the whole step is one kernel, timed by the headline loop
    itself; the separate entry points are then reported as components);
  * cpu_baseline: the float64 oracle on this host's cores, on a bounded
    sample of the same workload.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer µs/call + HBM GB/s at T=1,64; TFLOP/s (MFMA util) at T=4096"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
INFINITY_CACHE = 256 << 20


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", type=int, default=1, choices=range(7))
    ap.add_argument("--rotations", type=int, default=0, help="weight copies (0 = auto)")
    ap.add_argument("--bm", type=int, default=None, choices=(16, 32, 64, 128),
                    help="token tile (default: the library's moe_pick_bm rule)")
    ap.add_argument("--layout", default="blocked", choices=("canonical", "blocked"),
                    help="byte layout of the packed expert codes (blocked: repacked at load)")
    ap.add_argument("--no-graph", action="store_true", help="time eager calls instead of graphs")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (known bytes) for counter scaling")
    return ap.parse_args()


def expert_bytes(H, I):
    return 2 * I * H // 2 + 2 * I * H // 32 + H * I // 2 + H * I // 32


def gateup_bytes(H, I):
    return 2 * I * H // 2 + 2 * I * H // 32


def cpu_baseline(inp, seconds):
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    T = inp["T"]
    if T <= 64:
        tokens, what = None, f"full layer (all {T} tokens)"
    else:
        tokens = np.arange(0, T, T // 16)
        what = (f"routing + tile table for all {T} tokens, expert FFN + combine for "
                f"{len(tokens)} evenly spaced tokens, scaled by {T}/{len(tokens)}")
    calls, t0 = 0, time.perf_counter()
    while True:
        oracle.moe_layer(inp, BM=16, tokens=tokens)
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds or calls >= 50:
            break
    per_call = el / calls
    if tokens is not None:
        per_call *= T / len(tokens)
    return {"value": round(per_call * 1e6, 1), "unit": "us/call", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{what}; {calls} call(s) in {el:.1f} s of float64 numpy"}


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` at `workload` from the rocprofv3
    FETCH_SIZE/WRITE_SIZE summary in profiles/, or None when there is no row
    or the kernel source changed since the counters were taken."""
    import hashlib
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        "traffic_counters.md")
    if not os.path.exists(path):
        return None
    root = os.path.dirname(path)[: -len("profiles")]
    for line in open(path):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) != 9 or cells[0] != workload or cells[1] != kernel:
            continue
        src = os.path.join(root, cells[7])
        if not os.path.exists(src):
            return None
        if hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] != cells[8]:
            return None
        return int(cells[6])
    return None


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

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
    mode = "hip_graph"
    graphs = []
    if not args.no_graph:
        try:
            with torch.cuda.stream(stream):
                g_full = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g_full, stream=stream):
                    for r in range(R):
                        step(r)
                graphs.append(g_full)
                rem = steps % R
                if rem:
                    g_rem = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g_rem, stream=stream):
                        for r in range(rem):
                            step(r)
                    graphs.append(g_rem)
            torch.cuda.synchronize()
        except Exception as exc:  # graph capture unavailable: time eagerly
            print(f"graph capture failed ({exc}); timing eager calls", file=sys.stderr)
            graphs = []
    if not graphs:
        mode = "eager"

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        if graphs:
            for _ in range(max(1, warmup // R)):
                graphs[0].replay()
            torch.cuda.synchronize()
            start.record(stream)
            for _ in range(steps // R):
                graphs[0].replay()
            if steps % R:
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
        with torch.cuda.stream(stream):
            if graphs:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for r in range(L):
                        fn(r % R)
                g.replay()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    g.replay()
                e1.record(stream)
            else:
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
    # the 128-row matrix-core kernels run when the library picks them
    # (expert_mma_ok: 128-row tiles, K <= 3072, >= 32 slots per expert)
    uses_mma = BM == 128 and max(H, I) <= 3072 and T * k >= 32 * E
    traffic_key = inp["name"] + ("" if args.layout == "canonical" else "/" + args.layout)
    if layer.one_launch:
        # the step is one launch: every byte the layer touches, per launch of it
        achieved = touched / (us * 1e-6) / 1e9
        kname = "moe_layer_one_token_kernel"
        roof = {"kernel": kname, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(traffic_key, kname),
                "algorithmic_bytes_per_launch": touched, "avg_launch_us": round(us, 2)}
    elif T <= 64 or not uses_mma:
        gu_bytes = n_touched * gateup_bytes(H, I) + T * H * 2 + T * k * I * 2
        achieved = gu_bytes / (gu_us * 1e-6) / 1e9
        kname = "expert_gemm_kernel<gate/up>"
        roof = {"kernel": kname, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(traffic_key, kname),
                "algorithmic_bytes_per_launch": gu_bytes, "avg_launch_us": round(gu_us, 2)}
    else:
        gu_flops = 2 * T * k * 2 * I * H
        achieved = gu_flops / (gu_us * 1e-6) / 1e12
        kname = "expert_mma_kernel<gate/up>"
        roof = {"kernel": kname, "bound": "mfma", "achieved": round(achieved, 1),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(traffic_key, kname),
                "algorithmic_flops_per_launch": gu_flops, "avg_launch_us": round(gu_us, 2)}

    gbps = touched / (us * 1e-6) / 1e9
    tflops = layer_flops / (us * 1e-6) / 1e12
    result = {
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
                   "gating": inp["gating"], "weight_layout": args.layout,
                   "routing": ("moe_layer_one_token" if layer.one_launch else
                               "moe_route_tiles" if layer.fused else
                               "moe_route+moe_build_tiles")},
        "tokens_per_s": round(T / (us * 1e-6), 1),
        "hbm_gbps": round(gbps, 1),
        "hbm_frac": round(gbps / HBM_PEAK_GBS, 4),
        "tflops": round(tflops, 3),
        "algorithmic_bytes_per_call": touched,
        "kernel_us": {n: round(v, 2) for n, v in kernel_us.items()},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        full = make_workload(wid)
        result["cpu_baseline"] = cpu_baseline(full, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
