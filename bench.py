#!/usr/bin/env python3
"""Throughput of M=1 attention over a resident KV-cache prefix on one MI355X.

Workload (one "step"): the decode shape H_q = H_kv = 8, N = 2048, D = 128, M = 1,
fp16 K/V resident in 32 independent (sid, layer) slots, queried back-to-back, fp32
out + LSE per layer - the shape the pages quote their M=1 latency on. Inputs are the
seeded synthetic generators (K with per-channel lognormal(0, 0.5) scales, Q and V
N(0, 1)); all of it is resident in HBM before the timed region starts.

Timed region: K steps on one HIP stream. Default (--mode layers): a step is one
pion_prefix_query_layers call covering the 32 layers (one kernel launch). --mode calls:
a step is 32 pion_prefix_query calls. The step's calls are captured once into a HIP
graph (after an eager warm-up) and the graph is replayed per step (--eager issues them
from the host instead). Per-launch duration: after the timed region, the same calls
are issued eagerly with a HIP event pair around each one on the launch stream; the
roofline figure uses the algorithmic K/V bytes of one launch (per layer: 8 heads x
2048 tokens x (K + V) x 128 x 2 B = 8,388,608 B; 268,435,456 B for the 32-layer launch)
over the mean of those durations.

cpu_baseline: the fp64 numpy oracle as it stands, one thread, on whole 32-layer passes
of the same inputs, repeated for about 10 s.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="issue calls from the host, no graph")
    ap.add_argument("--mode", choices=["layers", "calls"], default="layers",
                    help="layers: one pion_prefix_query_layers launch per step; "
                         "calls: 32 pion_prefix_query calls per step")
    return ap.parse_args()


def cpu_baseline(case, inputs, seconds):
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits
    passes = 0
    t0 = time.perf_counter()
    with threadpool_limits(1):
        while True:
            for inp in inputs:
                oracle.prefix_query(inp.Q, inp.K, inp.V)
            passes += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    bytes_per_pass = case.layers * case.H_kv * case.N * case.D * 2 * 2
    return {"value": round(bytes_per_pass * passes / el / 1e9, 4), "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{passes} whole 32-layer passes of the decode workload "
                      f"({el:.1f} s, fp64 numpy, 1 thread)"}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import kv_cache_prefix_amd as kp
    import synth

    case = synth.DECODE
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inputs = [synth.generate(case, l) for l in range(case.layers)]
    sid = "bench-decode"
    Qs, outs, lses = [], [], []
    for l, inp in enumerate(inputs):
        K = torch.from_numpy(inp.K).to(dev)
        V = torch.from_numpy(inp.V).to(dev)
        kp.pion_prefix_store(sid, l, K, V)
        Qs.append(torch.from_numpy(inp.Q).to(dev))
        outs.append(torch.empty((case.H_q, 1, case.D), dtype=torch.float32, device=dev))
        lses.append(torch.empty((case.H_q, 1), dtype=torch.float32, device=dev))
    torch.cuda.synchronize()

    lib = kp.lib()
    sidb = sid.encode()
    stream = torch.cuda.Stream(device=dev)
    # raw arguments, marshalled once
    Qall = torch.stack(Qs).contiguous()
    out_all = torch.empty((case.layers, case.H_q, 1, case.D), dtype=torch.float32, device=dev)
    lse_all = torch.empty((case.layers, case.H_q, 1), dtype=torch.float32, device=dev)
    if args.mode == "layers":
        fn = lib.pion_prefix_query_layers
        calls = [(sidb, 0, case.layers, case.H_q, case.D, 1, Qall.data_ptr(), None,
                  out_all.data_ptr(), lse_all.data_ptr())]
        outs = list(out_all)
        lses = list(lse_all)
    else:
        fn = lib.pion_prefix_query
        calls = [(sidb, l, case.H_q, case.D, 1, Qs[l].data_ptr(), None, outs[l].data_ptr(),
                  lses[l].data_ptr()) for l in range(case.layers)]
    starts = [torch.cuda.Event(enable_timing=True) for _ in calls]
    ends = [torch.cuda.Event(enable_timing=True) for _ in calls]

    def step(timed_events: bool):
        h = torch.cuda.current_stream().cuda_stream
        for i, c in enumerate(calls):
            if timed_events:
                starts[i].record()
            rc = fn(*c, h)
            if rc != 0:
                raise kp.PionError(rc, fn.__name__)
            if timed_events:
                ends[i].record()

    with torch.cuda.stream(stream):
        for _ in range(3):
            step(False)
    torch.cuda.synchronize()

    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step(False)
        torch.cuda.synchronize()

    def run(n):
        with torch.cuda.stream(stream):
            for _ in range(n):
                if graph is not None:
                    graph.replay()
                else:
                    step(False)

    run(args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-launch duration: the same calls issued eagerly with a HIP event pair around
    # each one on the launch stream (the kernel runs alone between its events)
    launch_ms = []
    with torch.cuda.stream(stream):
        for _ in range(max(1, min(args.steps, 50))):
            step(True)
            torch.cuda.synchronize()
            launch_ms += [s.elapsed_time(e) for s, e in zip(starts, ends)]
    ms_per_step = wall * 1e3 / args.steps
    avg_launch_us = 1e3 * float(np.mean(launch_ms))
    bytes_per_layer = case.H_kv * case.N * case.D * 2 * 2
    bytes_per_step = bytes_per_layer * case.layers
    bytes_per_launch = bytes_per_step // len(calls)
    value = bytes_per_step / (ms_per_step * 1e-3) / 1e9
    achieved = bytes_per_launch / (avg_launch_us * 1e-6) / 1e9

    # parity spot check of the last step's outputs (layer 0 and 31) against the oracle
    import oracle
    for l in (0, case.layers - 1):
        ref, ref_lse = oracle.prefix_query(inputs[l].Q, inputs[l].K, inputs[l].V)
        err = float(np.max(np.abs(outs[l].cpu().numpy() - ref)))
        lerr = float(np.max(np.abs(lses[l].cpu().numpy() - ref_lse)))
        if not (err <= 2e-3 and lerr <= 1e-4):
            raise SystemExit(f"bench outputs disagree with the oracle: {err} {lerr}")

    cpu = None if args.no_cpu_baseline else cpu_baseline(case, inputs, args.cpu_seconds)
    kp.pion_prefix_drop(sid, -1)

    line = {
        "metric": "prefix-attn K/V GB/s (M=1) & TFLOP/s (batched-Q), % of MI355X roofline",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 K/V, fp32 accumulate",
        "data": "synthetic (seeded numpy: K N(0,1) x lognormal(0,0.5) per channel, Q/V N(0,1))",
        "config": {"workload": "M=1 prefix attention, decode shape H_q=H_kv=8 N=2048 D=128, "
                               "32 resident layers queried back-to-back per step",
                   "entry": fn.__name__,
                   "launches_per_step": len(calls),
                   "launch": "eager" if graph is None else "hip-graph replay",
                   "bytes_per_step": bytes_per_step},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None,
                     "kernel": "attn_split_kernel<128,1,4,0> (split-KV decode + in-kernel merge)",
                     "bytes_per_launch": bytes_per_launch,
                     "avg_launch_us": round(avg_launch_us, 3)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
