#!/usr/bin/env python3
"""Throughput of attention over a resident KV-cache prefix on one MI355X.

Default workload (--config 2, one "step"): the decode shape H_q = H_kv = 8, N = 2048,
D = 128, M = 1, fp16 K/V resident in 32 independent (sid, layer) slots, fp32 out + LSE
per layer - the shape the pages quote their M=1 latency on. Inputs come from the
seeded synthetic generators (K with per-channel lognormal(0, 0.5) scales, Q and V
N(0, 1)); all of it is resident in HBM before the timed region starts.
  --mode layers (default): a step is one pion_prefix_query_layers call covering the 32
      layers (one kernel launch), issued eagerly.
  --mode calls: a step is 32 pion_prefix_query calls, captured once into a HIP graph
      (after an eager warm-up) and replayed per step (--eager: issued from the host).

Other workloads, one call per step (for the design notes; the default run is the one
above): --config 1 tiny dense query; --config 3 fused batched-Q prefill (TFLOP/s);
--config 4 mlx4g32 decode, 16 layers per launch (GB/s of resident codes/scales/biases,
plus the single-query latency); --config 5 sparse-auto
fused query (us/query); --config 6 QUERY_SPARSE over caller-supplied indices (us/query,
GB/s of gathered rows); --config 7 V-store fetch of whole layers from mlx4g32 records to
fp32 (GB/s read + written), with the whole-call time of a WARM rehydrate beside it;
--config 8 the decode step at every supported head dim and with fp32-resident slots
(configs 6, 7 and 8 are not headline workloads).

Timing: wall clock over K steps between device synchronizations; a HIP event pair on
the launch stream brackets the same timed region, and its elapsed time over the number
of launches is the mean launch duration (back-to-back launches, so inter-kernel gaps
count against the kernel). The roofline figure is the algorithmic bytes (or flops) of
one launch over that duration.

Cold memory-side cache: MI355X keeps up to 256 MB of recently used lines in its
memory-side (infinity) cache. The M=1 workloads therefore rotate over copies of their
resident data whose total is well above that (config 2: two 32-layer sets, 537 MB;
config 4: two sets of 16 layers, 1.34 GB; config 5: 4 slots), so each step reads data the previous
steps have evicted; `value` is that cold figure. `warm` repeats one set every step and
is reported beside it, labelled.

The default run reports both halves of the metric in one JSON line: `value` is the M=1
decode figure above (GB/s), and `batched_q` the fused batched-Q prefill (--config 3's
workload, TFLOP/s) with its own roofline and CPU baseline; `stream_ceiling` is a plain
streaming read of 1 GiB timed in the same run (the achievable HBM read rate), and
`batched_q.mfma_ceiling` fp16 MFMA products alone on every SIMD (the achievable matrix
rate under full load).

cpu_baseline (default run and --config 3): the fp64 numpy oracle as it stands, timed on
the host before the GPU is touched: worker processes (one BLAS thread each) over all
usable host cores (at most 16) on a fixed sample of the workload - whole 32-layer decode
passes, or every row of one prefill step - median of 3 runs, with the 1-thread figure of
a smaller sample beside it (`single_thread`). Other configs: one thread, about 10 s.
The same leg checks the GPU's results of the run against the oracle on the same inputs
(exiting on a disagreement; the prefill's max-abs errors go into its roofline object):
it is the only part of the bench that calls the oracle, and --no-cpu-baseline skips it.
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

# HBM bytes per launch, from rocprofv3 FETCH_SIZE / WRITE_SIZE counter passes scaled by
# the same counters on a plain 256 MiB copy (FETCH_SIZE x 1.9998, WRITE_SIZE x 1.0).
# Each figure is valid only for the kernel sources it was taken on (sha256 of the listed
# files, in order); any other source reports null.
DECODE_TRAFFIC = {"sources": ("attn_partial.hip", "split_common.h", "kernels.h"),
                  "sources_sha256": "5da6a98a744fbd32523d1ee6332b086633c214cfb42a54dc2c46e4d4279774b4",
                  "bytes_per_launch": 268719091}
# One fused prefill call (H_q 24, N 4096, M = S_suf = 512): prefill_kernel<128> reads
# 22,317,556 B and writes 15,979,110 B (the five splits' fp16 partials and their
# log-sum-exps), prefill_merge_kernel<128> reads 16,065,150 B and writes 6,340,608 B (out
# and lse).
PREFILL_TRAFFIC = {"sources": ("prefill_mfma.hip", "mfma_common.h", "kernels.h"),
                   "sources_sha256": "a70705e19e6f3443d27f57a953f484ffcc7973ef30d1d3278357953cba96ec0f",
                   "bytes_per_launch": 60702424}
# The 16-layer mlx4g32 decode launch (H_q 24, H_kv 8, N 32768): mlx4_mfma_kernel<8>
# reads 671,929,782 B (671,088,640 algorithmic) and writes 644,096 B.
MLX4_TRAFFIC = {"sources": ("attn_mlx4_mfma.hip", "mfma_common.h", "split_common.h", "kernels.h"),
                "sources_sha256": "88898101b5fd8c21a66c4048be28116ba7a71469c019597a634d56efb0282a31",
                "bytes_per_launch": 672573878}


def kernel_sources_sha256(files=DECODE_TRAFFIC["sources"]):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "kv_cache_prefix_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(entry):
    """The counted bytes per launch while the sources match the ones counted, else None."""
    ok = kernel_sources_sha256(entry["sources"]) == entry["sources_sha256"]
    return entry["bytes_per_launch"] if ok else None


FP16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "prefix-attn K/V GB/s (M=1) & TFLOP/s (batched-Q), % of MI355X roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5, 6, 7, 8])
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kmean-builds", type=int, default=0,
                    help="config 5: after the timed queries, rebuild the block means this many "
                         "times (store a slot again, query it once; untimed, for a kernel trace)")
    ap.add_argument("--eager", action="store_true", help="calls mode: no graph")
    ap.add_argument("--streams", type=int, default=1,
                    help="calls mode: the 32 layer calls of a step go round-robin to this "
                         "many streams (independent calls overlap), joined at the step end")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes (a known-size "
                         "reference for the HBM byte counters) and exit")
    ap.add_argument("--mode", choices=["layers", "calls"], default="layers",
                    help="config 2: one pion_prefix_query_layers launch per step, "
                         "or 32 pion_prefix_query calls per step")
    return ap.parse_args()


class Timed:
    """Times steps: `steps` is a list of host functions issuing ABI calls on the current
    stream; step i of the timed run is steps[i % len(steps)] (one graph each in graph
    mode)."""

    def __init__(self, torch, stream, steps, launches_per_step, use_graph):
        self.torch, self.stream = torch, stream
        self.steps = steps if isinstance(steps, list) else [steps]
        self.lps = launches_per_step
        self.graphs = None
        with torch.cuda.stream(stream):
            for _ in range(3):
                for st in self.steps:
                    st()
        torch.cuda.synchronize()
        if use_graph:
            self.graphs = []
            for st in self.steps:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    st()
                self.graphs.append(g)
            torch.cuda.synchronize()

    def _run(self, n):
        k = len(self.steps)
        with self.torch.cuda.stream(self.stream):
            for i in range(n):
                if self.graphs is not None:
                    self.graphs[i % k].replay()
                else:
                    self.steps[i % k]()

    def measure(self, steps, warmup):
        torch = self.torch
        self._run(warmup)
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(self.stream)
        self._run(steps)
        ev1.record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_per_step = wall * 1e3 / steps
        launch_us = ev0.elapsed_time(ev1) * 1e3 / (steps * self.lps)
        return ms_per_step, launch_us


def warm_cold(torch, stream, steps, lps, graph, args):
    """Cold figure (rotating over all step functions) and warm figure (the first one
    repeated)."""
    cold = Timed(torch, stream, steps, lps, graph).measure(args.steps, args.warmup)
    warm = Timed(torch, stream, steps[:1], lps, graph).measure(args.steps, args.warmup)
    return cold, warm


def cpu_time(fn, seconds):
    """Repeat fn() (one sample unit) for about `seconds` on one thread."""
    from threadpoolctl import threadpool_limits
    n = 0
    t0 = time.perf_counter()
    with threadpool_limits(1):
        while True:
            fn()
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return n, el


# ----------------------------------------------------------------- host CPU baseline
# Work shared with forked worker processes (set before the pool is created).
_CPU_WORK = {}
_PREFILL_ROWS = 64   # query rows per oracle work unit of the prefill baseline


def _worker_init():
    from threadpoolctl import threadpool_limits
    global _TPL
    _TPL = threadpool_limits(1)   # one BLAS thread per worker process


def _oracle_unit(unit):
    """One work unit of the oracle: a whole decode layer, or a block of prefill rows."""
    import oracle
    kind, a = unit
    if kind == "decode":
        inp = _CPU_WORK["decode"][a]
        oracle.prefix_query(inp.Q, inp.K, inp.V)
    else:
        inp = _CPU_WORK["prefill"]
        h, i0 = a
        M = inp.Q.shape[1]
        oracle.prefix_query_fused(inp.Q, inp.K, inp.V, inp.K_suf, inp.V_suf,
                                  rows=[(h, i) for i in range(i0, min(i0 + _PREFILL_ROWS, M))])
    return 0


def host_cores():
    """Host cores the oracle may use: this process's CPU affinity, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _median_time(fn, runs=3):
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return sorted(ts)[len(ts) // 2]


def cpu_baselines(decode_inputs=None, prefill_input=None):
    """Time the oracle on the host: all usable cores (worker processes forked before any
    GPU use, one BLAS thread each) over a fixed sample, and one thread on a smaller one;
    median of 3 runs each. Returns {"decode": ..., "prefill": ...} cpu_baseline objects."""
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits
    _CPU_WORK["decode"] = decode_inputs
    _CPU_WORK["prefill"] = prefill_input
    W = host_cores()
    res = {}
    with mp.get_context("fork").Pool(W, initializer=_worker_init) as pool:
        pool.map(_oracle_unit, [("decode", 0)] * W if decode_inputs else
                 [("prefill", (0, 0))] * W)   # warm the workers (imports)

        def measure(units_all, units_one):
            t_all = _median_time(lambda: pool.map(_oracle_unit, units_all, chunksize=1))
            with threadpool_limits(1):
                _oracle_unit(units_one[0])
                t_one = _median_time(lambda: [_oracle_unit(u) for u in units_one])
            return t_all, t_one

        if decode_inputs:
            L = len(decode_inputs)
            inp = decode_inputs[0]
            per_layer = inp.K.shape[0] * inp.K.shape[1] * inp.K.shape[2] * 2 * 2
            all_u = [("decode", l) for _ in range(6 * W) for l in range(L)]
            one_u = [("decode", l) for _ in range(6) for l in range(L)]
            t_all, t_one = measure(all_u, one_u)
            res["decode"] = {
                "value": round(len(all_u) * per_layer / t_all / 1e9, 4), "unit": "GB/s",
                "cores": W, "kind": "oracle",
                "sample": f"{6 * W} whole {L}-layer passes of this workload over {W} worker processes "
                          f"(fp64 numpy, one BLAS thread each), median of 3 runs "
                          f"({t_all:.2f} s)",
                "single_thread": {"value": round(len(one_u) * per_layer / t_one / 1e9, 4),
                                  "sample": f"6 whole passes, 1 thread, median of 3 ({t_one:.2f} s)"},
                "host_cpus": os.cpu_count()}
        if prefill_input is not None:
            H_q, M, D = prefill_input.Q.shape
            N = prefill_input.K.shape[1]
            S = 0 if prefill_input.K_suf is None else prefill_input.K_suf.shape[1]

            def flops(unit):
                h, i0 = unit[1]
                return sum(4 * D * (N + (S - M + i + 1 if S else 0))
                           for i in range(i0, min(i0 + _PREFILL_ROWS, M)))
            step_u = [("prefill", (h, i0)) for h in range(H_q) for i0 in range(0, M, _PREFILL_ROWS)]
            reps = max(1, W // 2)
            all_u = step_u * reps
            one_u = step_u[::2]
            t_all, t_one = measure(all_u, one_u)
            res["prefill"] = {
                "value": round(sum(map(flops, all_u)) / t_all / 1e12, 6), "unit": "TFLOP/s",
                "cores": W, "kind": "oracle",
                "sample": f"every row of {reps} steps ({H_q * M} rows each, in blocks of {_PREFILL_ROWS}) "
                          f"over {W} worker processes (fp64 numpy, one BLAS thread each), "
                          f"median of 3 runs ({t_all:.2f} s)",
                "single_thread": {"value": round(sum(map(flops, one_u)) / t_one / 1e12, 6),
                                  "sample": f"{len(one_u) * _PREFILL_ROWS} rows (every 2nd block), "
                                            f"1 thread, median of 3 ({t_one:.2f} s)"},
                "host_cpus": os.cpu_count()}
    _CPU_WORK.clear()
    return res


def oracle_leg(args):
    """True when this run includes the oracle leg: the oracle timed on the host cores
    (cpu_baseline) and, on the same inputs, the GPU's results checked against it. That leg
    is the only part of bench.py that calls the oracle; --no-cpu-baseline skips it."""
    return not args.no_cpu_baseline


def check_close(got, ref, tol, what):
    import numpy as np
    err = float(np.max(np.abs(np.asarray(got, np.float64) - ref)))
    if not err <= tol:
        raise SystemExit(f"bench {what} disagrees with the oracle: max-abs {err}")


# ----------------------------------------------------------------------------- configs
def run_decode(args, torch, kp, synth, dev, stream, inputs=None, cpu=None):
    import numpy as np
    case = synth.DECODE
    if inputs is None:
        inputs = [synth.generate(case, l) for l in range(case.layers)]
    sid = "bench-decode"
    NSET = 2   # layers [32 k, 32 k + 32) hold set k (the same data)
    for k in range(NSET):
        for l, inp in enumerate(inputs):
            kp.pion_prefix_store(sid, case.layers * k + l, torch.from_numpy(inp.K).to(dev),
                                 torch.from_numpy(inp.V).to(dev))
    Qall = torch.from_numpy(np.stack([i.Q for i in inputs])).to(dev)
    out = torch.empty((case.layers, case.H_q, 1, case.D), dtype=torch.float32, device=dev)
    lse = torch.empty((case.layers, case.H_q, 1), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    lib, sidb = kp.lib(), sid.encode()
    if args.mode == "layers":
        fn = lib.pion_prefix_query_layers
        calls = [[(sidb, case.layers * k, case.layers, case.H_q, case.D, 1, Qall.data_ptr(), None,
                   out.data_ptr(), lse.data_ptr())] for k in range(NSET)]
    else:
        fn = lib.pion_prefix_query
        calls = [[(sidb, case.layers * k + l, case.H_q, case.D, 1, Qall[l].data_ptr(), None,
                   out[l].data_ptr(), lse[l].data_ptr()) for l in range(case.layers)]
                 for k in range(NSET)]

    nstreams = max(1, args.streams) if args.mode == "calls" else 1
    side = [torch.cuda.Stream(device=dev) for _ in range(nstreams)] if nstreams > 1 else []

    def make_step(cs):
        def step():
            cur = torch.cuda.current_stream()
            if not side:
                for c in cs:
                    rc = fn(*c, cur.cuda_stream)
                    if rc != 0:
                        raise kp.PionError(rc, fn.__name__)
                return
            for sd in side:           # fork: every side stream starts after the step's start
                sd.wait_stream(cur)
            for i, c in enumerate(cs):
                rc = fn(*c, side[i % len(side)].cuda_stream)
                if rc != 0:
                    raise kp.PionError(rc, fn.__name__)
            for sd in side:           # join
                cur.wait_stream(sd)
        return step

    graph = args.mode == "calls" and not args.eager
    lps = len(calls[0])
    steps = [make_step(c) for c in calls]
    with torch.cuda.stream(stream):
        steps[0]()
    plan = kp.pion_prefix_last_plan()   # the kernel(s) of one launch of the step
    (ms, launch_us), (wms, wlaunch_us) = warm_cold(torch, stream, steps, lps, graph, args)
    if oracle_leg(args):   # the first and last layers against the oracle
        import oracle
        for l in (0, case.layers - 1):
            ref, ref_lse = oracle.prefix_query(inputs[l].Q, inputs[l].K, inputs[l].V)
            check_close(out[l].cpu().numpy(), ref, 2e-3, "out")
            check_close(lse[l].cpu().numpy(), ref_lse, 1e-4, "lse")
    bytes_layer = case.H_kv * case.N * case.D * 2 * 2
    bytes_step = bytes_layer * case.layers
    bytes_launch = bytes_step // lps
    kp.pion_prefix_drop(sid, -1)
    return {
        "value": bytes_step / (ms * 1e-3) / 1e9, "unit": "GB/s", "ms_per_step": ms,
        "dtype": "fp16 K/V, fp32 accumulate",
        "config": {"workload": "M=1 prefix attention, decode shape H_q=H_kv=8 N=2048 D=128, "
                               "32 resident layers queried per step",
                   "entry": fn.__name__, "launches_per_step": lps,
                   "launch": ("hip-graph replay" if graph else "eager") +
                             (f", calls round-robin over {nstreams} streams" if nstreams > 1 else ""),
                   "bytes_per_step": bytes_step,
                   "memory_side_cache": f"cold: steps alternate over {NSET} copies of the 32 "
                                        f"layers ({NSET * bytes_step / 1e6:.0f} MB)"},
        "roofline": {"bound": "hbm", "achieved": bytes_launch / (launch_us * 1e-6) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "traffic": (measured_traffic(DECODE_TRAFFIC)
                                 if args.mode == "layers" else None),
                     "kernel": plan,
                     "bytes_per_launch": bytes_launch, "avg_launch_us": launch_us},
        "warm": {"value": round(bytes_step / (wms * 1e-3) / 1e9, 3), "unit": "GB/s",
                 "avg_launch_us": round(wlaunch_us, 3),
                 "note": "the same 32 layers every step (memory-side cache warm)"},
        "cpu_baseline": cpu,
    }


def run_prefill(args, torch, kp, synth, dev, stream, inp=None, cpu=None, calls=None):
    """The fused batched-Q prefill: `calls` timed back-to-back calls (default: --steps)
    between one pair of HIP events on the launch stream, whose mean is the roofline's
    launch time; a second pass with an event after every call gives the median."""
    case = synth.PREFILL
    if inp is None:
        inp = synth.generate(case)
    sid = "bench-prefill"
    kp.pion_prefix_store(sid, 0, torch.from_numpy(inp.K).to(dev),
                         torch.from_numpy(inp.V).to(dev))
    Q, Ks, Vs = (torch.from_numpy(a).to(dev) for a in (inp.Q, inp.K_suf, inp.V_suf))
    out = torch.empty((case.H_q, case.M, case.D), dtype=torch.float32, device=dev)
    lse = torch.empty((case.H_q, case.M), dtype=torch.float32, device=dev)
    lib, sidb = kp.lib(), sid.encode()
    a = (sidb, 0, case.H_q, case.D, case.M, case.S_suf, case.H_kv, Q.data_ptr(),
         Ks.data_ptr(), Vs.data_ptr(), None, out.data_ptr(), lse.data_ptr())

    def step():
        rc = lib.pion_prefix_query_fused(*a, torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise kp.PionError(rc, "pion_prefix_query_fused")

    with torch.cuda.stream(stream):
        for _ in range(3):
            step()
    plan = kp.pion_prefix_last_plan()
    n = calls or args.steps
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()
    # the timed region: n calls back to back between one pair of HIP events (an event
    # between calls inserts a marker packet that costs a few us per call on this stack)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        ev0.record(stream)
        for i in range(n):
            step()
        ev1.record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / n
    launch_us = ev0.elapsed_time(ev1) * 1e3 / n
    # the per-call spread: a second pass with an event after every call (its median
    # includes that marker cost)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    with torch.cuda.stream(stream):
        evs[0].record(stream)
        for i in range(n):
            step()
            evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_call = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(n))
    median_us = per_call[n // 2]
    err = None
    if oracle_leg(args):   # every row against the oracle (the timed calls all wrote it)
        import oracle
        ref, ref_lse = oracle.prefix_query_fused(inp.Q, inp.K, inp.V, inp.K_suf, inp.V_suf)
        o, l = out.cpu().numpy(), lse.cpu().numpy()
        check_close(o, ref, 2e-3, "out")
        check_close(l, ref_lse, 1e-4, "lse")
        err = {"out": float(abs(o - ref).max()), "lse": float(abs(l - ref_lse).max())}
    flops = 4 * case.H_q * case.D * (case.M * case.N + case.M * (case.M + 1) // 2)
    kp.pion_prefix_drop(sid, -1)
    return {
        "value": flops / (ms * 1e-3) / 1e12, "unit": "TFLOP/s", "ms_per_step": ms,
        "dtype": "fp16 in, fp32 accumulate",
        "config": {"workload": "fused batched-Q prefill H_q=24 H_kv=8 (h//3) D=128 N=4096 "
                               "M=S_suf=512 causal suffix", "entry": "pion_prefix_query_fused",
                   "calls_timed": n, "flops_per_call": flops},
        "roofline": {"bound": "mfma", "achieved": flops / (launch_us * 1e-6) / 1e12,
                     "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "traffic": measured_traffic(PREFILL_TRAFFIC),
                     "kernel": plan, "flops_per_launch": flops,
                     "avg_launch_us": launch_us, "median_launch_us": round(median_us, 3),
                     "median_TFLOP/s": round(flops / (median_us * 1e-6) / 1e12, 2),
                     "median_note": "median of a second pass with a HIP event after every call",
                     "max_abs_err": err},
        "cpu_baseline": cpu,
    }


def stream_ceiling(torch, kp, dev, stream, nbytes=1 << 30, reps=20, nbufs=1):
    """A plain streaming read of `nbytes` (past the 256 MB memory-side cache: one buffer
    of at least that size, or `nbufs` buffers read in rotation), `reps` times back to
    back: the achievable HBM read rate for a pass of that size, timed with HIP events."""
    bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(nbufs)]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i in range(3):
            kp.pion_bench_stream_read(bufs[i % nbufs], sink)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for i in range(reps):
            kp.pion_bench_stream_read(bufs[i % nbufs], sink)
        ev1.record(stream)
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / reps
    del bufs
    return {"value": round(nbytes / (us * 1e-6) / 1e9, 1), "unit": "GB/s",
            "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "avg_launch_us": round(us, 2), "kernel": "stream_read_kernel",
            "note": f"plain streaming read of {nbytes >> 20} MiB with 16-byte non-temporal "
                    f"loads, one contiguous chunk per workgroup, {reps} launches back to back"
                    + (f" over {nbufs} buffers in rotation" if nbufs > 1 else "")
                    + " (cold: past the memory-side cache)"}


def mfma_ceiling(torch, kp, dev, stream, iters=2048, reps=20):
    """fp16 MFMA products alone on every SIMD (four waves per SIMD, no memory traffic),
    `reps` launches of about 0.5 ms back to back, as long as a batched-Q run: the dense
    fp16 rate the chip sustains under full matrix load, timed with HIP events."""
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(3):
            flops = kp.pion_bench_mfma_peak(iters, sink)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(reps):
            kp.pion_bench_mfma_peak(iters, sink)
        ev1.record(stream)
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / reps
    tflops = flops / (us * 1e-6) / 1e12
    return {"value": round(tflops, 1), "unit": "TFLOP/s",
            "frac_of_peak": round(tflops / FP16_MFMA_PEAK_TFLOPS, 4),
            "avg_launch_us": round(us, 2), "kernel": "mfma_peak_kernel",
            "note": f"v_mfma_f32_32x32x16_f16 alone, {iters} rounds of 4 independent products "
                    f"per wave, 4 waves per SIMD, {reps} launches back to back"}


def run_mlx4(args, torch, kp, synth, dev, stream):
    case = synth.MLX4_DECODE
    LAYERS, NSET = 16, 2   # 16 layers per step (671 MB); two sets alternate (1.34 GB)
    inp = synth.generate(case)
    sid = "bench-mlx4"
    K16, V16 = torch.from_numpy(inp.K).to(dev), torch.from_numpy(inp.V).to(dev)
    for k in range(NSET * LAYERS):   # the same quantized prefix in every layer slot
        kp.pion_prefix_store(sid, k, K16, V16, kp.PION_KV_MLX4G32)
    Q1 = torch.from_numpy(inp.Q).to(dev)
    Q = Q1.unsqueeze(0).expand(LAYERS, -1, -1, -1).contiguous()
    out = torch.empty((LAYERS, case.H_q, 1, case.D), dtype=torch.float32, device=dev)
    lse = torch.empty((LAYERS, case.H_q, 1), dtype=torch.float32, device=dev)
    lib, sidb = kp.lib(), sid.encode()

    def make_step(k):
        a = (sidb, LAYERS * k, LAYERS, case.H_q, case.D, 1, Q.data_ptr(), None, out.data_ptr(),
             lse.data_ptr())

        def step():
            rc = lib.pion_prefix_query_layers(*a, torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise kp.PionError(rc, "pion_prefix_query_layers")
        return step

    (ms, launch_us), (wms, wlaunch_us) = warm_cold(
        torch, stream, [make_step(k) for k in range(NSET)], 1, False, args)
    plan = kp.pion_prefix_last_plan()   # the kernel of the 16-layer launch

    # single M=1 query per launch, rotating over the 32 slots (cold) - latency figure
    def make_one(k):
        a = (sidb, k, case.H_q, case.D, 1, Q1.data_ptr(), None, out[0].data_ptr(),
             lse[0].data_ptr())

        def step():
            rc = lib.pion_prefix_query(*a, torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise kp.PionError(rc, "pion_prefix_query")
        return step
    one_ms, one_us = Timed(torch, stream, [make_one(k) for k in range(NSET * LAYERS)], 1,
                           False).measure(args.steps, args.warmup)

    # the store-side encoder over this shape's K and V: one call over both, stacked as
    # 2 H N rows (the encoder works row by row), one launch per step
    rows = case.H_kv * case.N
    codes = torch.empty((2 * rows, case.D // 8), dtype=torch.int32, device=dev)
    scales = torch.empty((2 * rows, case.D // 32), dtype=torch.float16, device=dev)
    biases = torch.empty((2 * rows, case.D // 32), dtype=torch.float16, device=dev)
    xkv = torch.cat([K16.reshape(rows, case.D), V16.reshape(rows, case.D)])

    def quant():
        rc = lib.pion_kv_quantize_mlx4g32(xkv.data_ptr(), 2 * rows, case.D, codes.data_ptr(),
                                          scales.data_ptr(), biases.data_ptr(),
                                          torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise kp.PionError(rc, "pion_kv_quantize_mlx4g32")
    q_ms, _ = Timed(torch, stream, quant, 2, False).measure(args.steps // 4 + 1, args.warmup)
    q_read, q_written = 2 * rows * case.D * 2, 2 * rows * (case.D // 2 + case.D // 32 * 4)
    del codes, scales, biases

    # the same shape resident in fp16 (16 layers per launch, two sets alternating)
    sid16 = "bench-mlx4-fp16"
    for k in range(NSET * LAYERS):
        kp.pion_prefix_store(sid16, k, K16, V16)
    del K16, V16, xkv
    sid16b = sid16.encode()
    out16, lse16 = torch.empty_like(out), torch.empty_like(lse)   # out keeps the mlx4g32 result

    def make_step16(k):
        a = (sid16b, LAYERS * k, LAYERS, case.H_q, case.D, 1, Q.data_ptr(), None,
             out16.data_ptr(), lse16.data_ptr())

        def step():
            rc = lib.pion_prefix_query_layers(*a, torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise kp.PionError(rc, "pion_prefix_query_layers")
        return step
    (ms16, _), _ = warm_cold(torch, stream, [make_step16(k) for k in range(NSET)], 1, False,
                             args)
    if oracle_leg(args):
        import oracle
        ref16, _ = oracle.prefix_query(inp.Q, inp.K, inp.V)
        check_close(out16[LAYERS - 1].cpu().numpy(), ref16, 2e-3, "out")
    kp.pion_prefix_drop(sid16, -1)
    del out16, lse16
    nbytes16 = LAYERS * case.H_kv * case.N * case.D * 4

    nbytes_layer = case.H_kv * case.N * 160
    nbytes = nbytes_layer * LAYERS
    cpu = None
    if oracle_leg(args):   # the first and last layers against the oracle, then its timing
        import oracle
        Kh = oracle.dequantize(*oracle.quantize(inp.K.reshape(-1, 128))).reshape(inp.K.shape)
        Vh = oracle.dequantize(*oracle.quantize(inp.V.reshape(-1, 128))).reshape(inp.V.shape)
        ref, ref_lse = oracle.prefix_query(inp.Q, Kh, Vh)
        o = out.cpu().numpy()
        for l in (0, LAYERS - 1):
            check_close(o[l], ref, 2e-3, "out")
        check_close(lse[LAYERS - 1].cpu().numpy(), ref_lse, 1e-4, "lse")

        def one_layer():
            oracle.prefix_query(inp.Q, Kh, Vh)
        n, el = cpu_time(one_layer, args.cpu_seconds)
        cpu = {"value": round(nbytes_layer * n / el / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"{n} single-layer M=1 queries of this workload on the dequantized "
                         f"K/V ({el:.1f} s, fp64 numpy, 1 thread)"}
    kp.pion_prefix_drop(sid, -1)
    return {
        "value": nbytes / (ms * 1e-3) / 1e9, "unit": "GB/s", "ms_per_step": ms,
        "dtype": "int4 codes + fp16 scale/bias, fp32 accumulate",
        "config": {"workload": "mlx4g32 decode H_q=24 H_kv=8 (h//3) D=128 N=32768 M=1, "
                               f"{LAYERS} resident layers queried per step",
                   "entry": "pion_prefix_query_layers", "launches_per_step": 1,
                   "bytes_per_step": nbytes,
                   "memory_side_cache": f"cold: steps alternate over {NSET} sets of {LAYERS} "
                                        f"slots ({NSET * nbytes / 1e6:.0f} MB)"},
        "roofline": {"bound": "hbm", "achieved": nbytes / (launch_us * 1e-6) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "traffic": measured_traffic(MLX4_TRAFFIC),
                     "kernel": plan,
                     "bytes_per_launch": nbytes, "avg_launch_us": launch_us},
        "warm": {"value": round(nbytes / (wms * 1e-3) / 1e9, 3), "unit": "GB/s",
                 "avg_launch_us": round(wlaunch_us, 3),
                 "note": "one set every step (memory-side cache warm)"},
        "quantize": {"GB/s": round((q_read + q_written) / (q_ms * 1e-3) / 1e9, 1),
                     "us_per_step": round(q_ms * 1e3, 3),
                     "note": f"pion_kv_quantize_mlx4g32 of this shape's K and V ({q_read} B read, "
                             f"{q_written} B written per step; one call over both, stacked as 2 H N rows: one launch)"},
        "fp16_resident": {"GB/s": round(nbytes16 / (ms16 * 1e-3) / 1e9, 1),
                          "us_per_layer": round(ms16 * 1e3 / LAYERS, 3),
                          "mlx4g32_us_per_layer": round(ms * 1e3 / LAYERS, 3),
                          "note": "the same shape and launch with fp16 K/V "
                                  f"({nbytes16} B per {LAYERS}-layer launch, cold)"},
        "single_query": {"us_per_query": round(one_ms * 1e3, 3),
                         "GB/s": round(nbytes_layer / (one_ms * 1e-3) / 1e9, 3),
                         "note": "one M=1 pion_prefix_query per launch over one 41.9 MB "
                                 "prefix, rotating over 32 slots (cold)"},
        "cpu_baseline": cpu,
    }


def run_sparse(args, torch, kp, synth, dev, stream):
    case = synth.SPARSE
    inp = synth.generate(case)
    sid = "bench-sparse"
    NSLOT = 4   # the same prefix in 4 slots (268 MB)
    K16, V16 = torch.from_numpy(inp.K).to(dev), torch.from_numpy(inp.V).to(dev)
    for k in range(NSLOT):
        kp.pion_prefix_store(sid, k, K16, V16)
    del K16, V16
    Q, Ks, Vs = (torch.from_numpy(a).to(dev) for a in (inp.Q, inp.K_suf, inp.V_suf))
    out = torch.empty((case.H_q, case.D), dtype=torch.float32, device=dev)
    blocks = torch.empty((case.H_kv, case.K_top), dtype=torch.int32, device=dev)
    lib, sidb = kp.lib(), sid.encode()

    def make_step(k):
        a = (sidb, k, case.H_q, case.D, case.B, case.K_top, case.H_kv, case.S_suf, Q.data_ptr(),
             Ks.data_ptr(), Vs.data_ptr(), None, out.data_ptr(), None, blocks.data_ptr())

        def step():
            rc = lib.pion_prefix_query_sparse_auto(*a, torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise kp.PionError(rc, "pion_prefix_query_sparse_auto")
        return step

    # 2 launches per query: block selection, then the split kernel (block means cached
    # per slot by the first query, inside the untimed warm-up)
    (ms, _), (wms, _) = warm_cold(torch, stream, [make_step(k) for k in range(NSLOT)], 2,
                                  False, args)
    if oracle_leg(args):
        import oracle
        ref, _, ref_blocks = oracle.prefix_query_sparse_auto(
            inp.Q, inp.K, inp.V, case.B, case.K_top, None, inp.K_suf, inp.V_suf)
        check_close(out.cpu().numpy(), ref, 2e-3, "out")
        if not (blocks.cpu().numpy() == ref_blocks).all():
            raise SystemExit("bench sparse blocks disagree with the oracle")
    if args.kmean_builds > 0:   # a STORE replaces the slot, so its next query rebuilds K_mean
        K16 = torch.from_numpy(inp.K).to(dev)
        V16 = torch.from_numpy(inp.V).to(dev)
        for i in range(args.kmean_builds):
            kp.pion_prefix_store(sid, i % NSLOT, K16, V16)
            make_step(i % NSLOT)()
        torch.cuda.synchronize()
        del K16, V16
    # a plain read of the bytes one K_mean build reads (the keys of the slot), as the
    # ceiling for a pass of that size
    kmean_ceiling = stream_ceiling(torch, kp, dev, stream, case.H_kv * case.N * case.D * 2,
                                   reps=50, nbufs=10)
    nb = case.N // case.B
    nbytes = (case.H_kv * nb * case.D * 4 + case.K_top * case.B * case.D * 4
              + case.S_suf * case.D * 4 + case.H_q * case.D * 6)
    kp.pion_prefix_drop(sid, -1)
    return {
        "value": ms * 1e3, "unit": "us/query", "ms_per_step": ms,
        "dtype": "fp16 K/V, fp32 accumulate",
        "config": {"workload": "sparse-auto fused H_q=8 H_kv=1 D=256 N=65536 B=64 K_top=8 "
                               "S_suf=64 M=1 (block means cached)", "bytes_per_step": nbytes,
                   "memory_side_cache": f"cold: steps rotate over {NSLOT} slots"},
        "roofline": {"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "traffic": None},
        "warm": {"value": round(wms * 1e3, 3), "unit": "us/query",
                 "note": "one slot every step (memory-side cache warm)"},
        "kmean_read_ceiling": kmean_ceiling,
        "cpu_baseline": None,
    }


def run_tiny(args, torch, kp, synth, dev, stream):
    case = synth.TINY
    inp = synth.generate(case)
    kp.pion_prefix_store("bench-tiny", 0, torch.from_numpy(inp.K).to(dev),
                         torch.from_numpy(inp.V).to(dev))
    Q = torch.from_numpy(inp.Q).to(dev)
    out = torch.empty((2, 1, 64), dtype=torch.float32, device=dev)
    lib = kp.lib()
    a = (b"bench-tiny", 0, 2, 64, 1, Q.data_ptr(), None, out.data_ptr(), None)

    def step():
        rc = lib.pion_prefix_query(*a, torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise kp.PionError(rc, "pion_prefix_query")

    t = Timed(torch, stream, step, 1, False)
    ms, _ = t.measure(args.steps, args.warmup)
    if oracle_leg(args):
        import oracle
        check_close(out.cpu().numpy(), oracle.prefix_query(inp.Q, inp.K, inp.V)[0], 2e-3, "out")
    kp.pion_prefix_drop("bench-tiny", -1)
    return {"value": ms * 1e3, "unit": "us/query", "ms_per_step": ms, "dtype": "fp16",
            "config": {"workload": "tiny dense query H=2 N=128 D=64 M=1"},
            "roofline": None, "cpu_baseline": None}


def run_query_sparse(args, torch, kp, synth, dev, stream):
    """QUERY_SPARSE (caller-supplied indices): H = 8 heads, N = 65536 fp16 tokens, D = 128,
    K_sparse_max = 2048 uniform random token indices per head (all counted), M = 1.
    Not one of the five headline workloads; it measures the QUERY_SPARSE row. Bytes are
    the gathered K and V rows: H * K_sparse_max * 2 * D * 2."""
    import numpy as np
    H, N, D, KS = 8, 65536, 128, 2048
    NSLOT = 4   # 4 slots of 268 MB each (1.07 GB)
    inp = synth.generate(synth.DECODE, 21, N=N, H_q=H, H_kv=H, D=D)
    rng = np.random.default_rng(21)
    idx = rng.integers(0, N, size=(H, KS)).astype(np.int32)
    counts = np.full(H, KS, np.int32)
    K16, V16 = torch.from_numpy(inp.K).to(dev), torch.from_numpy(inp.V).to(dev)
    sid = "bench-qsparse"
    for k in range(NSLOT):
        kp.pion_prefix_store(sid, k, K16, V16)
    del K16, V16
    Q = torch.from_numpy(inp.Q).to(dev)
    ti, tc = torch.from_numpy(idx).to(dev), torch.from_numpy(counts).to(dev)
    out = torch.empty((H, D), dtype=torch.float32, device=dev)
    lse = torch.empty((H,), dtype=torch.float32, device=dev)
    lib, sidb = kp.lib(), sid.encode()

    def make_step(k):
        a = (sidb, k, H, D, KS, Q.data_ptr(), ti.data_ptr(), tc.data_ptr(), out.data_ptr(),
             lse.data_ptr())

        def step():
            rc = lib.pion_prefix_query_sparse(*a, torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise kp.PionError(rc, "pion_prefix_query_sparse")
        return step

    (ms, launch_us), (wms, _) = warm_cold(torch, stream, [make_step(k) for k in range(NSLOT)],
                                          1, False, args)
    nbytes = H * KS * 2 * D * 2
    cpu = None
    if oracle_leg(args):   # the result against the oracle, then its timing
        import oracle
        ref, _ = oracle.prefix_query_sparse(inp.Q, inp.K, inp.V, idx, counts)
        check_close(out.cpu().numpy(), ref, 2e-3, "out")

        def one_query():
            oracle.prefix_query_sparse(inp.Q, inp.K, inp.V, idx, counts)
        n, el = cpu_time(one_query, args.cpu_seconds)
        cpu = {"value": round(el / n * 1e6, 1), "unit": "us/query", "cores": 1, "kind": "oracle",
               "sample": f"{n} whole queries of this workload ({el:.1f} s)"}
    kp.pion_prefix_drop(sid, -1)
    return {
        "value": ms * 1e3, "unit": "us/query", "ms_per_step": ms, "dtype": "fp16 K/V, fp32 accumulate",
        "config": {"workload": f"QUERY_SPARSE H={H} N={N} D={D} K_sparse_max={KS} uniform random "
                               "indices M=1", "bytes_per_step": nbytes,
                   "memory_side_cache": f"cold: steps rotate over {NSLOT} slots"},
        "roofline": {"bound": "hbm", "achieved": nbytes / (launch_us * 1e-6) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "traffic": None,
                     "avg_launch_us": launch_us},
        "warm": {"value": round(wms * 1e3, 3), "unit": "us/query",
                 "note": "one slot every step (memory-side cache warm)"},
        "cpu_baseline": cpu,
    }


def run_sweep(args, torch, kp, synth, dev, stream):
    """The decode step (H_q = H_kv = 8, N = 2048, 32 layers per launch, cold over two sets)
    at every supported head dim with fp16 slots, and with fp32-resident slots at D = 64,
    128 and 256. One seeded layer per case is stored in all 64 slots."""
    import numpy as np
    LAYERS, NSET, H, N = 32, 2, 8, 2048
    cases = [(D, kp.PION_KV_FP16) for D in (32, 64, 96, 128, 160, 192, 256, 512)]
    cases += [(D, kp.PION_KV_FP32) for D in (64, 128, 256)]
    lib = kp.lib()
    rows, head = [], None
    for D, fmt in cases:
        f32 = fmt == kp.PION_KV_FP32
        inp = synth.generate(synth.DECODE, 0, D=D, dtype="float32" if f32 else "float16")
        sid = f"bench-sweep-{D}-{fmt}"
        K, V = torch.from_numpy(inp.K).to(dev), torch.from_numpy(inp.V).to(dev)
        for k in range(NSET * LAYERS):
            kp.pion_prefix_store(sid, k, K, V, fmt)
        del K, V
        Q = torch.from_numpy(np.stack([inp.Q] * LAYERS)).to(dev)
        out = torch.empty((LAYERS, H, 1, D), dtype=torch.float32, device=dev)
        lse = torch.empty((LAYERS, H, 1), dtype=torch.float32, device=dev)
        sidb = sid.encode()

        def make_step(k):
            a = (sidb, LAYERS * k, LAYERS, H, D, 1, Q.data_ptr(), None, out.data_ptr(),
                 lse.data_ptr())

            def step():
                rc = lib.pion_prefix_query_layers(*a, torch.cuda.current_stream().cuda_stream)
                if rc != 0:
                    raise kp.PionError(rc, "pion_prefix_query_layers")
            return step
        ms, launch_us = Timed(torch, stream, [make_step(k) for k in range(NSET)], 1,
                              False).measure(args.steps, args.warmup)
        if oracle_leg(args):
            import oracle
            ref, ref_lse = oracle.prefix_query(inp.Q, inp.K, inp.V)
            check_close(out[LAYERS - 1].cpu().numpy(), ref, 1e-4 if f32 else 2e-3, "out")
            check_close(lse[LAYERS - 1].cpu().numpy(), ref_lse, 2e-5 if f32 else 1e-4, "lse")
        kp.pion_prefix_drop(sid, -1)
        nbytes = LAYERS * H * N * D * 2 * (4 if f32 else 2)
        row = {"D": D, "resident": "fp32" if f32 else "fp16", "bytes_per_launch": nbytes,
               "avg_launch_us": round(launch_us, 3),
               "GB/s": round(nbytes / (launch_us * 1e-6) / 1e9, 1),
               "frac": round(nbytes / (launch_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        rows.append(row)
        if D == 128 and not f32:
            head = (ms, launch_us, nbytes)
    ms, launch_us, nbytes = head
    return {
        "value": nbytes / (ms * 1e-3) / 1e9, "unit": "GB/s", "ms_per_step": ms,
        "dtype": "fp16 or fp32 K/V, fp32 accumulate",
        "config": {"workload": "M=1 decode H_q=H_kv=8 N=2048, 32 layers per launch, at every "
                               "supported head dim (fp16) and D=64/128/256 fp32-resident; value: "
                               "the D=128 fp16 case",
                   "entry": "pion_prefix_query_layers", "launches_per_step": 1,
                   "memory_side_cache": f"cold: steps alternate over {NSET} sets of {LAYERS} slots"},
        "roofline": {"bound": "hbm", "achieved": nbytes / (launch_us * 1e-6) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "traffic": None,
                     "bytes_per_launch": nbytes, "avg_launch_us": launch_us},
        "sweep": rows,
        "cpu_baseline": None,
    }


def run_vstore(args, torch, kp, synth, dev, stream):
    """V-store side of the decode shape: 32 layers, K and V, H = 8, N = 2048, D = 128
    (kv = 1024, the 640 B/token mlx4g32 record). A step fetches every layer-side's whole
    token range as fp32 (64 launches of the dequantizing fetch). Bytes per launch: records
    read (640 B/token) + fp32 written (4 kv B/token). Steps rotate over 4 copies of the
    records (336 MB) so the reads are cold. Beside it, `warm_call`: the whole-call time of
    pion_prefix_warm (K and V of one layer into an fp16 slot, replacing the live slot:
    allocation, two relayout launches, the free of the old slot), host work included."""
    import numpy as np
    L, H, N, D = 32, 8, 2048, 128
    kv = H * D
    NCOPY = 4
    recs = [synth.mlx4_records(N, kv, [7, l, side]) for l in range(L) for side in range(2)]
    rb = recs[0].shape[1]
    dev_recs = [[torch.from_numpy(r).to(dev) for r in recs] for _ in range(NCOPY)]
    out = [torch.empty((N, kv), dtype=torch.float32, device=dev) for _ in range(2)]
    lib = kp.lib()

    def make_step(c):
        calls = [(dev_recs[c][i].data_ptr(), out[i % 2].data_ptr()) for i in range(2 * L)]

        def step():
            s = torch.cuda.current_stream().cuda_stream
            for rp, op in calls:
                rc = lib.pion_vstore_fetch_f32(rp, 1, N, kv, 0, N, op, s)
                if rc != 0:
                    raise kp.PionError(rc, "pion_vstore_fetch_f32")
        return step

    (ms, launch_us), (wms, _) = warm_cold(torch, stream, [make_step(c) for c in range(NCOPY)],
                                          2 * L, False, args)
    if oracle_leg(args):
        from oracle import vstore as ovs
        got = out[1].cpu().numpy()                  # the last launch: layer 31, V
        want = ovs.fetch_f32(recs[-1], ovs.MLX4G32, kv, 0, N)
        if not np.array_equal(got.view(np.uint32), want.view(np.uint32)):
            raise SystemExit("bench fetch disagrees with the oracle")
    per_launch = N * (rb + 4 * kv)
    nbytes = 2 * L * per_launch

    # whole WARM calls (replacing live slots), one layer per call
    sid = "bench-warm"
    for l in range(L):
        kp.pion_prefix_warm(sid, l, H, D, dev_recs[0][2 * l], dev_recs[0][2 * l + 1], 1)
    torch.cuda.synchronize()
    reps = 3
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for _ in range(reps):
            for l in range(L):
                kp.pion_prefix_warm(sid, l, H, D, dev_recs[1][2 * l], dev_recs[1][2 * l + 1], 1)
    torch.cuda.synchronize()
    warm_us = (time.perf_counter() - t0) * 1e6 / (reps * L)
    kp.pion_prefix_drop(sid, -1)

    cpu = None
    if oracle_leg(args):
        i = [0]

        def one_layer_side():
            ovs.fetch_f32(recs[i[0] % len(recs)], ovs.MLX4G32, kv, 0, N)
            i[0] += 1
        n, el = cpu_time(one_layer_side, args.cpu_seconds)
        cpu = {"value": round(n * per_launch / el / 1e9, 3), "unit": "GB/s", "cores": 1,
               "kind": "oracle", "sample": f"{n} whole layer-side fetches of this workload ({el:.1f} s)"}
    return {
        "value": nbytes / (ms * 1e-3) / 1e9, "unit": "GB/s", "ms_per_step": ms,
        "dtype": "int4 codes + fp16 scale/bias -> fp32",
        "config": {"workload": f"V-store fetch, mlx4g32 records -> fp32, {L} layers x K,V, "
                               f"H={H} N={N} D={D} (kv={kv}, {rb} B/token)",
                   "bytes_per_step": nbytes,
                   "memory_side_cache": f"cold: steps rotate over {NCOPY} copies of the records"},
        "roofline": {"bound": "hbm", "achieved": per_launch / (launch_us * 1e-6) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "traffic": None,
                     "avg_launch_us": launch_us},
        "warm": {"value": round(nbytes / (wms * 1e-3) / 1e9, 3), "unit": "GB/s",
                 "note": "one copy of the records every step (memory-side cache warm)"},
        "warm_call": {"value": round(warm_us, 1), "unit": "us per layer",
                      "note": "pion_prefix_warm, K and V of one layer, mlx4g32 records -> fp16 "
                              "slot replacing the live one (allocation and free included)"},
        "cpu_baseline": cpu,
    }


def _finish_roofline(roof):
    roof["achieved"] = round(roof["achieved"], 2)
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    if "avg_launch_us" in roof:
        roof["avg_launch_us"] = round(roof["avg_launch_us"], 3)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    # Inputs of the default run, and the oracle timed on the host cores, before anything
    # touches the GPU (the worker processes are forked from this process).
    pre, cpu = {}, {}
    if args.config in (2, 3) and args.copy_bytes <= 0:
        import synth
        if args.config == 2:
            pre["decode"] = [synth.generate(synth.DECODE, l) for l in range(synth.DECODE.layers)]
        if args.config == 3 or args.mode == "layers":
            pre["prefill"] = synth.generate(synth.PREFILL)
        if not args.no_cpu_baseline:
            cpu = cpu_baselines(pre.get("decode"), pre.get("prefill"))
    import torch
    if args.copy_bytes > 0:
        x = torch.ones(args.copy_bytes, dtype=torch.uint8, device="cuda:0")
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "copies": 5}), flush=True)
        return
    import kv_cache_prefix_amd as kp
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(device=dev)
    if args.config == 2:
        r = run_decode(args, torch, kp, synth, dev, stream, inputs=pre.get("decode"),
                       cpu=cpu.get("decode"))
        if args.mode == "layers":   # the default run: both halves of the metric
            bq = run_prefill(args, torch, kp, synth, dev, stream, inp=pre.get("prefill"),
                             cpu=cpu.get("prefill"), calls=max(args.steps, 100))
            _finish_roofline(bq["roofline"])
            r["batched_q"] = {k: (round(v, 4) if isinstance(v, float) else v)
                              for k, v in bq.items()}
            r["batched_q"]["mfma_ceiling"] = mfma_ceiling(torch, kp, dev, stream)
            r["stream_ceiling"] = stream_ceiling(torch, kp, dev, stream)
    elif args.config == 3:
        r = run_prefill(args, torch, kp, synth, dev, stream, inp=pre.get("prefill"),
                        cpu=cpu.get("prefill"))
        r["mfma_ceiling"] = mfma_ceiling(torch, kp, dev, stream)
    else:
        runner = {1: run_tiny, 4: run_mlx4, 5: run_sparse, 6: run_query_sparse,
                  7: run_vstore, 8: run_sweep}[args.config]
        r = runner(args, torch, kp, synth, dev, stream)
    roof = r["roofline"]
    if roof is not None:
        _finish_roofline(roof)
    line = {
        "metric": METRIC,
        "value": round(r["value"], 3),
        "unit": r["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": r["unit"] != "us/query",
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": r["dtype"],
        "data": "synthetic (seeded numpy generators; see synth/)",
        "config": r["config"],
        "roofline": roof,
        "cpu_baseline": r["cpu_baseline"],
    }
    for extra in ("warm", "batched_q", "stream_ceiling", "mfma_ceiling", "single_query",
                  "warm_call",
                  "quantize", "fp16_resident", "sweep", "kmean_read_ceiling"):
        if extra in r:
            line[extra] = r[extra]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
