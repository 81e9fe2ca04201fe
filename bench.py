#!/usr/bin/env python3
"""Benchmark: fp32 inclusive sum scan of n = 1e8 elements on one MI355X.

A step is one scan_inclusive call (one kernel launch of the single-pass
look-back scan) over the resident 1e8-element fp32 array (uniform [0,1),
seed 1).  W untimed warmup steps, then K timed steps bracketed by device
synchronisation, timed with HIP events on the stream the kernels run on.

Prints one JSON line with the throughput (GElem/s), the roofline of the scan
kernel (algorithmic bytes = one read + one write of n fp32 values per launch,
over the measured average launch duration, against 8 TB/s HBM), the copy
ceiling measured the same way, and the CPU oracle timed on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "GElem/s and % of HBM roofline, fp32 inclusive scan n=1e8 on 1 MI355X"
HBM_PEAK_GBS = 8000.0
N = 10 ** 8
# HBM bytes per launch measured with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE on
# the scan kernel, each scaled by what the counter reads for the copy kernel of
# known size (profiles/lookback_scan_fp32_1e8_hbm_counters.md).  Valid only for
# the kernel sources that were measured: reported as null once they change.
TRAFFIC_BYTES = 8.044e8
TRAFFIC_SOURCES_SHA = "42001f70c2cfdd68"


def _kernel_sources_sha():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "stream_compaction_wave64_amd", "csrc")
    for f in ("lookback.hip", "tile.hpp", "device.hpp"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--algo", default="lookback", choices=["lookback", "reduce_then_scan"])
    ap.add_argument("--block", type=int, default=0, help="tuning: threads per workgroup")
    ap.add_argument("--ipt", type=int, default=0, help="tuning: items per thread")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle leg (profiling runs)")
    ap.add_argument("--no-verify", action="store_true")
    return ap.parse_args()


def timed(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms per step


def cpu_baseline(x: np.ndarray):
    """The oracle as it stands (sequential C, one thread) on the full array."""
    import oracle
    oracle.build(force=False)
    best = float("inf")
    ref = None
    runs = 0
    t_total = time.perf_counter()
    while runs < 3 or (time.perf_counter() - t_total < 10.0 and runs < 10):
        t0 = time.perf_counter()
        ref = oracle.scan(x, "sum")
        best = min(best, time.perf_counter() - t0)
        runs += 1
    return {"value": round(x.size / best / 1e9, 4), "unit": "GElem/s", "cores": 1, "kind": "oracle",
            "sample": f"full {x.size:.0e}-element fp32 array, sequential fp64 accumulation, best of {runs} runs",
            "host_cpus": os.cpu_count()}, ref


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        return 2
    import torch
    import stream_compaction_wave64_amd as sw
    from stream_compaction_wave64_amd import inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    x_host = inputs.f32_uniform_01(N, seed=1)
    x = torch.from_numpy(x_host).to(dev)
    out = torch.empty_like(x)
    tuning = {"algo": args.algo}
    if args.block:
        tuning["block_size"] = args.block
    if args.ipt:
        tuning["items_per_thread"] = args.ipt
    plan = sw.plan("scan", torch.float32, "sum", 1, N, tuning=tuning)

    ms = timed(lambda: sw.scan_inclusive(x, out=out, tuning=tuning), args.steps, args.warmup, stream)
    copy_out = torch.empty_like(x)
    ms_copy = timed(lambda: sw.scan_copy(x, copy_out), args.steps, args.warmup, stream)

    alg_bytes = 2 * N * 4
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    copy_gbs = alg_bytes / (ms_copy * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(N / (ms * 1e-3) / 1e9, 3),
        "unit": "GElem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "fp32 inclusive sum scan, n=1e8, uniform [0,1) float32, seed 1",
                   "n": N, "op": "sum", "algo": args.algo, "kernel": plan["kernel"],
                   "launches_per_step": plan["launches"], "block": plan["block_size"],
                   "items_per_thread": plan["items_per_thread"], "tile_elems": plan["tile_elems"],
                   "num_tiles": plan["num_tiles"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": TRAFFIC_BYTES if (_kernel_sources_sha() == TRAFFIC_SOURCES_SHA
                                                  and args.algo == "lookback" and not args.block
                                                  and not args.ipt) else None},
        "copy_ceiling": {"achieved": round(copy_gbs, 1), "unit": "GB/s", "frac": round(copy_gbs / HBM_PEAK_GBS, 4),
                         "scan_vs_copy": round(achieved / copy_gbs, 4)},
    }

    ref = None
    if not args.no_cpu_baseline:
        result["cpu_baseline"], ref = cpu_baseline(x_host)
    if not args.no_verify:
        import oracle
        if ref is None:
            ref = oracle.scan(x_host, "sum")
        got = out.cpu().numpy().astype(np.float64)
        tol = 1e-5 * ref + 1e-6  # inputs are non-negative: P_i equals the prefix
        result["parity"] = bool(np.all(np.abs(got - ref) <= tol))
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
