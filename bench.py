#!/usr/bin/env python3
"""Benchmark: fp32 inclusive sum scan of n = 1e8 elements on one MI355X.

A step is one scan_inclusive call (one kernel launch of the single-pass
look-back scan) over the resident 1e8-element fp32 array (uniform [0,1),
seed 1).  W untimed warmup steps, then K timed steps bracketed by device
synchronisation, timed with HIP events on the stream the kernels run on.
The K timed calls are captured into one HIP graph and replayed once, so the
time between launches is the device's, not the Python host's (--eager
launches them one by one).

Prints one JSON line with the throughput (GElem/s), the roofline of the scan
kernel (algorithmic bytes = one read + one write of n fp32 values per launch,
over the measured average launch duration, against 8 TB/s HBM), the copy
ceiling measured the same way, and the CPU oracle timed on this host.

Beside the headline figure, "rows" times every other workload of the path
once each: int32 2^20 inclusive and exclusive, fp64 1e7, fp32 1e7 with and
without the operator's identity (the pages' "no neutral" row), the reduce-then-scan
comparison on the fp32 1e8 array, the four 2-D scans (4096 x 4096 along rows
and along columns, 1e6 x 8 along its long axis, 2 x 1e7 along rows),
compaction of 1e7 fp32 with x > 0.5, its stable partition, count-scan-emit
packing of 1e7 Poisson(3) counts, the segmented scan over those segments, and
the 136-byte and 96-byte struct scans of 1e6 elements.  Each row
rotates over enough copies of its buffers (> 512 MB in all) that no call
finds its data in the 256 MB Infinity Cache, replays the calls from a HIP
graph (so small launches are not timed against the Python host), and reports
the algorithmic bytes of one call over its average duration.  Each row is
also timed the way AcceleratedKernels.jl PR #208 times its table (timing
paragraph): the device time of one call, best of 20, as the median (and
range) of 3 runs interleaved across the rows.
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
TRAFFIC_BYTES = 8.010e8
TRAFFIC_SOURCES_SHA = "2ea649ecb2e64ddc"


def _kernel_sources_sha():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "stream_compaction_wave64_amd", "csrc")
    for f in ("lookback.hip", "pipeline.hpp", "tile.hpp", "device.hpp"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--algo", default="lookback", choices=["lookback", "reduce_then_scan"])
    ap.add_argument("--block", type=int, default=0, help="tuning: threads per workgroup")
    ap.add_argument("--ipt", type=int, default=0, help="tuning: items per thread")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle leg (profiling runs)")
    ap.add_argument("--no-verify", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch the timed headline steps one by one instead of from one HIP graph")
    ap.add_argument("--no-rows", action="store_true", help="time only the headline fp32 1e8 scan")
    ap.add_argument("--row-steps", type=int, default=20, help="calls timed per row")
    ap.add_argument("--rows", default="", help="comma-separated row names to time (default: every row)")
    return ap.parse_args()


def _upload_graph(g, stream):
    """Upload the instantiated graph to the device before it is timed, so that
    the timed replay does not include the one-time upload (no kernel runs)."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        hip.hipGraphUpload.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        rc = hip.hipGraphUpload(ctypes.c_void_p(g.raw_cuda_graph_exec()), ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            print(f"# hipGraphUpload returned {rc}; the timed replay includes the upload", file=sys.stderr)
    except (OSError, AttributeError, RuntimeError, TypeError) as e:
        print(f"# graph upload skipped ({e}); the timed replay includes the upload", file=sys.stderr)


def timed(fn, steps, warmup, graph=True):
    """ms per step: `warmup` eager calls, then the `steps` calls, launched
    from one HIP graph holding all of them (default) or one by one.  All on
    one side stream, whose workspace the warmup allocates (at least one
    warmup call with a graph, so nothing is allocated during capture)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(max(warmup, 1) if graph else warmup):
            fn()
        torch.cuda.synchronize()
        g = None
        if graph:
            g = torch.cuda.CUDAGraph()
            g.capture_begin()
            try:
                for _ in range(steps):
                    fn()
            finally:
                g.capture_end()
            _upload_graph(g, side)
            torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(side)
        if g is not None:
            g.replay()
        else:
            for _ in range(steps):
                fn()
        end.record(side)
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
            "host_cpus": os.cpu_count(), "cpu_model": _cpu_model()}, ref


def _cpu_model():
    """The host CPU's model name from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ------------------------------------------------------------------ rows
COLD_BYTES = 512 << 20  # buffers touched per rotation: twice the Infinity Cache


class _Row:
    """One workload: `sets` copies of its buffers and a call per copy."""

    def __init__(self, name, workload, elems, alg_bytes, set_bytes, make, check=None):
        self.name, self.workload, self.elems, self.alg_bytes = name, workload, elems, alg_bytes
        self.sets = max(1, -(-COLD_BYTES // max(set_bytes, 1)))
        self.make, self.check = make, check


def _rows(dev, lib, binding, inputs):
    """Row definitions; each make(k) returns (call(stream), outputs) for buffer set k."""
    import torch
    vp = lambda t: t.data_ptr()  # noqa: E731
    null = binding._tuning(None)
    rows = []

    def ws_for(call, dtype, op, outer, length, inner, tuning=None):
        p = binding.plan(call, dtype, op, outer, length, inner, tuning)
        return torch.zeros(max(int(p["workspace_bytes"]), 1 << 16), dtype=torch.uint8, device=dev)

    def scan_row(name, workload, host, width=1, excl=False, algo=None, elems=None, tuning=None):
        x0 = torch.from_numpy(host).to(dev)
        n = x0.numel() // width
        tun = dict(tuning or {}, **({"algo": algo} if algo else {})) or None
        ws = ws_for("scan", x0.dtype, "sum", 1, n, width, tun)
        fn = lib.scan_exclusive if excl else lib.scan_inclusive
        t = binding._tuning(tun)
        dt = binding._dtype(x0)

        def make(k):
            x = x0 if k == 0 else x0.clone()
            y = torch.empty_like(x)
            return (lambda s: fn(vp(x), vp(y), n, dt, 0, width, vp(ws), ws.numel(), t, s)), [y]
        b = x0.numel() * x0.element_size()
        rows.append(_Row(name, workload, elems or n, 2 * b, 2 * b, make))

    def dim_row(name, workload, host, dim):
        x0 = torch.from_numpy(np.ascontiguousarray(host)).to(dev)
        shape = list(x0.shape)
        outer = int(np.prod(shape[:dim], dtype=np.int64))
        length = shape[dim]
        inner = int(np.prod(shape[dim + 1:], dtype=np.int64))
        ws = ws_for("scan", x0.dtype, "sum", outer, length, inner)
        dt = binding._dtype(x0)

        def make(k):
            x = x0 if k == 0 else x0.clone()
            y = torch.empty_like(x)
            return (lambda s: lib.scan_dim(vp(x), vp(y), outer, length, inner, dt, 0, 0, vp(ws), ws.numel(),
                                           null, s)), [y]
        b = x0.numel() * x0.element_size()
        rows.append(_Row(name, workload, x0.numel(), 2 * b, 2 * b, make))

    scan_row("int32_incl_2p20", "int32 inclusive sum scan, n=2^20, uniform 0..100, seed 0",
             inputs.int32_uniform_0_100(2 ** 20, 0))
    scan_row("int32_excl_2p20", "int32 exclusive sum scan, n=2^20, uniform 0..100, seed 0",
             inputs.int32_uniform_0_100(2 ** 20, 0), excl=True)
    scan_row("fp64_incl_1e7", "fp64 inclusive sum scan, n=1e7, uniform [-1,1), seed 1",
             inputs.f64_uniform_pm1(10 ** 7, 1))
    f7 = inputs.f32_uniform_01(10 ** 7, 1)
    scan_row("fp32_incl_1e7", "fp32 inclusive sum scan, n=1e7, uniform [0,1), seed 1", f7)
    scan_row("fp32_incl_1e7_no_neutral", "fp32 inclusive sum scan, n=1e7, uniform [0,1), seed 1, computed "
             "without the operator's identity (Optional partials)", f7, tuning={"no_identity": 1})
    del f7
    scan_row("fp32_incl_1e8_reduce_then_scan", "fp32 inclusive sum scan, n=1e8, reduce-then-scan (3 launches)",
             inputs.f32_uniform_01(N, 1), algo="reduce_then_scan")
    sq, tall, wide = inputs.dims_arrays(3)
    dim_row("fp32_4096x4096_along_rows", "4096 x 4096 fp32 row-major, scan along rows (dim 1), seed 3", sq, 1)
    dim_row("fp32_4096x4096_along_cols", "4096 x 4096 fp32 row-major, scan along columns (dim 0), seed 3", sq, 0)
    dim_row("fp32_1e6x8_along_dim0", "1e6 x 8 fp32, scan along the 1e6 axis (dim 0), seed 3", tall, 0)
    dim_row("fp32_2x1e7_along_rows", "2 x 1e7 fp32, scan along rows (dim 1), seed 3", wide, 1)
    del sq, tall, wide

    xc, counts = inputs.compaction_inputs(10 ** 7, 4)
    x0 = torch.from_numpy(xc).to(dev)
    n = x0.numel()
    kept = int(np.count_nonzero(xc > np.float32(0.5)))
    ws_c = ws_for("compact", torch.float32, "sum", 1, n, 1)

    def make_compact(k):
        x = x0 if k == 0 else x0.clone()
        idx = torch.empty(n, dtype=torch.int32, device=dev)
        cnt = torch.empty(1, dtype=torch.int32, device=dev)
        return (lambda s: lib.compact_if(vp(x), n, 3, 0, 0.5, vp(idx), vp(cnt), vp(ws_c), ws_c.numel(), null,
                                         s)), [idx, cnt]
    rows.append(_Row("compact_fp32_gt_half_1e7", "compaction of 1e7 fp32 uniform [0,1) with x > 0.5, seed 4",
                     n, 4 * n + 4 * kept + 4, 4 * n + 4 * kept, make_compact))

    ws_q = ws_for("partition", torch.float32, "sum", 1, n, 1)

    def make_partition(k):
        x = x0 if k == 0 else x0.clone()
        vals = torch.empty(n, dtype=torch.float32, device=dev)
        idx = torch.empty(n, dtype=torch.int32, device=dev)
        cnt = torch.empty(1, dtype=torch.int32, device=dev)
        return (lambda s: lib.partition_if(vp(x), n, 3, 0, 0.5, vp(vals), vp(idx), vp(cnt), vp(ws_q), ws_q.numel(),
                                           null, s)), [vals, idx, cnt]
    # algorithmic bytes: one read of x, the values and their source indices
    # written once (the count pass's second read of x is not counted)
    rows.append(_Row("partition_fp32_gt_half_1e7", "stable partition of 1e7 fp32 uniform [0,1) by x > 0.5: "
                     "values and source indices (2 launches), seed 4", n, 12 * n + 4, 12 * n, make_partition))

    c0 = torch.from_numpy(counts).to(dev)
    total = int(counts.sum(dtype=np.int64))
    ws_p = ws_for("pack", torch.int32, "sum", 1, n, 1)

    def make_pack(k):
        c = c0 if k == 0 else c0.clone()
        off = torch.empty(n + 1, dtype=torch.int32, device=dev)
        rec = torch.empty(total, dtype=torch.int32, device=dev)

        def call(s):
            st = lib.pack_offsets(vp(c), n, vp(off), vp(ws_p), ws_p.numel(), null, s)
            return st or lib.pack_emit_neighbors(vp(off), n, vp(rec), s)
        return call, [off, rec]
    rows.append(_Row("pack_offsets_emit_1e7", "count-scan-emit: offsets of 1e7 Poisson(3) int32 counts, then "
                     "emit of every record (2 launches), seed 4", n, 4 * n + 4 * (n + 1) + 4 * total,
                     4 * n + 8 * (n + 1) + 4 * total, make_pack))
    del xc, counts

    # segmented scan over the count-scan-emit layout: the 1e7 Poisson(3)
    # counts as segment lengths (offsets from the library's pack_offsets,
    # set-up only), one fp32 value per record
    counts_s, vals_s = inputs.segmented_inputs(10 ** 7, 4)
    nseg, nv = counts_s.size, vals_s.size
    c_dev = torch.from_numpy(counts_s).to(dev)
    off_s = torch.empty(nseg + 1, dtype=torch.int32, device=dev)
    ws_o = ws_for("pack", torch.int32, "sum", 1, nseg, 1)
    assert lib.pack_offsets(vp(c_dev), nseg, vp(off_s), vp(ws_o), ws_o.numel(), null,
                            torch.cuda.current_stream(dev).cuda_stream) == 0
    v0 = torch.from_numpy(vals_s).to(dev)
    ws_s = ws_for("segmented", torch.float32, "sum", nseg, nv, 1)

    def make_seg(k):
        v = v0 if k == 0 else v0.clone()
        o = off_s if k == 0 else off_s.clone()
        y = torch.empty_like(v)
        return (lambda s: lib.scan_segmented(vp(v), vp(y), nv, vp(o), nseg, 3, 0, 0, vp(ws_s), ws_s.numel(), null,
                                             s)), [y]
    rows.append(_Row("segscan_fp32_poisson3_1e7", "segmented inclusive sum of ~3e7 fp32 uniform [0,1) records in "
                     "1e7 Poisson(3)-length segments (offsets from pack_offsets), seed 4", nv,
                     8 * nv + 4 * (nseg + 1), 8 * nv + 4 * (nseg + 1), make_seg))
    del counts_s, vals_s

    s64, s32 = inputs.struct_inputs(10 ** 6, 5)
    scan_row("struct136_fp64x17_1e6", "1e6 elements of 17 fp64 (136 B), elementwise sum, seed 5", s64.reshape(-1),
             width=17)
    scan_row("struct96_fp32x24_1e6", "1e6 elements of 24 fp32 (96 B), elementwise sum, seed 5", s32.reshape(-1),
             width=24)
    return rows


def prepare_row(row):
    """The row's calls and outputs, one per buffer set."""
    calls, outs = [], []
    for k in range(row.sets):
        c, o = row.make(k)
        calls.append(c)
        outs.append(o)
    return calls, outs


def best_single_call_us(row, calls, lib, count=20):
    """Best device time of `count` single calls (HIP events around each call
    on its stream), cycling through the buffer sets."""
    import torch
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(count)]
    for i in range(count):
        ev[i][0].record(stream)
        st = calls[i % len(calls)](stream.cuda_stream)
        ev[i][1].record(stream)
        if st != 0:
            raise RuntimeError(f"{row.name}: {lib.scan_status_string(st).decode()} (status {st})")
    torch.cuda.synchronize()
    return min(a.elapsed_time(b) * 1e3 for a, b in ev)


def time_row(row, calls, outs, lib, steps, warmup, use_graph=True):
    """Average duration of one call of the row, cycling through its buffer sets."""
    import torch
    stream = torch.cuda.current_stream()

    def run_all(s):
        for c in calls:
            st = c(s)
            if st != 0:
                raise RuntimeError(f"{row.name}: {lib.scan_status_string(st).decode()} (status {st})")

    for _ in range(max(warmup, 1)):
        run_all(stream.cuda_stream)
    torch.cuda.synchronize()
    eager = [[t.clone() for t in o] for o in outs[:1]]
    graph = None
    if use_graph:
        try:
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                g.capture_begin()
                try:
                    run_all(side.cuda_stream)
                finally:
                    g.capture_end()
            stream.wait_stream(side)
            torch.cuda.synchronize()
            graph = g
        except Exception as e:  # report and time eagerly
            print(f"# {row.name}: graph capture failed ({e}); timing eager calls", file=sys.stderr)
            graph = None
    reps = max(2, -(-steps // row.sets))
    fn = graph.replay if graph is not None else (lambda: run_all(stream.cuda_stream))
    fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1e3 / (reps * row.sets)
    same = all(_same(a, b) for a, b in zip(eager[0], outs[0]))
    gbs = row.alg_bytes / (us * 1e-6) / 1e9
    return {"workload": row.workload, "us_per_call": round(us, 3), "gelem_s": round(row.elems / us / 1e3, 3),
            "alg_bytes": int(row.alg_bytes), "achieved_gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
            "buffer_sets": row.sets, "hip_graph": graph is not None, "replay_matches_eager": same}


def _same(a, b):
    import torch
    if a.dtype.is_floating_point:
        # look-back combines predecessors in an order that depends on timing
        return bool(torch.allclose(a, b, rtol=1e-5, atol=1e-3))
    return bool(torch.equal(a, b))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        return 2
    import torch
    import stream_compaction_wave64_amd as sw
    from stream_compaction_wave64_amd import inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x_host = inputs.f32_uniform_01(N, seed=1)
    x = torch.from_numpy(x_host).to(dev)
    out = torch.empty_like(x)
    tuning = {"algo": args.algo}
    if args.block:
        tuning["block_size"] = args.block
    if args.ipt:
        tuning["items_per_thread"] = args.ipt
    plan = sw.plan("scan", torch.float32, "sum", 1, N, tuning=tuning)

    graph = not args.eager
    ms = timed(lambda: sw.scan_inclusive(x, out=out, tuning=tuning), args.steps, args.warmup, graph)
    copy_out = torch.empty_like(x)
    ms_copy = timed(lambda: sw.scan_copy(x, copy_out), args.steps, args.warmup, graph)

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
                   "num_tiles": plan["num_tiles"],
                   "launch": "one HIP graph of the timed steps" if graph else "one call per step"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": TRAFFIC_BYTES if (_kernel_sources_sha() == TRAFFIC_SOURCES_SHA
                                                  and args.algo == "lookback" and not args.block
                                                  and not args.ipt) else None},
        "copy_ceiling": {"achieved": round(copy_gbs, 1), "unit": "GB/s", "frac": round(copy_gbs / HBM_PEAK_GBS, 4),
                         "scan_vs_copy": round(achieved / copy_gbs, 4)},
    }

    if not args.no_rows:
        from stream_compaction_wave64_amd import binding
        lib = binding.load_library()
        rows = {}
        prepared = []
        wanted = set(filter(None, args.rows.split(",")))
        for row in _rows(dev, lib, binding, inputs):
            if wanted and row.name not in wanted:
                continue
            calls, outs = prepare_row(row)
            rows[row.name] = time_row(row, calls, outs, lib, args.row_steps, 2)
            prepared.append((row, calls))
        # AcceleratedKernels.jl PR #208's method: best of 20 single calls,
        # median of 3 runs interleaved across the rows
        best = {row.name: [] for row, _ in prepared}
        for _ in range(3):
            for row, calls in prepared:
                best[row.name].append(best_single_call_us(row, calls, lib))
        for row, _ in prepared:
            b = sorted(best[row.name])
            rows[row.name]["best_of_20_us"] = round(b[1], 3)
            rows[row.name]["best_of_20_range_us"] = [round(b[0], 3), round(b[2], 3)]
            rows[row.name]["best_of_20_frac"] = round(row.alg_bytes / (b[1] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        del prepared
        torch.cuda.empty_cache()
        result["rows"] = rows

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
