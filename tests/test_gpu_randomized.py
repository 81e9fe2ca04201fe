"""Seeded randomized parity sweep over every entry point: array lengths drawn
around tile and vector boundaries (and at random), every dtype and operator,
inclusive and exclusive, aligned and misaligned data, and tunings that change
the tile shape, the grid, the algorithm and the chunk count.  Each case is
compared with the oracle under the usual rules (bit-exact for integers,
max/min, indices and moved values; the stated tolerance for fp sums and
products).  The draw is fixed by the seed, so a failure names a reproducible
case."""
import numpy as np
import pytest
import torch

import oracle
import stream_compaction_wave64_amd as sw
from stream_compaction_wave64_amd import inputs
from gpu_util import DEV, assert_scan_matches, assert_segscan_matches, to_dev, to_host

pytestmark = pytest.mark.gpu

DTYPES = [np.int32, np.uint32, np.int64, np.float32, np.float64]
OPS = ["sum", "prod", "max", "min"]
TORCH_OF = {np.int32: torch.int32, np.uint32: torch.uint32, np.int64: torch.int64, np.float32: torch.float32,
            np.float64: torch.float64}
CASES = 150


def _length(rng, tile):
    kind = rng.integers(0, 4)
    if kind == 0:  # just around a multiple of the tile
        return int(max(1, tile * rng.integers(1, 9) + rng.integers(-5, 6)))
    if kind == 1:  # tiny
        return int(rng.integers(1, 200))
    if kind == 2:  # a few vectors off a vector boundary
        return int(4 * rng.integers(1, 20000) + rng.integers(0, 4))
    return int(rng.integers(1, 600_000))


def _values(dt, n, seed, op):
    kind = "near1" if op == "prod" and np.issubdtype(dt, np.floating) else "wide"
    if op == "sum" and np.issubdtype(dt, np.floating):
        kind = "default"
    return inputs.generic(dt, n, seed, kind)


def _device(x, offset):
    if not offset:
        return to_dev(x), None
    buf = to_dev(np.concatenate([np.zeros(offset, x.dtype), x]))
    out = torch.empty(x.size + offset, dtype=buf.dtype, device=DEV)
    return buf[offset:], out[offset:]


def _tuning(rng, vec):
    choices = [None,
               {"block_size": 256, "items_per_thread": vec},
               {"grid_blocks": int(rng.integers(1, 40))},
               {"algo": "reduce_then_scan"},
               {"algo": "reduce_then_scan", "rts_blocks": int(rng.integers(1, 300))}]
    return choices[int(rng.integers(0, len(choices)))]


def test_random_scans():
    rng = np.random.default_rng(2026)
    for case in range(CASES):
        dt = DTYPES[int(rng.integers(0, len(DTYPES)))]
        op = OPS[int(rng.integers(0, len(OPS)))]
        excl = bool(rng.integers(0, 2))
        vec = 16 // np.dtype(dt).itemsize
        tile = sw.plan("scan", torch.float64 if vec == 2 else torch.float32, "sum", 1, 1 << 20)["tile_elems"]
        n = _length(rng, tile)
        offset = int(rng.integers(0, vec)) if rng.integers(0, 4) == 0 else 0
        tuning = _tuning(rng, vec)
        x = _values(dt, n, 100 + case, op)
        xd, out = _device(x, offset)
        fn = sw.scan_exclusive if excl else sw.scan_inclusive
        r = fn(xd, op=op, out=out, tuning=tuning)
        torch.cuda.synchronize()
        assert_scan_matches(x, to_host(r), op, excl,
                            what=f"case {case}: {np.dtype(dt).name} {op} excl={excl} n={n} off={offset} {tuning}")


def test_random_scan_dims():
    rng = np.random.default_rng(2027)
    for case in range(CASES // 2):
        dt = DTYPES[int(rng.integers(0, len(DTYPES)))]
        op = OPS[int(rng.integers(0, len(OPS)))]
        excl = bool(rng.integers(0, 2))
        rows, cols = int(rng.integers(1, 700)), int(rng.integers(1, 700))
        dim = int(rng.integers(0, 2))
        x = _values(dt, rows * cols, 200 + case, op).reshape(rows, cols)
        r = sw.scan_dim(to_dev(x), dim, op=op, exclusive=excl)
        torch.cuda.synchronize()
        dims = (1, rows, cols) if dim == 0 else (rows, cols, 1)  # (outer, len, inner)
        assert_scan_matches(x.ravel(), to_host(r).ravel(), op, excl, dims=dims,
                            what=f"case {case}: {np.dtype(dt).name} {op} excl={excl} {rows}x{cols} dim={dim}")


def test_random_compaction_and_partition():
    rng = np.random.default_rng(2028)
    cmps = ["gt", "ge", "lt", "le", "eq", "ne"]
    for case in range(CASES):
        n = _length(rng, 14336)
        dt = [np.float32, np.int32, np.uint32][int(rng.integers(0, 3))]
        cmp = cmps[int(rng.integers(0, len(cmps)))]
        if dt == np.float32:
            x = rng.random(n, dtype=np.float32)
            t = float(rng.choice([0.0, 0.25, 0.5, 0.99]))
            x[rng.integers(0, n, max(1, n // 50))] = np.float32(t)  # ties
        else:
            x = rng.integers(0, 64, n).astype(dt)
            t = int(rng.integers(0, 64))
        tuning = [None, {"block_size": 256, "items_per_thread": 4}, {"grid_blocks": int(rng.integers(1, 30))}][
            int(rng.integers(0, 3))]
        what = f"case {case}: {np.dtype(dt).name} {cmp} {t} n={n} {tuning}"
        idx, count = sw.compact_if(to_dev(x), cmp, t, tuning=tuning)
        torch.cuda.synchronize()
        ref = oracle.compact(x, cmp, t)
        c = int(count.item())
        assert c == ref.size, what
        assert np.array_equal(to_host(idx)[:c], ref), what
        vals, vidx, k = oracle.partition(x, cmp, t)
        out, oidx, count = sw.partition_if(to_dev(x), cmp, t, tuning=tuning)
        torch.cuda.synchronize()
        assert int(count.item()) == k, what
        assert np.array_equal(to_host(out)[:n].view(np.uint32), vals.view(np.uint32)), what
        assert np.array_equal(to_host(oidx)[:n], vidx), what


def test_random_packing_and_segments():
    rng = np.random.default_rng(2029)
    for case in range(CASES // 2):
        nobj = int(rng.integers(1, 300_000))
        mean = float(rng.choice([0.2, 1.0, 3.0, 17.0]))
        counts = rng.poisson(mean, nobj).astype(np.int32)
        ref_off, ref_total = oracle.pack_offsets(counts)
        off = sw.pack_offsets(to_dev(counts))
        torch.cuda.synchronize()
        got_off = to_host(off)
        assert np.array_equal(got_off, ref_off), f"case {case}: offsets nobj={nobj} mean={mean}"
        total = int(ref_total)
        if total > 0:
            rec = sw.pack_emit_neighbors(off, total)
            torch.cuda.synchronize()
            assert np.array_equal(to_host(rec), oracle.pack_emit(ref_off)), f"case {case}: records"
            dt = DTYPES[int(rng.integers(0, len(DTYPES)))]
            op = OPS[int(rng.integers(0, len(OPS)))]
            excl = bool(rng.integers(0, 2))
            x = _values(dt, total, 300 + case, op)
            tuning = [None, {"algo": "lookback"}, {"block_size": 256, "items_per_thread": 16 // np.dtype(dt).itemsize},
                      {"algo": "lookback", "grid_blocks": int(rng.integers(1, 20))}][int(rng.integers(0, 4))]
            r = sw.scan_segmented(to_dev(x), off, op, excl, tuning=tuning)
            torch.cuda.synchronize()
            assert_segscan_matches(x, ref_off, to_host(r), op, excl,
                                   what=f"case {case}: {np.dtype(dt).name} {op} excl={excl} nobj={nobj} {tuning}")


def test_random_single_pass_paths():
    # The one-step paths at random sizes: whole arrays and rows of 8 MiB up to
    # the resident pass's capacity (most with whole 128-bit vectors, some
    # not: those fall back to the pipeline; whole arrays from 28 MiB, 40 MiB
    # for 8-byte elements, with two tiles per workgroup), and column scans
    # whose register tiles fit one per compute unit.  Every case against the oracle; the planner's choice is
    # recorded so that the sweep keeps reaching them.
    rng = np.random.default_rng(2030)
    kernels = {}
    for case in range(24):
        dt = DTYPES[int(rng.integers(0, len(DTYPES)))]
        op = OPS[int(rng.integers(0, len(OPS)))]
        excl = bool(rng.integers(0, 2))
        es = np.dtype(dt).itemsize
        vec = 16 // es
        cap = 256 * (17 if es == 4 else 21) * 960 * vec
        outer = int(rng.integers(1, 4)) if rng.integers(0, 3) == 0 else 1
        lo = -(-(8 << 20) // (es * outer))
        length = int(rng.integers(lo, cap // outer + 1))
        if rng.integers(0, 4):
            length -= length % vec  # whole vectors (the resident pass)
        p = sw.plan("scan", TORCH_OF[dt], op, outer, length)
        kind = p["kernel"] + (" x2" if p["tiles_per_block"] == 2 else "")
        kernels[kind] = kernels.get(kind, 0) + 1
        x = _values(dt, outer * length, 300 + case, op)
        if outer == 1:
            fn = sw.scan_exclusive if excl else sw.scan_inclusive
            r = fn(to_dev(x), op=op)
        else:
            r = sw.scan_dim(to_dev(x.reshape(outer, length)), 1, op=op, exclusive=excl)
        torch.cuda.synchronize()
        assert_scan_matches(x, to_host(r).ravel(), op, excl, dims=(outer, length, 1),
                            what=f"case {case}: {np.dtype(dt).name} {op} excl={excl} {outer}x{length} ({kind})")
    for case in range(12):
        dt = DTYPES[int(rng.integers(0, len(DTYPES)))]
        op = OPS[int(rng.integers(0, len(OPS)))]
        excl = bool(rng.integers(0, 2))
        vec = 16 // np.dtype(dt).itemsize
        tc = 64 * vec  # columns per strip
        cols = vec * int(rng.integers(tc // (2 * vec), 4096 // vec + 1))
        strips = -(-cols // tc)
        rows = int(rng.integers(1, min(4096, 256 * 64 // strips) + 1))
        kind = sw.plan("scan", TORCH_OF[dt], op, 1, rows, cols)["kernel"]
        kernels[kind] = kernels.get(kind, 0) + 1
        x = _values(dt, rows * cols, 400 + case, op).reshape(rows, cols)
        r = sw.scan_dim(to_dev(x), 0, op=op, exclusive=excl)
        torch.cuda.synchronize()
        assert_scan_matches(x.ravel(), to_host(r).ravel(), op, excl, dims=(1, rows, cols),
                            what=f"case {case}: {np.dtype(dt).name} {op} excl={excl} {rows}x{cols} dim 0 ({kind})")
    assert kernels.get("resident", 0) >= 8 and kernels.get("resident x2", 0) >= 8, kernels
    assert kernels.get("columns_lookback", 0) >= 6, kernels


def test_random_no_identity():
    # Inclusive scans without the operator's identity at random sizes, from
    # tiny arrays to the resident pass's range, whole arrays and rows, against
    # the oracle's scan that never uses the identity.
    rng = np.random.default_rng(2031)
    kernels = {}
    for case in range(CASES // 3):
        dt = DTYPES[int(rng.integers(0, len(DTYPES)))]
        op = OPS[int(rng.integers(0, len(OPS)))]
        es = np.dtype(dt).itemsize
        vec = 16 // es
        if rng.integers(0, 3) == 0:  # the resident pass's range
            cap = 256 * (17 if es == 4 else 21) * 960 * vec
            n = int(rng.integers(-(-(8 << 20) // es), cap + 1))
            n -= n % vec
        else:
            n = _length(rng, 19712)
        outer = 1 if rng.integers(0, 3) else int(rng.integers(2, 5))
        n = max(outer, n - n % outer)
        length = n // outer
        tuning = [{"no_identity": 1}, {"no_identity": 1, "block_size": 256, "items_per_thread": vec},
                  {"no_identity": 1, "grid_blocks": int(rng.integers(1, 40))}][int(rng.integers(0, 3))]
        kind = sw.plan("scan", TORCH_OF[dt], op, outer, length, tuning=tuning)["kernel"]
        kernels[kind] = kernels.get(kind, 0) + 1
        x = _values(dt, n, 500 + case, op)
        if outer == 1:
            r = sw.scan_inclusive(to_dev(x), op=op, tuning=tuning)
        else:
            r = sw.scan_dim(to_dev(x.reshape(outer, length)), 1, op=op, tuning=tuning)
        torch.cuda.synchronize()
        assert_scan_matches(x, to_host(r).ravel(), op, False, dims=(outer, length, 1), noid=True,
                            what=f"case {case}: {np.dtype(dt).name} {op} {outer}x{length} {tuning} ({kind})")
    assert kernels.get("resident", 0) > 0 and kernels.get("lookback", 0) > 0, kernels


def test_random_rows_kernel():
    # Many rows that each fit one tile of the rows kernel (one workgroup per
    # row), at random row lengths and counts, against the oracle.
    rng = np.random.default_rng(2032)
    kernels = {}
    for case in range(CASES // 3):
        dt = DTYPES[int(rng.integers(0, len(DTYPES)))]
        op = OPS[int(rng.integers(0, len(OPS)))]
        excl = bool(rng.integers(0, 2))
        vec = 16 // np.dtype(dt).itemsize
        cols = vec * int(rng.integers(64, 2048 + 1))
        rows = int(rng.integers(2, max(3, min(3000, 4_000_000 // cols))))
        kind = sw.plan("scan", TORCH_OF[dt], op, rows, cols)["kernel"]
        kernels[kind] = kernels.get(kind, 0) + 1
        x = _values(dt, rows * cols, 600 + case, op).reshape(rows, cols)
        r = sw.scan_dim(to_dev(x), 1, op=op, exclusive=excl)
        torch.cuda.synchronize()
        assert_scan_matches(x.ravel(), to_host(r).ravel(), op, excl, dims=(rows, cols, 1),
                            what=f"case {case}: {np.dtype(dt).name} {op} excl={excl} {rows}x{cols} ({kind})")
    assert kernels.get("rows", 0) > 0, kernels


def test_random_element_scans():
    # Scans of elements of W components (every built width) at random sizes,
    # shapes and chunk counts, against the oracle's (outer, len, W) scan.
    rng = np.random.default_rng(2033)
    widths = [2, 3, 4, 8, 16, 17, 24]
    for case in range(CASES // 3):
        dt = [np.float32, np.float64, np.int32, np.int64][int(rng.integers(0, 4))]
        op = OPS[int(rng.integers(0, len(OPS)))]
        excl = bool(rng.integers(0, 2))
        w = widths[int(rng.integers(0, len(widths)))]
        n = int(rng.integers(1, 200_000 // w + 2))
        tuning = [None, {"block_size": 64}, {"rts_blocks": int(rng.integers(1, 3000))},
                  {"block_size": 128, "rts_blocks": int(rng.integers(1, 3000))}][int(rng.integers(0, 4))]
        x = _values(dt, n * w, 700 + case, op)
        fn = sw.scan_exclusive if excl else sw.scan_inclusive
        r = fn(to_dev(x), op=op, width=w, tuning=tuning)
        torch.cuda.synchronize()
        assert_scan_matches(x, to_host(r), op, excl, dims=(1, n, w),
                            what=f"case {case}: {np.dtype(dt).name} {op} excl={excl} n={n} w={w} {tuning}")
