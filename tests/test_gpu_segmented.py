"""GPU parity of the ragged segmented scan against the oracle: every dtype and
operator, inclusive and exclusive, on segmentations of every kind -- short
Poisson lengths with empty segments, segments spanning many tiles and
chunks, boundaries on tile edges, one segment, one element per segment,
runs of empty segments -- with vector and element-wise access, small tiles
and few chunks, in place, and the count-scan-emit shape at full size."""
import numpy as np
import pytest
import torch

import oracle
import stream_compaction_wave64_amd as sw
from stream_compaction_wave64_amd import inputs
from gpu_util import DEV, assert_segscan_matches, to_dev, to_host

pytestmark = pytest.mark.gpu

DTYPES = [np.int32, np.uint32, np.int64, np.float32, np.float64]
OPS = ["sum", "prod", "max", "min"]


def _values(dt, n, seed, op):
    kind = "near1" if op == "prod" and np.issubdtype(dt, np.floating) else "wide"
    if op == "sum" and np.issubdtype(dt, np.floating):
        kind = "default"
    return inputs.generic(dt, n, seed, kind)


def _offsets(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def _poisson(n, mean, seed):
    rng = np.random.default_rng(seed)
    lens = rng.poisson(mean, n + 1)
    off = np.concatenate([[0], np.cumsum(lens)])
    off = off[off < n]
    return np.concatenate([off, [n]]).astype(np.int32)


def _run(x, off, op, excl, tuning=None, offset=0, in_place=False):
    if offset:
        buf = to_dev(np.concatenate([np.zeros(offset, x.dtype), x]))
        xd = buf[offset:]
    else:
        xd = to_dev(x)
    r = sw.scan_segmented(xd, to_dev(off), op, excl, out=xd if in_place else None, tuning=tuning)
    torch.cuda.synchronize()
    return to_host(r)


def _check(x, off, op, excl, what="", **kw):
    assert_segscan_matches(x, off, _run(x, off, op, excl, **kw), op, excl, what=what)


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: np.dtype(d).name)
@pytest.mark.parametrize("op", OPS)
def test_segmentations(dt, op):
    n = 200_003
    tile = sw.plan("segmented", torch.empty(0, dtype=torch.float64 if np.dtype(dt).itemsize == 8
                                            else torch.float32).dtype, op, 1, n)["tile_elems"]
    cases = {
        "poisson3": _poisson(n, 3.0, 1),
        "poisson0.5 (many empty)": _poisson(n, 0.5, 2),
        "long": _poisson(n, 40_000.0, 3),
        "tile edges": np.unique(np.concatenate([np.arange(0, n, tile), [n]])).astype(np.int32),
        "one": np.array([0, n], np.int32),
        "each": np.arange(n + 1, dtype=np.int32),
        "empty runs": np.sort(np.concatenate([_poisson(n, 50.0, 4)] * 3)).astype(np.int32),
    }
    x = _values(dt, n, 7, op)
    for name, off in cases.items():
        for excl in (False, True):
            for algo in (None, "lookback"):  # reduce-then-scan (default), single pass
                tu = {"algo": algo} if algo else None
                _check(x, off, op, excl, tuning=tu, what=f"{name} excl={excl} algo={algo}")


@pytest.mark.parametrize("dt", [np.int32, np.float32, np.float64], ids=lambda d: np.dtype(d).name)
def test_small_tiles_few_chunks_misaligned_in_place(dt):
    n = 100_001
    x = _values(dt, n, 8, "sum")
    off = _poisson(n, 25.0, 5)
    vec = 16 // np.dtype(dt).itemsize
    for tuning in ({"block_size": 256, "items_per_thread": vec},
                   {"block_size": 256, "items_per_thread": vec, "rts_blocks": 3},
                   {"rts_blocks": 1},
                   {"algo": "lookback", "block_size": 256, "items_per_thread": vec, "grid_blocks": 3},
                   {"algo": "lookback", "grid_blocks": 1},
                   {"algo": "lookback", "rts_blocks": 3}):
        for excl in (False, True):
            _check(x, off, "sum", excl, tuning=tuning, what=f"{tuning} excl={excl}")
    _check(x, off, "sum", False, offset=1, what="element-wise")
    _check(x, off, "max", True, offset=1, what="element-wise max")
    _check(x, off, "sum", False, in_place=True, what="in place")


def test_edges():
    for n in (1, 2, 5, 1000):
        x = np.arange(1, n + 1, dtype=np.int32)
        for off in (np.array([0, n], np.int32), np.arange(n + 1, dtype=np.int32),
                    np.array([0, 0, 0, n, n], np.int32)):
            for excl in (False, True):
                _check(x, off, "sum", excl, what=f"n={n} {off[:6]}")
    empty = sw.scan_segmented(torch.empty(0, dtype=torch.float32, device=DEV),
                              torch.zeros(1, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert empty.numel() == 0


def test_count_scan_emit_shape_full_size():
    # the bench workload: 1e7 Poisson(3) segments over about 3e7 fp32 values
    counts, vals = inputs.segmented_inputs(10 ** 7, seed=4)
    off, _ = oracle.pack_offsets(counts)
    got = _run(vals, off, "sum", False)
    ref = oracle.scan_segmented(vals, off, "sum")
    p = oracle.segment_abs_prefix(vals, off)
    assert np.all(np.abs(got.astype(np.float64) - ref) <= 1e-5 * p + 1e-6)
    got = _run(vals, off, "max", True)
    assert np.array_equal(got, oracle.scan_segmented(vals, off, "max", exclusive=True).astype(np.float32))


@pytest.mark.parametrize("dt", [np.int32, np.float32, np.float64], ids=lambda d: np.dtype(d).name)
def test_single_pass_dynamic_claiming(dt):
    # A start count that wraps past the grid size never confirms that all
    # workgroups are resident, so the single pass (algo look-back) claims
    # tiles one by one and
    # resolves prefixes with the windowed look-back, whose (flag, value)
    # pairs must combine in tile order.  Long segments carry across many
    # tiles; short ones restart inside tiles.
    from stream_compaction_wave64_amd import binding
    n = 600_011
    x = _values(dt, n, 9, "sum")
    vec = 16 // np.dtype(dt).itemsize
    key = (torch.device(DEV).index, binding._stream(torch.device(DEV)))
    saved = binding.workspaces._ws.get(key)
    try:
        for off in (_poisson(n, 30_000.0, 6), _poisson(n, 3.0, 7), np.array([0, n], np.int32)):
            for tuning in ({"algo": "lookback", "mode_limit": 8},
                           {"algo": "lookback", "mode_limit": 8, "block_size": 256, "items_per_thread": vec}):
                ws = torch.zeros(1 << 24, dtype=torch.uint8, device=DEV)
                ws[128:132].view(torch.int32)[0] = -1  # first started-count slot
                binding.workspaces._ws[key] = ws
                for excl in (False, True):
                    _check(x, off, "sum", excl, tuning=tuning, what=f"{tuning} excl={excl}")
                    assert sw.scan_workspace_error(ws) == 4, tuning  # the dynamic path ran, no wait gave up
                    ws[128:132].view(torch.int32)[0] = -1  # the call reset it; force the fallback again
    finally:
        if saved is None:
            binding.workspaces._ws.pop(key, None)
        else:
            binding.workspaces._ws[key] = saved
