"""GPU parity of scan_dim against the oracle's (outer, len, inner) scan:
rows of a matrix (segmented look-back), columns and other wide inner extents
(reduce-then-scan over row chunks), and the 2-D configurations at full size."""
import numpy as np
import pytest
import torch

import stream_compaction_wave64_amd as sw
from stream_compaction_wave64_amd import inputs
from gpu_util import DEV, TORCH, assert_scan_matches, to_dev, to_host

pytestmark = pytest.mark.gpu


def _dims(shape, dim):
    outer = int(np.prod(shape[:dim])) if dim else 1
    inner = int(np.prod(shape[dim + 1:])) if dim + 1 < len(shape) else 1
    return outer, shape[dim], inner


def _check(x, dim, op="sum", excl=False, offset=0):
    if offset:
        buf = to_dev(np.concatenate([np.zeros(offset, x.dtype), x.ravel()]))
        xd = buf[offset:].view(x.shape)
    else:
        xd = to_dev(x)
    r = sw.scan_dim(xd, dim, op=op, exclusive=excl)
    torch.cuda.synchronize()
    assert_scan_matches(x.ravel(), to_host(r).ravel(), op, excl, dims=_dims(x.shape, dim),
                        what=f"{x.shape} dim={dim} {op} excl={excl} off={offset}")


@pytest.mark.parametrize("dt", [np.float32, np.float64, np.int32, np.int64])
def test_rows_and_columns_small(dt):
    rng = np.random.default_rng(90)
    for shape in ((37, 53), (1, 1000), (1000, 1), (64, 4096), (300, 257), (5, 3, 700)):
        x = rng.integers(-9, 10, shape).astype(dt) if np.issubdtype(dt, np.integer) else \
            (2 * rng.random(shape) - 1).astype(dt)
        for dim in range(len(shape)):
            for excl in (False, True):
                _check(x, dim, "sum", excl)


@pytest.mark.parametrize("op", ["prod", "max", "min"])
def test_columns_other_ops(op):
    rng = np.random.default_rng(91)
    x = (1 + (rng.random((777, 1100)) - 0.5) * 0.002).astype(np.float32) if op == "prod" else \
        rng.random((777, 1100), dtype=np.float32)
    _check(x, 0, op)
    xi = rng.integers(-1000, 1000, (501, 333)).astype(np.int32)
    _check(xi, 0, op)


def test_wide_inner_misaligned_and_ragged():
    rng = np.random.default_rng(92)
    x = rng.random((2000, 1027), dtype=np.float32)  # inner not a multiple of 4
    _check(x, 0)
    y = rng.random((300, 1024), dtype=np.float32)
    _check(y, 0, offset=1)                           # element-wide column access
    z = rng.random((4, 100_000, 5), dtype=np.float32)  # unbuilt element width -> column kernel
    _check(z, 1)


@pytest.mark.parametrize("grid", [64, 300, 0])
def test_rows_many_tiles_per_row(grid):
    # rows of 131 one-row tiles: a workgroup's consecutive tiles cross row
    # (segment) boundaries; grids of 64 and 300 use the aggregate-only
    # look-back, the resident grid of one-row tiles (above 513) the windowed one
    rng = np.random.default_rng(93)
    tuning = {"block_size": 256, "items_per_thread": 4, "grid_blocks": grid}
    for dt in (np.float32, np.int32):
        x = rng.integers(-9, 10, (7, 100_000)).astype(dt) if dt == np.int32 else \
            (2 * rng.random((7, 100_000)) - 1).astype(dt)
        xd = to_dev(x)
        for excl in (False, True):
            r = sw.scan_dim(xd, 1, op="sum", exclusive=excl, tuning=tuning)
            torch.cuda.synchronize()
            assert_scan_matches(x.ravel(), to_host(r).ravel(), "sum", excl, dims=(7, 100_000, 1),
                                what=f"grid={grid} {np.dtype(dt).name} excl={excl}")


def test_configs_2d_full_size():
    square, tall, wide = inputs.dims_arrays(seed=3)
    _check(square, 1)   # 4096 x 4096 along rows
    _check(square, 0)   # 4096 x 4096 along columns
    _check(wide, 1)     # 2 x 1e7 along rows
    _check(tall, 0)     # 1e6 x 8 along the long axis


# The single pass for wide inner extents: register tiles of 256 rows x
# (64 x vec) columns, one per workgroup, each adding the column aggregates of
# the tiles above it.  Shapes: several row blocks and strips, ragged rows, a
# partial last strip, outer slices, the most row blocks per strip (64), and a
# strip just half full.
SINGLE_SHAPES = [(1, 4096, 4096), (1, 300, 1024), (3, 257, 520), (1, 16384, 256), (1, 1, 4096), (2, 513, 128)]
TORCH_DT = {np.float32: torch.float32, np.float64: torch.float64, np.int32: torch.int32, np.int64: torch.int64,
            np.uint32: torch.uint32}


def _single_input(dt, shape, seed, op):
    rng = np.random.default_rng(seed)
    if np.issubdtype(dt, np.integer):
        return rng.integers(-1000, 1000, shape).astype(dt) if dt != np.uint32 else \
            rng.integers(0, 2000, shape).astype(dt)
    if op == "prod":
        return (1 + (rng.random(shape) - 0.5) * 0.002).astype(dt)
    return (2 * rng.random(shape) - 1).astype(dt)


@pytest.mark.parametrize("dt", [np.float32, np.float64, np.int32, np.uint32, np.int64], ids=lambda d: np.dtype(d).name)
@pytest.mark.parametrize("op", ["sum", "prod", "max", "min"])
def test_columns_single_pass(dt, op):
    vec = 16 // np.dtype(dt).itemsize
    for i, (outer, length, inner) in enumerate(SINGLE_SHAPES):
        if 2 * inner < 64 * vec:
            continue
        if op != "sum" and length * inner > 2 ** 22:
            continue
        p = sw.plan("scan", TORCH_DT[dt], op, outer, length, inner)
        tiles = outer * -(-inner // (64 * vec)) * -(-length // 256)
        # more tiles than compute units: the three-launch path
        want = ("columns_lookback", 1) if tiles <= 256 else ("columns", 3)
        assert (p["kernel"], p["launches"]) == want, (outer, length, inner, p)
        x = _single_input(dt, (outer, length, inner), 95 + i, op)
        for excl in (False, True):
            _check(x, 1, op, excl)


def test_columns_single_pass_dynamic_claiming():
    # a start count that never confirms residency: tiles are claimed in order
    # (error word bit 2), results still exact
    from stream_compaction_wave64_amd import binding
    x = _single_input(np.int32, (1, 4096, 4096), 99, "sum")
    xd = to_dev(x)
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    key = (torch.device(DEV).index, binding._stream(torch.device(DEV)))
    saved = binding.workspaces._ws.get(key)
    binding.workspaces._ws[key] = ws
    try:
        for excl in (False, True):
            ws[128:132].view(torch.int32)[0] = -1
            r = sw.scan_dim(xd, 1, exclusive=excl, tuning={"mode_limit": 8})
            torch.cuda.synchronize()
            assert sw.scan_workspace_error(ws) == 4
            assert_scan_matches(x.ravel(), to_host(r).ravel(), "sum", excl, dims=(1, 4096, 4096),
                                what=f"dynamic excl={excl}")
            sw.scan_workspace_init(ws)
        r = sw.scan_dim(xd, 1)
        torch.cuda.synchronize()
        assert sw.scan_workspace_error(ws) == 0
        assert_scan_matches(x.ravel(), to_host(r).ravel(), "sum", False, dims=(1, 4096, 4096))
    finally:
        if saved is None:
            binding.workspaces._ws.pop(key, None)
        else:
            binding.workspaces._ws[key] = saved


def test_columns_reduce_then_scan_on_request():
    # the three-launch path stays available (algo reduce-then-scan) for the
    # shapes the single pass takes
    x = _single_input(np.float32, (1, 4096, 4096), 98, "sum")
    p = sw.plan("scan", torch.float32, "sum", 1, 4096, 4096, tuning={"algo": "reduce_then_scan"})
    assert p["kernel"] == "columns" and p["launches"] == 3
    r = sw.scan_dim(to_dev(x), 1, tuning={"algo": "reduce_then_scan"})
    torch.cuda.synchronize()
    assert_scan_matches(x.ravel(), to_host(r).ravel(), "sum", False, dims=(1, 4096, 4096))


@pytest.mark.parametrize("dt", [np.float32, np.float64, np.int32, np.uint32, np.int64], ids=lambda d: np.dtype(d).name)
@pytest.mark.parametrize("op", ["sum", "prod", "max", "min"])
def test_rows_kernel_one_workgroup_per_row(dt, op):
    # Rows that each fit one tile of the rows kernel (256 threads x 1, 2, 4 or
    # 8 rows of 128-bit vectors): every tile-row count at a full tile and just
    # past the previous one (a ragged end inside a tile row), the shortest row
    # it takes (one wave's vectors), inclusive and exclusive, in place, and a
    # 3-D array scanned along its last axis.
    vec = 16 // np.dtype(dt).itemsize
    rng = np.random.default_rng(91)
    lengths = [64 * vec, 256 * vec - vec, 256 * vec, 256 * vec + vec, 512 * vec, 1024 * vec - vec, 1024 * vec,
               1024 * vec + vec, 2048 * vec]
    for i, length in enumerate(lengths):
        rows = 37 if length > 1024 * vec else 301
        assert sw.plan("scan", TORCH[np.dtype(dt)], op, rows, length)["kernel"] == "rows"
        if op == "prod" and np.issubdtype(dt, np.floating):
            x = (1.0 + (rng.random((rows, length)) - 0.5) * 0.002).astype(dt)
        elif np.issubdtype(dt, np.floating):
            x = (2 * rng.random((rows, length)) - 1).astype(dt)
        else:
            x = rng.integers(-9 if dt != np.uint32 else 0, 10, (rows, length)).astype(dt)
        for excl in (False, True):
            _check(x, 1, op, excl)
    # in place: each row is read whole before any of it is written
    x = inputs.generic(dt, 129 * 1024, 92, "wide" if np.issubdtype(dt, np.integer) else "default")
    x = x.reshape(129, 1024)
    xd = to_dev(x)
    sw.scan_dim(xd, 1, op=op, out=xd)
    torch.cuda.synchronize()
    assert_scan_matches(x.ravel(), to_host(xd).ravel(), op, False, dims=(129, 1024, 1), what="in place")
    x3 = x.reshape(3, 43, 1024)
    _check(x3, 2, op, False)
    # thousands of workgroups
    x = inputs.generic(dt, 2049 * 64 * vec, 93, "wide" if np.issubdtype(dt, np.integer) else "default")
    _check(x.reshape(2049, 64 * vec), 1, op, op == "max")

