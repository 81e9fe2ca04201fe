"""GPU parity of scan_dim against the oracle's (outer, len, inner) scan:
rows of a matrix (segmented look-back), columns and other wide inner extents
(reduce-then-scan over row chunks), and the 2-D configurations at full size."""
import numpy as np
import pytest
import torch

import stream_compaction_wave64_amd as sw
from stream_compaction_wave64_amd import inputs
from gpu_util import DEV, assert_scan_matches, to_dev, to_host

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
