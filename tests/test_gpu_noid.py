"""GPU parity of the inclusive scan that never uses the operator's identity
(AcceleratedKernels.jl PR #208, description, first bullet: Optional partials
for operators with no neutral element; its timing table's "no neutral"
cumsum row), against the oracle's scan_noid.

Sizes span one partial tile, tile boundaries, several tiles with a ragged
tail and many tiles; every dtype x op; the default, small-array, short-row
and one-row tile shapes of the look-back pipeline, and the resident single
pass (arrays of 8 MiB and more that fit one register tile per compute unit,
the fp32 1e7 config among them); misaligned (element-wide) data; rows of 2-D
arrays; small persistent grids.  Negative zeros tell the two
paths apart: -0.0 + -0.0 = -0.0 but 0.0 + -0.0 = +0.0, so a sum of negative
zeros stays -0.0 everywhere only if no identity enters any partial result
(thread, wave, workgroup, look-back carry)."""
import numpy as np
import pytest
import torch

import stream_compaction_wave64_amd as sw
from stream_compaction_wave64_amd import inputs
from gpu_util import DEV, TORCH, assert_scan_matches, to_dev, to_host

pytestmark = pytest.mark.gpu

DTYPES = [np.int32, np.uint32, np.int64, np.float32, np.float64]
OPS = ["sum", "prod", "max", "min"]
NOID = {"no_identity": 1}


def _input(dt, n, seed, op):
    kind = "near1" if op == "prod" and np.issubdtype(dt, np.floating) else "wide"
    if op == "sum" and np.issubdtype(dt, np.floating):
        kind = "default"
    return inputs.generic(dt, n, seed, kind)


def _run(x, op, tuning=None, offset=0):
    t = dict(NOID, **(tuning or {}))
    if offset:
        buf = to_dev(np.concatenate([np.zeros(offset, x.dtype), x]))
        xd = buf[offset:]
        out = torch.empty(x.size + offset, dtype=xd.dtype, device=DEV)[offset:]
    else:
        xd, out = to_dev(x), None
    res = sw.scan_inclusive(xd, op=op, out=out, tuning=t)
    torch.cuda.synchronize()
    return to_host(res)


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: np.dtype(d).name)
@pytest.mark.parametrize("op", OPS)
def test_noid_parity_planner_shapes(dt, op):
    # sizes around the small-array look-back tiles (448 x 5 rows), with the
    # planner's choice and with that shape pinned (the pipeline)
    vec = 16 // np.dtype(dt).itemsize
    small = {"block_size": 512, "items_per_thread": 5 * vec}
    p = sw.plan("scan", TORCH[np.dtype(dt)], op, 1, 10 ** 6, tuning=dict(NOID, **small))
    assert p["kernel"] == "lookback"
    tile = p["tile_elems"]
    edge = 256 * tile  # the planner's last size for that shape under a grid cap
    for i, n in enumerate([1, 2, 3, 63, 64, 65, 1000, tile - 4, tile, tile + 4, 3 * tile + 12, 65 * tile + 4,
                           edge, edge + vec]):
        x = _input(dt, n, 700 + i, op)
        assert_scan_matches(x, _run(x, op), op, False, what=f"n={n}", noid=True)
        if n <= edge:
            assert_scan_matches(x, _run(x, op, small), op, False, what=f"n={n} small tiles", noid=True)


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: np.dtype(d).name)
@pytest.mark.parametrize("op", OPS)
def test_noid_parity_default_shape_and_small_tiles(dt, op):
    # the pipeline's default shape (1e8 elements exceed the resident pass)
    big = sw.plan("scan", TORCH[np.dtype(dt)], op, 1, 10 ** 8, tuning=NOID)
    assert big["kernel"] == "lookback"
    default = {"block_size": big["block_size"], "items_per_thread": big["items_per_thread"]}
    tile = big["tile_elems"]
    for i, n in enumerate([tile - 4, tile + 4, 40 * tile + 8]):
        x = _input(dt, n, 800 + i, op)
        assert_scan_matches(x, _run(x, op, default), op, False, what=f"default n={n}", noid=True)
    # one row per tile: hundreds of tiles, the windowed look-back of large grids
    vec = 16 // np.dtype(dt).itemsize
    small = {"block_size": 256, "items_per_thread": vec}
    for i, n in enumerate([100_000, 256 * vec * 70 + 8]):
        x = _input(dt, n, 900 + i, op)
        assert_scan_matches(x, _run(x, op, small), op, False, what=f"small tiles n={n}", noid=True)


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: np.dtype(d).name)
@pytest.mark.parametrize("grid", [1, 3, 64])
def test_noid_small_persistent_grid(dt, grid):
    vec = 16 // np.dtype(dt).itemsize
    tuning = {"block_size": 256, "items_per_thread": vec, "grid_blocks": grid}
    for n, seed in ((256 * vec * 37 + 4 * vec, 3), (5 * vec, 5)):
        x = _input(dt, n, seed, "sum")
        assert_scan_matches(x, _run(x, "sum", tuning), "sum", False, what=f"n={n}", noid=True)


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: np.dtype(d).name)
def test_noid_misaligned_element_wide(dt):
    for op in OPS:
        for n in (1, 77, 100_003):
            x = _input(dt, n, 1000 + n, op)
            assert_scan_matches(x, _run(x, op, offset=1), op, False, what=f"{op} n={n}", noid=True)


@pytest.mark.parametrize("dt", [np.float32, np.float64])
def test_noid_negative_zeros_stay_negative(dt):
    # every partial result a workgroup, wave, thread or look-back carry forms
    # is a sum of -0.0 values: each output must be -0.0, sign bit set.  The
    # identity path turns them into +0.0 (0.0 + -0.0 = +0.0).
    vec = 16 // np.dtype(dt).itemsize
    tile = sw.plan("scan", TORCH[np.dtype(dt)], "sum", 1, 10 ** 7, tuning=NOID)["tile_elems"]
    cases = [(5 * tile + 3, None), (3_000_001, None), (200_003, {"block_size": 256, "items_per_thread": vec}),
             (100_001, {"block_size": 256, "items_per_thread": vec, "grid_blocks": 2})]
    for n, tuning in cases:
        z = np.full(n, -0.0, dtype=dt)
        got = _run(z, "sum", tuning)
        assert np.all(got == 0) and np.all(np.signbit(got)), f"n={n} tuning={tuning}: a +0.0 appeared"
        ident = sw.scan_inclusive(to_dev(z), tuning=tuning)
        torch.cuda.synchronize()
        assert not np.any(np.signbit(to_host(ident))), "the identity path keeps -0.0?"
    # misaligned (element-wide) too, and a first element of -0.0 before other values
    z = np.full(70_001, -0.0, dtype=dt)
    assert np.all(np.signbit(_run(z, "sum", offset=1)))
    x = inputs.generic(dt, 50_000, 11)
    x[0] = -0.0
    got = _run(x, "sum")
    assert np.signbit(got[0]) and got[0] == 0
    assert_scan_matches(x, got, "sum", False, noid=True)


@pytest.mark.parametrize("dt", [np.int32, np.float32, np.float64])
def test_noid_rows(dt):
    # rows of 2-D arrays: short rows (one tile each, several shapes) and rows
    # of several tiles; each row starts from its own first element
    for shape in ((300, 17), (64, 4096), (3, 200_003), (2, 2_000_000)):
        x = inputs.generic(dt, shape[0] * shape[1], sum(shape), "default").reshape(shape)
        res = sw.scan_dim(to_dev(x), dim=1, tuning=NOID)
        torch.cuda.synchronize()
        assert_scan_matches(x, to_host(res), "sum", False, dims=(shape[0], shape[1], 1), what=f"{shape}",
                            noid=True)
    if np.issubdtype(dt, np.floating):
        z = np.full((5, 100_000), -0.0, dtype=dt)
        res = to_host(sw.scan_dim(to_dev(z), dim=1, tuning=NOID))
        assert np.all(np.signbit(res))


def test_noid_fp32_1e7_config():
    # the pages' "cumsum F32 1e7, no neutral" row, on the seeded uniform [0,1)
    assert sw.plan("scan", torch.float32, "sum", 1, 10 ** 7, tuning=NOID)["kernel"] == "resident"
    x = inputs.f32_uniform_01(10 ** 7, seed=1)
    got = _run(x, "sum")
    assert_scan_matches(x, got, "sum", False, what="fp32 1e7 no neutral", noid=True)


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: np.dtype(d).name)
@pytest.mark.parametrize("op", OPS)
def test_noid_resident_pass(dt, op):
    # The resident single pass without an identity: from 8 MiB to its
    # capacity (256 tiles of 17 rows of 960 x 4 elements, or
    # 21 rows of 960 x 2), tile ends ragged inside a row; rows of 2-D arrays,
    # several tiles per row and one tile per row (no row has a prefix).
    isz = np.dtype(dt).itemsize
    vec = 16 // isz
    cap = 256 * (17 if vec == 4 else 21) * 960 * vec
    sizes = [(8 << 20) // isz, 3_000_000 + 4 * vec]
    if op == "sum":
        sizes += [cap - 7 * vec, cap]
    for i, n in enumerate(sizes):
        assert sw.plan("scan", TORCH[np.dtype(dt)], op, 1, n, tuning=NOID)["kernel"] == "resident", n
        x = _input(dt, n, 1100 + i, op)
        assert_scan_matches(x, _run(x, op), op, False, what=f"n={n}", noid=True)
    for shape in ((3, 1_000_000 + 4 * vec), (200, 10_500 * 4 // vec)):
        assert sw.plan("scan", TORCH[np.dtype(dt)], op, shape[0], shape[1], tuning=NOID)["kernel"] == "resident"
        x = _input(dt, shape[0] * shape[1], sum(shape), op).reshape(shape)
        res = sw.scan_dim(to_dev(x), dim=1, op=op, tuning=NOID)
        torch.cuda.synchronize()
        assert_scan_matches(x, to_host(res), op, False, dims=(shape[0], shape[1], 1), what=f"{shape}", noid=True)
    if op == "sum" and np.issubdtype(dt, np.floating):
        # no identity enters any partial result: -0.0 everywhere stays -0.0
        for shape in ((1, 3_000_000 + 4 * vec), (200, 10_500 * 4 // vec)):
            z = np.full(shape, -0.0, dtype=dt)
            res = to_host(sw.scan_dim(to_dev(z), dim=1, tuning=NOID))
            assert np.all(res == 0) and np.all(np.signbit(res)), f"{shape}: a +0.0 appeared"


def test_noid_unsupported_forms():
    x = to_dev(inputs.generic(np.float32, 1000, 1))
    for fn in (lambda: sw.scan_exclusive(x, tuning=NOID),
               lambda: sw.scan_inclusive(x, tuning=dict(NOID, algo="reduce_then_scan")),
               lambda: sw.scan_inclusive(x, width=4, tuning=NOID),
               lambda: sw.compact_if(x, "gt", 0.5, tuning=NOID)):
        with pytest.raises(sw.ScanError) as e:
            fn()
        assert e.value.status == -2
