"""GPU parity of large-element scans (structs of W components, combined
component-wise) and of scan_dim with a small inner extent, against the
oracle's (outer, len, inner) scan."""
import numpy as np
import pytest
import torch

import stream_compaction_wave64_amd as sw
from stream_compaction_wave64_amd import inputs
from gpu_util import DEV, assert_scan_matches, to_dev, to_host

pytestmark = pytest.mark.gpu

WIDTHS = [2, 3, 4, 8, 16, 17, 24]


def _struct_input(dt, n, w, seed, op):
    rng = np.random.default_rng(seed)
    if np.issubdtype(dt, np.floating):
        if op == "prod":
            return (1.0 + (rng.random((n, w)) - 0.5) * 0.002).astype(dt)
        return (2 * rng.random((n, w)) - 1).astype(dt)
    return rng.integers(-1000, 1001, (n, w)).astype(dt)


@pytest.mark.parametrize("w", WIDTHS)
@pytest.mark.parametrize("dt", [np.float32, np.float64, np.int32], ids=["f32", "f64", "i32"])
def test_struct_scan_parity(w, dt):
    for n, tuning in ((1, None), (65, None), (1000, None), (100_003, None),
                      (20_001, {"block_size": 64}), (20_001, {"block_size": 64, "grid_blocks": 3})):
        x = _struct_input(dt, n, w, 70 + w, "sum")
        for excl in (False, True):
            fn = sw.scan_exclusive if excl else sw.scan_inclusive
            r = fn(to_dev(x), width=w, tuning=tuning)
            torch.cuda.synchronize()
            assert_scan_matches(x.ravel(), to_host(r).ravel(), "sum", excl, dims=(1, n, w),
                                what=f"n={n} w={w} {tuning} excl={excl}")


@pytest.mark.parametrize("op", ["prod", "max", "min"])
@pytest.mark.parametrize("w", [3, 17, 24])
def test_struct_scan_other_ops(op, w):
    for dt in (np.float32, np.float64, np.int32):
        x = _struct_input(dt, 30_007, w, 80, op)
        r = sw.scan_inclusive(to_dev(x), op=op, width=w, tuning={"block_size": 64})
        torch.cuda.synchronize()
        assert_scan_matches(x.ravel(), to_host(r).ravel(), op, False, dims=(1, x.shape[0], w), what=f"{dt} {op}")


@pytest.mark.parametrize("w,dt,n", [(24, np.float32, 600_001), (17, np.float64, 300_001), (8, np.int32, 300_001)])
def test_struct_scan_many_chunks(w, dt, n):
    # more than 2048 chunks: the partials pass runs several chunks per thread
    # of its 1024; and a single chunk holding every tile
    x = _struct_input(dt, n, w, 90 + w, "sum")
    for tuning in ({"rts_blocks": 8192, "block_size": 64}, {"rts_blocks": 1, "block_size": 64}):
        for excl in (False, True):
            fn = sw.scan_exclusive if excl else sw.scan_inclusive
            r = fn(to_dev(x), width=w, tuning=tuning)
            torch.cuda.synchronize()
            assert_scan_matches(x.ravel(), to_host(r).ravel(), "sum", excl, dims=(1, n, w),
                                what=f"w={w} {tuning} excl={excl}")
    # segments (outer > 1) each get their own run of chunks
    xs = x[: (n // 3) * 3].reshape(3, n // 3, w)
    r = sw.scan_dim(to_dev(xs), 1, tuning={"rts_blocks": 8192, "block_size": 64})
    torch.cuda.synchronize()
    assert_scan_matches(xs.ravel(), to_host(r).ravel(), "sum", False, dims=xs.shape, what="3 segments")


def test_dim_small_inner_segments():
    # (outer, len, inner) with outer > 1: each outer slice scanned independently
    rng = np.random.default_rng(81)
    for shape, dim in (((5, 7001, 8), 1), ((3, 40_000, 4), 1), ((2, 5, 3), 1), ((7, 1, 8), 1)):
        x = rng.random(shape, dtype=np.float32)
        r = sw.scan_dim(to_dev(x), dim)
        torch.cuda.synchronize()
        assert_scan_matches(x.ravel(), to_host(r).ravel(), "sum", False, dims=shape, what=str(shape))
        r = sw.scan_dim(to_dev(x), dim, exclusive=True)
        torch.cuda.synchronize()
        assert_scan_matches(x.ravel(), to_host(r).ravel(), "sum", True, dims=shape, what=str(shape))


def test_config_1e6x8_along_long_axis():
    _, tall, _ = inputs.dims_arrays(seed=3)
    r = sw.scan_dim(to_dev(tall), 0)
    torch.cuda.synchronize()
    assert_scan_matches(tall.ravel(), to_host(r).ravel(), "sum", False, dims=(1, 10 ** 6, 8), what="1e6x8 dim 0")


def test_config_structs_136B_and_96B():
    s64, s32 = inputs.struct_inputs(seed=5)
    r = sw.scan_inclusive(to_dev(s64), width=17)
    torch.cuda.synchronize()
    assert_scan_matches(s64.ravel(), to_host(r).ravel(), "sum", False, dims=(1, 10 ** 6, 17), what="17 x fp64")
    r = sw.scan_inclusive(to_dev(s32), width=24)
    torch.cuda.synchronize()
    assert_scan_matches(s32.ravel(), to_host(r).ravel(), "sum", False, dims=(1, 10 ** 6, 24), what="24 x fp32")


def test_misaligned_struct_rows_use_element_wide_access():
    x = _struct_input(np.float32, 10_001, 8, 82, "sum")
    buf = to_dev(np.concatenate([np.zeros(1, np.float32), x.ravel()]))
    xd = buf[1:]
    r = sw.scan_inclusive(xd, width=8)
    torch.cuda.synchronize()
    assert_scan_matches(x.ravel(), to_host(r).ravel(), "sum", False, dims=(1, 10_001, 8))


def test_element_calls_leave_workspace_untagged():
    # The element partials share the workspace's descriptor area: after
    # element scans of every carry width and operator (and exclusive scans,
    # and segments), a look-back scan on the same workspace must see no
    # leftover word that reads as published.
    follow = inputs.generic(np.int32, 2_000_003, 83, "wide")
    fd = to_dev(follow)
    cases = [(np.float32, 8, 1_000_003, "sum", False), (np.float64, 4, 700_001, "sum", True),
             (np.int64, 4, 300_007, "max", True), (np.int32, 8, 500_001, "min", False),
             (np.float32, 8, 500_003, "prod", False), (np.float32, 3, 400_009, "sum", True),
             (np.float64, 17, 100_003, "sum", False)]
    for dt, w, n, op, excl in cases:
        x = _struct_input(dt, n, w, 84 + w, op)
        fn = sw.scan_exclusive if excl else sw.scan_inclusive
        r = fn(to_dev(x), op=op, width=w)
        torch.cuda.synchronize()
        assert_scan_matches(x.ravel(), to_host(r).ravel(), op, excl, dims=(1, n, w), what=f"{dt} w={w} n={n} {op}")
        f = sw.scan_inclusive(fd)
        torch.cuda.synchronize()
        assert_scan_matches(follow, to_host(f), "sum", False, what=f"look-back after {dt} w={w} n={n}")
    xs = _struct_input(np.float32, 4 * 250_000, 4, 85, "sum").reshape(4, 250_000, 4)
    r = sw.scan_dim(to_dev(xs), 1)
    torch.cuda.synchronize()
    assert_scan_matches(xs.ravel(), to_host(r).ravel(), "sum", False, dims=xs.shape, what="4 segments")
    f = sw.scan_inclusive(fd)
    torch.cuda.synchronize()
    assert_scan_matches(follow, to_host(f), "sum", False, what="look-back after segments")
