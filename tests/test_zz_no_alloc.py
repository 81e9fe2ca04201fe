"""scan_inclusive_noalloc, the entry point for callers that cannot allocate:
called through the C ABI, two calls in a row (the second smaller), its
output compared with scan_inclusive's on the same input and with the oracle.
Integer sums and max/min must match scan_inclusive bit for bit; fp sums may
associate differently from run to run (the look-back combines predecessors'
aggregates in arrival order), so both results must meet the oracle's
tolerance and differ from each other by at most twice it."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import stream_compaction_wave64_amd as sw
from stream_compaction_wave64_amd import binding, inputs
from gpu_util import DEV, F32_ABS, F32_REL, F64_REL, assert_scan_matches, to_dev, to_host

pytestmark = pytest.mark.gpu

DT = {np.int32: 0, np.uint32: 1, np.int64: 2, np.float32: 3, np.float64: 4}
OPS = {"sum": 0, "prod": 1, "max": 2, "min": 3}


def _noalloc(x: np.ndarray, op: str, width: int = 1) -> np.ndarray:
    lib = binding.load_library()
    xd = to_dev(x)
    out = torch.empty_like(xd)
    n = x.size // width
    rc = lib.scan_inclusive_noalloc(xd.data_ptr(), out.data_ptr(), n, DT[x.dtype.type], OPS[op], width, None,
                                    binding._stream(torch.device(DEV)))
    assert rc == 0, lib.scan_status_string(rc).decode()
    torch.cuda.synchronize()
    return to_host(out)


def _with_workspace(x: np.ndarray, op: str, width: int = 1) -> np.ndarray:
    r = sw.scan_inclusive(to_dev(x), op=op, width=width)
    torch.cuda.synchronize()
    return to_host(r)


def _same_result(x: np.ndarray, a: np.ndarray, b: np.ndarray, op: str, dims=None, what=""):
    """a and b are both correct results for x: identical for integers and
    max/min, within twice the fp sum tolerance of each other otherwise."""
    if np.issubdtype(x.dtype, np.integer) or op in ("max", "min"):
        assert np.array_equal(a, b), f"{what}: differs from scan_inclusive"
        return
    assert op == "sum"
    p = oracle.abs_prefix(x, dims=dims).ravel()
    tol = F32_REL * p + F32_ABS if x.dtype == np.float32 else F64_REL * p
    d = np.abs(a.astype(np.float64).ravel() - b.astype(np.float64).ravel())
    assert np.all(d <= 2 * tol), f"{what}: {np.count_nonzero(d > 2 * tol)} outside twice the tolerance"


@pytest.mark.parametrize("dt,op", [(np.int32, "sum"), (np.uint32, "max"), (np.int64, "sum"), (np.float32, "sum"),
                                   (np.float64, "sum"), (np.float32, "min")])
def test_noalloc_matches_scan_inclusive_two_calls(dt, op):
    kind = "default" if np.issubdtype(dt, np.floating) and op == "sum" else "wide"
    for i, n in enumerate([3_000_007 if np.dtype(dt).itemsize == 4 else 1_500_003, 100_003]):
        x = inputs.generic(dt, n, 500 + i, kind)
        got = _noalloc(x, op)
        assert_scan_matches(x, got, op, False, what=f"noalloc n={n}")
        _same_result(x, got, _with_workspace(x, op), op, what=f"n={n}")


def test_noalloc_metric_size_then_small():
    x = inputs.f32_uniform_01(10 ** 8, seed=1)
    # the metric's size, checked against scan_inclusive's result everywhere
    # and against the oracle on samples plus the ends
    got = _noalloc(x, "sum")
    _same_result(x, got, _with_workspace(x, "sum"), "sum", what="1e8")
    ref = oracle.scan(x, "sum")
    p = oracle.abs_prefix(x)
    idx = np.r_[0:1000, 10 ** 8 - 1000:10 ** 8, np.random.default_rng(3).integers(0, 10 ** 8, 2000)]
    assert np.all(np.abs(got[idx].astype(np.float64) - ref[idx]) <= F32_REL * p[idx] + F32_ABS)
    y = inputs.generic(np.float32, 777, 9)
    got = _noalloc(y, "sum")
    assert_scan_matches(y, got, "sum", False, what="small after large")
    _same_result(y, got, _with_workspace(y, "sum"), "sum", what="small after large")


def test_noalloc_struct_elements():
    # 17-component fp64 elements take the element kernel, its partials in the array
    for i, n in enumerate([20_011, 3_001]):
        x = inputs.generic(np.float64, n * 17, 600 + i)
        got = _noalloc(x, "sum", width=17)
        assert_scan_matches(x.reshape(n, 17), got.reshape(n, 17), "sum", False, dims=(1, n, 17),
                            what=f"struct n={n}")
        _same_result(x, got, _with_workspace(x, "sum", width=17), "sum", dims=(1, n, 17), what=f"struct n={n}")


@pytest.mark.parametrize("dt,op", [(np.int32, "sum"), (np.float64, "sum"), (np.float32, "max")])
def test_noalloc_two_tile_resident_then_smaller(dt, op):
    # whole arrays of 40 MiB or more take the resident pass with two tiles per
    # workgroup; then a one-tile resident call on the same scratch array
    es = np.dtype(dt).itemsize
    kind = "default" if np.issubdtype(dt, np.floating) and op == "sum" else "wide"
    big = (40 << 20) // es + 16 // es
    assert sw.plan("scan", torch.int32 if es == 4 else torch.float64, "sum", 1, big)["tiles_per_block"] == 2
    for i, n in enumerate([big, (12 << 20) // es]):
        x = inputs.generic(dt, n, 520 + i, kind)
        got = _noalloc(x, op)
        assert_scan_matches(x, got, op, False, what=f"noalloc n={n}")
        _same_result(x, got, _with_workspace(x, op), op, what=f"n={n}")
