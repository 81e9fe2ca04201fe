"""GPU parity of the stable partition (and its one-bit radix digit pass)
against the oracle: bit-exact values, source indices and counts, at the
configuration size (n = 1e7, the compaction input) and on edge cases (one
element, all / none selected, alternating, exact ties, ragged ends, many
tiles, small grids, element-wide access for misaligned data, no index
output); a full LSD radix sort of 32-bit keys from 32 device passes; and a
workspace shared with scans of other sizes."""
import numpy as np
import pytest
import torch

import oracle
import stream_compaction_wave64_amd as sw
from stream_compaction_wave64_amd import inputs
from gpu_util import DEV, to_dev, to_host

pytestmark = pytest.mark.gpu


def _partition(x, cmp="gt", t=0.5, tuning=None, offset=0, with_idx=True):
    if offset:
        buf = to_dev(np.concatenate([np.zeros(offset, x.dtype), x]))
        xd = buf[offset:]
    else:
        xd = to_dev(x)
    out, idx, count = sw.partition_if(xd, cmp, t, with_idx=with_idx, tuning=tuning)
    torch.cuda.synchronize()
    n = x.size
    return to_host(out)[:n], (to_host(idx)[:n] if idx is not None else None), int(count.item())


def _check(x, cmp="gt", t=0.5, **kw):
    vals, idx, k = oracle.partition(x, cmp, t)
    got_v, got_i, got_k = _partition(x, cmp, t, **kw)
    assert got_k == k, (got_k, k)
    assert np.array_equal(got_v.view(np.uint32), vals.view(np.uint32))
    if got_i is not None:
        assert np.array_equal(got_i, idx)


def test_partition_config_1e7():
    x, _ = inputs.compaction_inputs(10 ** 7, seed=4)
    _check(x, "gt", 0.5)


@pytest.mark.parametrize("cmp", ["gt", "ge", "lt", "le", "eq", "ne"])
def test_partition_comparisons(cmp):
    rng = np.random.default_rng(50)
    x = rng.random(300_001, dtype=np.float32)
    x[::97] = np.float32(0.5)  # exact ties
    _check(x, cmp, 0.5)
    xi = rng.integers(-50, 51, 300_001, dtype=np.int32)
    _check(xi, cmp, 3)
    _check(xi, cmp, 3, tuning={"block_size": 256, "items_per_thread": 4})


@pytest.mark.parametrize("dt", [np.int32, np.uint32])
def test_partition_bit_digits(dt):
    rng = np.random.default_rng(51)
    keys = rng.integers(0, 2 ** 32, 200_003, dtype=np.uint64).astype(np.uint32).view(dt)
    for b in (0, 7, 31):
        _check(keys, "bit_clear", b)
        _check(keys, "bit_set", b)


def test_partition_edges_and_shapes():
    for n in (1, 3, 4, 5, 1000, 8448, 8449, 14336, 14337, 100_003):
        _check(np.ones(n, np.float32))                               # all selected: identity
        _check(np.zeros(n, np.float32))                              # none selected: identity
        _check(np.tile(np.array([0, 1], np.float32), n)[:n])         # odd indices first
    x, _ = inputs.compaction_inputs(500_003, seed=52)
    _check(x, offset=1)                                              # element-wide access
    _check(x, with_idx=False)
    for tuning in ({"block_size": 256, "items_per_thread": 4},
                   {"block_size": 256, "items_per_thread": 4, "grid_blocks": 3},
                   {"grid_blocks": 1}):
        _check(x, tuning=tuning)
    out, idx, count = sw.partition_if(torch.empty(0, dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    assert int(count.item()) == 0


def test_radix_sort_from_device_bit_passes():
    rng = np.random.default_rng(53)
    keys = rng.integers(0, 2 ** 32, 100_000, dtype=np.uint64).astype(np.uint32)
    keys[::5] = keys[11]
    cur = to_dev(keys)
    perm = torch.arange(keys.size, dtype=torch.int64, device=DEV)
    for b in range(32):
        cur, idx, _ = sw.partition_if(cur, "bit_clear", b)
        perm = perm[idx.long()]
    torch.cuda.synchronize()
    assert np.array_equal(to_host(cur), np.sort(keys))
    assert np.array_equal(perm.cpu().numpy(), np.argsort(keys, kind="stable"))


def test_partition_shares_workspace_with_scans():
    # the count pass's words sit above the tile descriptors within the
    # call's words; calls of other sizes on the same workspace must neither
    # see them nor leave stale words the partition could read
    x, _ = inputs.compaction_inputs(2_000_003, seed=54)
    small = x[:30_000]
    for _ in range(2):
        _check(x)
        s = sw.scan_inclusive(to_dev(small))
        torch.cuda.synchronize()
        assert np.allclose(to_host(s), np.cumsum(small.astype(np.float64)), rtol=1e-5, atol=1e-3)
        _check(small)
        big = sw.scan_inclusive(to_dev(x))
        torch.cuda.synchronize()
        assert abs(float(to_host(big)[-1]) - float(x.astype(np.float64).sum())) < 1e-3 * x.size
    ws = sw.workspaces.get(DEV, 1)
    assert sw.scan_workspace_error(ws) == 0


@pytest.mark.parametrize("shifts", [(1, 2), (3, 1), (2, 0)])
def test_partition_misaligned_outputs(shifts):
    # Values and indices go out as contiguous ranges cut at each output's own
    # 16-byte boundaries; outputs 1-3 elements off a boundary (and off each
    # other) exercise the partial quads.  Sentinels around both stay intact.
    sv, si = shifts
    x, _ = inputs.compaction_inputs(300_007, seed=53)
    vals, idx, k = oracle.partition(x, "gt", 0.5)
    n = x.size
    for tuning in (None, {"block_size": 256, "items_per_thread": 4}):
        vbuf = torch.full((n + 8,), -1.0, dtype=torch.float32, device=DEV)
        ibuf = torch.full((n + 8,), -7, dtype=torch.int32, device=DEV)
        _, _, count = sw.partition_if(to_dev(x), "gt", 0.5, out=vbuf[sv:sv + n], out_idx=ibuf[si:si + n],
                                      tuning=tuning)
        torch.cuda.synchronize()
        assert int(count.item()) == k
        gv, gi = to_host(vbuf), to_host(ibuf)
        assert np.array_equal(gv[sv:sv + n].view(np.uint32), vals.view(np.uint32))
        assert np.array_equal(gi[si:si + n], idx)
        assert (gv[:sv] == -1.0).all() and (gv[sv + n:] == -1.0).all()
        assert (gi[:si] == -7).all() and (gi[si + n:] == -7).all()


@pytest.mark.parametrize("cmp", ["gt", "eq", "ne"])
def test_partition_special_floats(cmp):
    # NaNs (with their bit patterns), signed zeros and infinities move as raw
    # 32-bit values; the predicate follows IEEE comparisons in fp32.
    rng = np.random.default_rng(54)
    x = rng.random(70_001, dtype=np.float32) - np.float32(0.5)
    specials = np.array([np.nan, -np.nan, np.inf, -np.inf, 0.0, -0.0], np.float32)
    x[rng.integers(0, x.size, 5000)] = specials[rng.integers(0, specials.size, 5000)]
    for t in (0.0, float("-inf")):
        _check(x, cmp, t)


def test_partition_resident():
    # x of whole 128-bit vectors that fits one register tile per compute unit
    # (at most 256 tiles of rows x 960 x 4 elements, rows <= 17) is
    # partitioned in one launch: both sides of the capacity, single-row and
    # ragged last tiles, comparisons, bit digits, closed forms, no index
    # output, misaligned outputs.
    cap = 256 * 17 * 3840
    assert sw.plan("partition", torch.float32, "sum", 1, 4096)["kernel"] == "partition_resident"
    assert sw.plan("partition", torch.float32, "sum", 1, cap)["kernel"] == "partition_resident"
    assert sw.plan("partition", torch.float32, "sum", 1, cap + 4)["kernel"] == "partition"
    assert sw.plan("partition", torch.float32, "sum", 1, 4097)["kernel"] == "partition"
    for n in (4096, 256 * 3840, 256 * 3840 + 4, cap, cap + 4):
        x, _ = inputs.compaction_inputs(n, seed=54)
        _check(x)
    rng = np.random.default_rng(55)
    n = 3 * 3840 * 200 + 44
    x = rng.random(n, dtype=np.float32)
    x[::97] = np.float32(0.5)
    for cmp in ("gt", "le", "eq", "ne"):
        _check(x, cmp, 0.5)
    _check(x, with_idx=False)
    keys = rng.integers(0, 2 ** 32, 7 * 3840 * 255 + 3840 + 12, dtype=np.uint64).astype(np.uint32)
    for dt in (np.int32, np.uint32):
        for b in (0, 31):
            _check(keys.view(dt), "bit_clear", b)
    for f in (np.ones(8192, np.float32), np.zeros(8192, np.float32), np.tile(np.array([0, 1], np.float32), 4096)):
        _check(f)
    x, _ = inputs.compaction_inputs(1_000_000, seed=56)
    vals, idx, k = oracle.partition(x, "gt", 0.5)
    vbuf = torch.full((x.size + 8,), -7, dtype=torch.int32, device=DEV)
    ibuf = torch.full((x.size + 8,), -7, dtype=torch.int32, device=DEV)
    _, _, count = sw.partition_if(to_dev(x), "gt", 0.5, out=vbuf[1:1 + x.size].view(torch.float32),
                                  out_idx=ibuf[3:3 + x.size])
    torch.cuda.synchronize()
    gv, gi = to_host(vbuf), to_host(ibuf)
    assert int(count.item()) == k
    assert np.array_equal(gv[1:1 + x.size].view(np.uint32), vals.view(np.uint32))
    assert np.array_equal(gi[3:3 + x.size], idx)
    assert (gv[:1] == -7).all() and (gv[1 + x.size:] == -7).all()
    assert (gi[:3] == -7).all() and (gi[3 + x.size:] == -7).all()
