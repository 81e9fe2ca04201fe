"""GPU parity of stream compaction and count-scan-emit packing against the
oracle: bit-exact indices, counts, offsets, totals and emitted records, at the
configuration sizes (n = 1e7) and on edge cases (empty, all/none selected,
alternating, ties at the threshold, ragged and misaligned inputs, many tiles,
zero and huge counts)."""
import numpy as np
import pytest
import torch

import oracle
import stream_compaction_wave64_amd as sw
from stream_compaction_wave64_amd import inputs
from gpu_util import DEV, to_dev, to_host

pytestmark = pytest.mark.gpu

CMPS = ["gt", "ge", "lt", "le", "eq", "ne"]


def _compact(x, cmp="gt", t=0.5, tuning=None, offset=0):
    if offset:
        buf = to_dev(np.concatenate([np.zeros(offset, x.dtype), x]))
        xd = buf[offset:]
    else:
        xd = to_dev(x)
    out, count = sw.compact_if(xd, cmp, t, tuning=tuning)
    torch.cuda.synchronize()
    c = int(count.item())
    return to_host(out[:c]) if c else np.zeros(0, np.int32), c


def _check_compact(x, cmp="gt", t=0.5, **kw):
    ref = oracle.compact(x, cmp, t)
    got, c = _compact(x, cmp, t, **kw)
    assert c == ref.size, (c, ref.size)
    assert np.array_equal(got, ref)


def test_compaction_config_1e7():
    x, _ = inputs.compaction_inputs(10 ** 7, seed=4)
    _check_compact(x, "gt", 0.5)


@pytest.mark.parametrize("cmp", CMPS)
@pytest.mark.parametrize("dt", [np.float32, np.int32])
def test_compaction_all_comparisons(cmp, dt):
    rng = np.random.default_rng(40)
    if dt == np.float32:
        x = rng.random(300_001, dtype=np.float32)
        x[::97] = np.float32(0.5)  # exact ties
        t = 0.5
    else:
        x = rng.integers(-50, 51, 300_001, dtype=np.int32)
        t = 3
    _check_compact(x, cmp, t)
    _check_compact(x, cmp, t, tuning={"block_size": 256, "items_per_thread": 4})


@pytest.mark.parametrize("dt", [np.int32, np.uint32])
def test_compaction_integer_keys_and_bit_predicates(dt):
    rng = np.random.default_rng(41)
    keys = rng.integers(0, 2 ** 32, 300_001, dtype=np.uint64).astype(np.uint32).view(dt)
    for b in (0, 9, 31):
        _check_compact(keys, "bit_clear", b)
        _check_compact(keys, "bit_set", b)
    _check_compact(keys, "gt", 2 ** 31 if dt == np.uint32 else 0)
    _check_compact(keys, "le", 12345, tuning={"block_size": 256, "items_per_thread": 4})


def test_compaction_closed_forms_and_edges():
    for n in (1, 3, 4, 5, 1000, 14080, 14081, 16384, 16385, 100_003):
        _check_compact(np.ones(n, np.float32))                      # all selected -> iota
        _check_compact(np.zeros(n, np.float32))                     # none selected
        _check_compact(np.tile(np.array([0, 1], np.float32), n)[:n])  # alternating -> 2k+1
    out, count = sw.compact_if(torch.empty(0, dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    assert int(count.item()) == 0


def test_compaction_ragged_misaligned_many_tiles():
    x, _ = inputs.compaction_inputs(500_003, seed=41)
    for tuning in (None, {"block_size": 256, "items_per_thread": 4},
                   {"block_size": 256, "items_per_thread": 4, "grid_blocks": 3}):
        _check_compact(x, tuning=tuning)
        _check_compact(x, tuning=tuning, offset=1)  # element-wide loads


def test_pack_config_1e7_offsets_and_emit():
    _, counts = inputs.compaction_inputs(10 ** 7, seed=4)
    ref_off, ref_total = oracle.pack_offsets(counts)
    off = sw.pack_offsets(to_dev(counts))
    torch.cuda.synchronize()
    got_off = to_host(off)
    assert np.array_equal(got_off, ref_off)
    total = int(got_off[-1])
    assert total == ref_total
    rec = sw.pack_emit_neighbors(off, total)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(rec)[:total], oracle.pack_emit(ref_off))


def test_emit_windows_wrap_and_alignment():
    # records staged through LDS windows of 4096: one object far longer than
    # a window, workgroups whose 1024 objects need several windows, counts
    # that wrap the record value past 2n, object counts that are not a
    # multiple of 1024; and outputs starting 1..3 elements past 16-byte
    # alignment, with guard values on both sides that must survive
    rng = np.random.default_rng(44)
    cases = [np.array([0, 10_000, 3, 0, 7], np.int32),
             np.full(3000, 20, np.int32),
             np.array([5, 7, 2], np.int32),
             rng.integers(0, 9, 1025).astype(np.int32),
             rng.integers(0, 40, 5000).astype(np.int32)]
    for counts in cases:
        ref_off, total = oracle.pack_offsets(counts)
        want = oracle.pack_emit(ref_off)
        off = to_dev(ref_off.astype(np.int32))
        for shift in (0, 1, 2, 3):
            buf = torch.full((total + 8,), -5, dtype=torch.int32, device=DEV)
            sw.pack_emit_neighbors(off, total, out=buf[shift:shift + total])
            torch.cuda.synchronize()
            got = to_host(buf)
            assert np.array_equal(got[shift:shift + total], want), (counts.size, shift)
            assert (got[:shift] == -5).all() and (got[shift + total:] == -5).all(), (counts.size, shift)


def test_pack_edges():
    cases = [np.zeros(1000, np.int32), np.ones(4097, np.int32), np.array([0, 0, 1000, 0], np.int32),
             np.array([5], np.int32), np.array([3, 2, 0, 1, 2], np.int32),
             inputs.compaction_inputs(300_001, seed=42)[1]]
    for counts in cases:
        ref_off, ref_total = oracle.pack_offsets(counts)
        for tuning in (None, {"block_size": 256, "items_per_thread": 4}):
            off = sw.pack_offsets(to_dev(counts), tuning=tuning)
            torch.cuda.synchronize()
            assert np.array_equal(to_host(off), ref_off)
        if ref_total:
            rec = sw.pack_emit_neighbors(off, ref_total)
            torch.cuda.synchronize()
            assert np.array_equal(to_host(rec)[:ref_total], oracle.pack_emit(ref_off))
    off = sw.pack_offsets(torch.empty(0, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert to_host(off).tolist() == [0]


@pytest.mark.parametrize("shift", [1, 2, 3])
def test_compaction_misaligned_output(shift):
    # The emit writes each tile's selected indices as one contiguous range cut
    # at the output's 16-byte boundaries: an output starting 1-3 elements past
    # a boundary exercises the partial quads at both ends of every range.
    # Sentinels around the output must stay untouched.
    x, _ = inputs.compaction_inputs(300_007, seed=44)
    ref = oracle.compact(x, "gt", 0.5)
    n = x.size
    for tuning in (None, {"block_size": 256, "items_per_thread": 4}):
        buf = torch.full((n + 8,), -7, dtype=torch.int32, device=DEV)
        out = buf[shift:shift + n]
        _, count = sw.compact_if(to_dev(x), "gt", 0.5, out=out, tuning=tuning)
        torch.cuda.synchronize()
        c = int(count.item())
        got = to_host(buf)
        assert c == ref.size
        assert np.array_equal(got[shift:shift + c], ref)
        assert (got[:shift] == -7).all() and (got[shift + n:] == -7).all()


@pytest.mark.parametrize("cmp", CMPS)
def test_compaction_special_floats(cmp):
    # IEEE comparisons: a NaN satisfies only "ne"; -0.0 equals 0.0; the
    # infinities order as usual.  Both sides compare in fp32.
    rng = np.random.default_rng(45)
    x = rng.random(70_001, dtype=np.float32) - np.float32(0.5)
    specials = np.array([np.nan, -np.nan, np.inf, -np.inf, 0.0, -0.0, 0.5, -0.5], np.float32)
    x[rng.integers(0, x.size, 5000)] = specials[rng.integers(0, specials.size, 5000)]
    for t in (0.0, 0.5, float("inf")):
        _check_compact(x, cmp, t)


def test_compaction_resident():
    # x of whole 128-bit vectors that fits one register tile per compute unit
    # (at most 256 tiles of rows x 960 x 4 elements, rows <= 17) takes the
    # resident compaction: both sides of its capacity, one-row and ragged
    # last tiles, every comparison, the bit predicates, closed forms and a
    # misaligned output.
    lo, cap = (8 << 20) // 4, 256 * 17 * 3840
    assert sw.plan("compact", torch.float32, "sum", 1, 4096)["kernel"] == "compact_resident"
    assert sw.plan("compact", torch.float32, "sum", 1, cap)["kernel"] == "compact_resident"
    assert sw.plan("compact", torch.float32, "sum", 1, cap + 4)["kernel"] == "compact"
    for n in (4096, 256 * 3840, 256 * 3840 + 4, cap, cap + 4):
        x, _ = inputs.compaction_inputs(n, seed=46)
        _check_compact(x)
    rng = np.random.default_rng(47)
    n = 3 * 3840 * 200 + 44  # 3 rows, 201 tiles, 44 elements in the last
    x = rng.random(n, dtype=np.float32)
    x[::97] = np.float32(0.5)  # exact ties
    for cmp in CMPS:
        _check_compact(x, cmp, 0.5)
    n = 7 * 3840 * 255 + 3840 + 12  # 7 rows, 256 tiles, the last with a row and 12 elements
    for dt in (np.int32, np.uint32):
        keys = rng.integers(0, 2 ** 32, n, dtype=np.uint64).astype(np.uint32).view(dt)
        for b in (0, 31):
            _check_compact(keys, "bit_set", b)
        _check_compact(keys, "le", 12345)
    for f in (np.ones(lo, np.float32), np.zeros(lo, np.float32), np.tile(np.array([0, 1], np.float32), lo // 2)):
        _check_compact(f)
    x, _ = inputs.compaction_inputs(lo + 4, seed=48)
    ref = oracle.compact(x, "gt", 0.5)
    buf = torch.full((x.size + 8,), -7, dtype=torch.int32, device=DEV)
    out = buf[3:3 + x.size]
    _, count = sw.compact_if(to_dev(x), "gt", 0.5, out=out)
    torch.cuda.synchronize()
    got = to_host(buf)
    assert int(count.item()) == ref.size
    assert np.array_equal(got[3:3 + ref.size], ref)
    assert (got[:3] == -7).all() and (got[3 + x.size:] == -7).all()
