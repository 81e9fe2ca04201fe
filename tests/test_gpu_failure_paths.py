"""Failure handling of the look-back, forced from the host so that every
kernel still exits normally: a workspace header that was never zeroed makes
the waits give up after a tiny spin limit and flag the error word; zeroing
the workspace again recovers."""
import numpy as np
import pytest
import torch

import stream_compaction_wave64_amd as sw
from stream_compaction_wave64_amd import binding, inputs
from gpu_util import DEV, assert_scan_matches, to_dev, to_host

pytestmark = pytest.mark.gpu


class _Installed:
    """Install `ws` as the binding's workspace for the current stream."""

    def __init__(self, ws):
        self.ws = ws
        self.key = (torch.device(DEV).index, binding._stream(torch.device(DEV)))

    def __enter__(self):
        self.saved = binding.workspaces._ws.get(self.key)
        binding.workspaces._ws[self.key] = self.ws
        return self.ws

    def __exit__(self, *exc):
        if self.saved is None:
            binding.workspaces._ws.pop(self.key, None)
        else:
            binding.workspaces._ws[self.key] = self.saved


def _recovers(ws, x, xd):
    sw.scan_workspace_init(ws)
    assert sw.scan_workspace_error(ws) == 0
    r = sw.scan_inclusive(xd)
    torch.cuda.synchronize()
    assert sw.scan_workspace_error(ws) == 0
    assert_scan_matches(x, to_host(r), "sum", False)


def test_garbage_epoch_times_out_lookback_and_reinit_recovers():
    x = inputs.generic(np.int32, 400_000, 21, "wide")
    xd = to_dev(x)
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device=DEV)
    ws[:16].view(torch.int32)[0] = 1 << 30  # an epoch no descriptor tag can carry
    with _Installed(ws):
        # the look-back pipeline's small-array tiles (the resident pass has
        # its own case below)
        sw.scan_inclusive(xd, tuning={"spin_limit": 32, "block_size": 512, "items_per_thread": 20})
        torch.cuda.synchronize()
        assert sw.scan_workspace_error(ws) & 1
        _recovers(ws, x, xd)


@pytest.mark.parametrize("dt", [np.int32, np.float32, np.float64])
def test_unconfirmed_residency_falls_back_to_dynamic_claiming(dt):
    # A start count that wraps past the grid size never confirms that all
    # workgroups are resident: the call must take the dynamic path (flag bit 2)
    # and still produce the exact result, over many tiles and small grids.
    x = inputs.generic(dt, 1_000_003, 23, "wide" if dt == np.int32 else "default")
    xd = to_dev(x)
    vec = 16 // np.dtype(dt).itemsize
    for tuning in ({"mode_limit": 8}, {"mode_limit": 8, "block_size": 256, "items_per_thread": vec},
                   {"mode_limit": 8, "grid_blocks": 5}):
        ws = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
        ws[128:132].view(torch.int32)[0] = -1  # first started-count slot
        with _Installed(ws):
            for excl in (False, True):
                fn = sw.scan_exclusive if excl else sw.scan_inclusive
                r = fn(xd, tuning=tuning)
                torch.cuda.synchronize()
                assert sw.scan_workspace_error(ws) == 4, tuning
                assert_scan_matches(x, to_host(r), "sum", excl, what=str(tuning))
                ws[128:132].view(torch.int32)[0] = -1  # the call reset it; force the fallback again
            _recovers(ws, x, xd)


def test_errors_never_set_in_normal_operation():
    # No call falls back to dynamic claiming or times out on its own: the
    # default shapes, and the persistent grids of 256-thread tiles whose
    # occupancy the runtime overstates (64-bit elements, one 16-byte row or
    # element-wide access).
    for ws in binding.workspaces._ws.values():
        sw.scan_workspace_init(ws)
    x = inputs.generic(np.float32, 3_000_000, 22)
    xd = to_dev(x)
    for _ in range(10):
        sw.scan_inclusive(xd)
    for dt in (np.int64, np.float64, np.int32):
        vec = 16 // np.dtype(dt).itemsize
        for n in (300_000 * vec, 300_001):
            y = to_dev(inputs.generic(dt, n, 24, "wide" if dt != np.float64 else "near1"))
            for op in ("sum", "prod", "max"):
                sw.scan_inclusive(y, op=op, tuning={"block_size": 256, "items_per_thread": vec})
    torch.cuda.synchronize()
    for ws in binding.workspaces._ws.values():
        assert sw.scan_workspace_error(ws) == 0


# Late publishers: tiles picked by a stride wait (s_sleep periods of about
# 1.7 us) before publishing their aggregate, so the look-back reaches its
# re-polls deterministically: the gap read of the static order re-reads the
# slots still unpublished, the windowed look-back of large grids and of
# dynamic claiming spins on a window with no P (The CUDA Handbook ch. 13,
# decoupled look-back section, Figure 13-11).  Results must stay exact and
# no wait may give up (default spin limit).
DELAYS = [(7, 1), (3, 8), (1, 2), (64, 30)]


@pytest.mark.parametrize("stride,sleeps", DELAYS)
def test_late_publishers_gap_read_and_windowed(stride, sleeps):
    delay = {"delay_stride": stride, "delay_sleeps": sleeps}
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    cases = [
        (np.float32, 30_000_001, {}),                                            # gap read, 256 workgroups
        (np.int32, 1_000_003, {"block_size": 256, "items_per_thread": 4}),       # windowed: > 513 workgroups
        (np.int64, 500_001, {"block_size": 256, "items_per_thread": 2, "grid_blocks": 5}),
        (np.float64, 2_000_003, {}),
    ]
    with _Installed(ws):
        for dt, n, tuning in cases:
            x = inputs.generic(dt, n, 40 + stride, "wide" if np.issubdtype(dt, np.integer) else "default")
            xd = to_dev(x)
            for excl in (False, True):
                fn = sw.scan_exclusive if excl else sw.scan_inclusive
                r = fn(xd, tuning=dict(tuning, **delay))
                torch.cuda.synchronize()
                assert_scan_matches(x, to_host(r), "sum", excl, what=f"{np.dtype(dt).name} {tuning} {delay}")
            assert sw.scan_workspace_error(ws) == 0, (tuning, delay)


@pytest.mark.parametrize("stride,sleeps", DELAYS[:2])
def test_late_publishers_dynamic_claiming_and_no_identity(stride, sleeps):
    delay = {"delay_stride": stride, "delay_sleeps": sleeps}
    x = inputs.generic(np.int32, 1_000_003, 50 + stride, "wide")
    xd = to_dev(x)
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    with _Installed(ws):
        ws[128:132].view(torch.int32)[0] = -1  # never confirms residency: dynamic claiming
        r = sw.scan_inclusive(xd, tuning=dict(delay, mode_limit=8, block_size=256, items_per_thread=4))
        torch.cuda.synchronize()
        assert sw.scan_workspace_error(ws) == 4
        assert_scan_matches(x, to_host(r), "sum", False, what="dynamic")
        sw.scan_workspace_init(ws)
        f = inputs.generic(np.float32, 3_000_001, 60 + stride)
        for tuning in ({}, {"block_size": 256, "items_per_thread": 4}):
            r = sw.scan_inclusive(to_dev(f), tuning=dict(tuning, no_identity=1, **delay))
            torch.cuda.synchronize()
            assert_scan_matches(f, to_host(r), "sum", False, what=f"no identity {tuning}", noid=True)
        assert sw.scan_workspace_error(ws) == 0


@pytest.mark.parametrize("n,rows", [(3_000_000, 4), (1_000_000, 2)])
def test_resident_pass_failure_paths(n, rows):
    # The resident single pass (arrays that fit one register tile per compute
    # unit) under the same forced conditions: a residency check that never
    # confirms (dynamic claiming, flag bit 2, exact results), late publishers
    # (the gap read's re-polls, exact results, no flag) and a garbage epoch
    # (the waits give up: flag bit 0).  4-row tiles decide the residency
    # while they load; 131 tiles of 2 rows publish their static tile first.
    x = inputs.generic(np.int32, n, 70, "wide")
    xd = to_dev(x)
    p = sw.plan("scan", torch.int32, "sum", 1, x.size)
    assert (p["kernel"], p["items_per_thread"], p["tiles_per_block"]) == ("resident", 4 * rows, 1), p
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    with _Installed(ws):
        for excl in (False, True):
            ws[128:132].view(torch.int32)[0] = -1
            fn = sw.scan_exclusive if excl else sw.scan_inclusive
            r = fn(xd, tuning={"mode_limit": 8})
            torch.cuda.synchronize()
            assert sw.scan_workspace_error(ws) == 4
            assert_scan_matches(x, to_host(r), "sum", excl, what=f"dynamic excl={excl}")
        sw.scan_workspace_init(ws)
        f = inputs.generic(np.float32, n, 71)
        fd = to_dev(f)
        for stride, sleeps in DELAYS:
            for excl in (False, True):
                fn = sw.scan_exclusive if excl else sw.scan_inclusive
                r = fn(fd, tuning={"delay_stride": stride, "delay_sleeps": sleeps})
                torch.cuda.synchronize()
                assert_scan_matches(f, to_host(r), "sum", excl, what=f"late publishers {stride} {sleeps}")
            # without an identity: the look-back's optional carries re-polled
            r = sw.scan_inclusive(fd, tuning={"delay_stride": stride, "delay_sleeps": sleeps, "no_identity": 1})
            torch.cuda.synchronize()
            assert_scan_matches(f, to_host(r), "sum", False, what=f"no identity, late {stride} {sleeps}", noid=True)
        assert sw.scan_workspace_error(ws) == 0
        # without an identity under dynamic claiming (each workgroup scans the
        # tile it claims, which need not be its own)
        assert sw.plan("scan", torch.int32, "max", 1, x.size, tuning={"no_identity": 1})["kernel"] == "resident"
        ws[128:132].view(torch.int32)[0] = -1
        r = sw.scan_inclusive(xd, op="max", tuning={"mode_limit": 8, "no_identity": 1})
        torch.cuda.synchronize()
        assert sw.scan_workspace_error(ws) == 4
        assert_scan_matches(x, to_host(r), "max", False, what="no identity, dynamic", noid=True)
        sw.scan_workspace_init(ws)
        ws[:16].view(torch.int32)[0] = 1 << 30
        sw.scan_inclusive(xd, tuning={"spin_limit": 32})
        torch.cuda.synchronize()
        assert sw.scan_workspace_error(ws) & 1
        _recovers(ws, x, xd)


def test_resident_two_tile_failure_paths():
    # The resident pass with two tiles per workgroup under the same forced
    # conditions: dynamic claiming (claim k takes tiles 2k and 2k + 1 and
    # reloads them; its first tile reads up to 510 aggregates, two gap reads),
    # late publishers on both tiles' aggregates (with and without an
    # identity), and a garbage epoch whose waits give up.
    x = inputs.generic(np.int32, 10_000_004, 72, "wide")
    xd = to_dev(x)
    p = sw.plan("scan", torch.int32, "sum", 1, x.size)
    assert (p["kernel"], p["tiles_per_block"], p["num_tiles"] % 2) == ("resident", 2, 1), p
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    with _Installed(ws):
        for excl in (False, True):
            ws[128:132].view(torch.int32)[0] = -1
            fn = sw.scan_exclusive if excl else sw.scan_inclusive
            r = fn(xd, tuning={"mode_limit": 8})
            torch.cuda.synchronize()
            assert sw.scan_workspace_error(ws) == 4
            assert_scan_matches(x, to_host(r), "sum", excl, what=f"dynamic excl={excl}")
        ws[128:132].view(torch.int32)[0] = -1
        r = sw.scan_inclusive(xd, op="max", tuning={"mode_limit": 8, "no_identity": 1})
        torch.cuda.synchronize()
        assert sw.scan_workspace_error(ws) == 4
        assert_scan_matches(x, to_host(r), "max", False, what="no identity, dynamic", noid=True)
        sw.scan_workspace_init(ws)
        f = inputs.generic(np.float32, 10_000_012, 73)
        fd = to_dev(f)
        assert sw.plan("scan", torch.float32, "sum", 1, f.size)["tiles_per_block"] == 2
        for stride, sleeps in DELAYS:
            for excl in (False, True):
                fn = sw.scan_exclusive if excl else sw.scan_inclusive
                r = fn(fd, tuning={"delay_stride": stride, "delay_sleeps": sleeps})
                torch.cuda.synchronize()
                assert_scan_matches(f, to_host(r), "sum", excl, what=f"late publishers {stride} {sleeps}")
            r = sw.scan_inclusive(fd, tuning={"delay_stride": stride, "delay_sleeps": sleeps, "no_identity": 1})
            torch.cuda.synchronize()
            assert_scan_matches(f, to_host(r), "sum", False, what=f"no identity, late {stride} {sleeps}", noid=True)
        assert sw.scan_workspace_error(ws) == 0
        ws[:16].view(torch.int32)[0] = 1 << 30
        sw.scan_inclusive(xd, tuning={"spin_limit": 32})
        torch.cuda.synchronize()
        assert sw.scan_workspace_error(ws) & 1
        _recovers(ws, x, xd)


@pytest.mark.parametrize("n,rows", [(3_000_000, 4), (10_000_000, 11)])
def test_resident_compaction_failure_paths(n, rows):
    # The resident compaction under the same forced conditions: dynamic
    # claiming (flag bit 2), late publishers, a garbage epoch (flag bit 0).
    # 4-row tiles publish their static tile's count before the residency
    # decision; 11-row tiles decide while they load.
    import oracle
    x, _ = inputs.compaction_inputs(n, seed=72)
    xd = to_dev(x)
    ref = oracle.compact(x, "gt", 0.5)
    p = sw.plan("compact", torch.float32, "sum", 1, x.size)
    assert (p["kernel"], p["items_per_thread"]) == ("compact_resident", 4 * rows), p

    def run(tuning):
        out, count = sw.compact_if(xd, "gt", 0.5, tuning=tuning)
        torch.cuda.synchronize()
        c = int(count.item())
        return c, to_host(out[:c])

    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    with _Installed(ws):
        ws[128:132].view(torch.int32)[0] = -1
        c, got = run({"mode_limit": 8})
        assert sw.scan_workspace_error(ws) == 4
        assert c == ref.size and np.array_equal(got, ref)
        sw.scan_workspace_init(ws)
        for stride, sleeps in DELAYS:
            c, got = run({"delay_stride": stride, "delay_sleeps": sleeps})
            assert c == ref.size and np.array_equal(got, ref), (stride, sleeps)
        assert sw.scan_workspace_error(ws) == 0
        ws[:16].view(torch.int32)[0] = 1 << 30
        run({"spin_limit": 32})
        assert sw.scan_workspace_error(ws) & 1
        sw.scan_workspace_init(ws)
        c, got = run(None)
        assert sw.scan_workspace_error(ws) == 0
        assert c == ref.size and np.array_equal(got, ref)


@pytest.mark.parametrize("n,rows", [(3_000_000, 4), (10_000_000, 11)])
def test_resident_partition_failure_paths(n, rows):
    # The resident partition under the same forced conditions: dynamic
    # claiming (flag bit 2), late publishers, a garbage epoch (flag bit 0),
    # with the residency decided after (4 rows) and before (11 rows)
    # the static tile's count is published.
    import oracle
    x, _ = inputs.compaction_inputs(n, seed=73)
    xd = to_dev(x)
    vals, idx, k = oracle.partition(x, "gt", 0.5)
    p = sw.plan("partition", torch.float32, "sum", 1, x.size)
    assert (p["kernel"], p["items_per_thread"]) == ("partition_resident", 4 * rows), p

    def run(tuning):
        out, oi, count = sw.partition_if(xd, "gt", 0.5, tuning=tuning)
        torch.cuda.synchronize()
        return int(count.item()), to_host(out).view(np.uint32), to_host(oi)

    def ok(res):
        c, v, i = res
        return c == k and np.array_equal(v, vals.view(np.uint32)) and np.array_equal(i, idx)

    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    with _Installed(ws):
        ws[128:132].view(torch.int32)[0] = -1
        assert ok(run({"mode_limit": 8}))
        assert sw.scan_workspace_error(ws) == 4
        sw.scan_workspace_init(ws)
        for stride, sleeps in DELAYS:
            assert ok(run({"delay_stride": stride, "delay_sleeps": sleeps})), (stride, sleeps)
        assert sw.scan_workspace_error(ws) == 0
        ws[:16].view(torch.int32)[0] = 1 << 30
        run({"spin_limit": 32})
        assert sw.scan_workspace_error(ws) & 1
        sw.scan_workspace_init(ws)
        assert ok(run(None))
        assert sw.scan_workspace_error(ws) == 0
