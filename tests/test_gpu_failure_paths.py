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
    ws[:16].view(torch.int32)[1] = 1 << 30  # an epoch no descriptor tag can carry
    with _Installed(ws):
        sw.scan_inclusive(xd, tuning={"spin_limit": 32})
        torch.cuda.synchronize()
        assert sw.scan_workspace_error(ws) & 1
        _recovers(ws, x, xd)


def test_wrapped_start_count_times_out_end_of_call():
    x = inputs.generic(np.int32, 400_000, 23, "wide")
    xd = to_dev(x)
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device=DEV)
    ws[:16].view(torch.int32)[0] = -1  # count of started workgroups wraps past the grid size
    with _Installed(ws):
        r = sw.scan_inclusive(xd, tuning={"spin_limit": 32})
        torch.cuda.synchronize()
        assert sw.scan_workspace_error(ws) & 2
        assert_scan_matches(x, to_host(r), "sum", False)  # the scan itself was unaffected
        _recovers(ws, x, xd)


def test_errors_never_set_in_normal_operation():
    x = inputs.generic(np.float32, 3_000_000, 22)
    xd = to_dev(x)
    for _ in range(10):
        sw.scan_inclusive(xd)
    torch.cuda.synchronize()
    for ws in binding.workspaces._ws.values():
        assert sw.scan_workspace_error(ws) == 0
