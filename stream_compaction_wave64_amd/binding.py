"""Thin ctypes binding of libscan_wave64.so (include/scan_wave64.h).

Argument marshalling only: every step of every scan runs in the library's HIP
kernels.  Tensors must be CUDA (ROCm) tensors; calls enqueue on the current
torch stream of the tensor's device and never synchronize.  torch is imported
before the library is loaded so the library binds to the same HIP runtime as
torch.  If the library is missing, every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libscan_wave64.so")

DTYPES = {torch.int32: 0, torch.uint32: 1, torch.int64: 2, torch.float32: 3, torch.float64: 4}
OPS = {"sum": 0, "prod": 1, "max": 2, "min": 3}
ALGOS = {"auto": 0, "lookback": 1, "reduce_then_scan": 2, "rts": 2}
CMPS = {"gt": 0, "ge": 1, "lt": 2, "le": 3, "eq": 4, "ne": 5, "bit_clear": 6, "bit_set": 7}
CALLS = {"scan": 0, "compact": 1, "pack": 2, "partition": 3, "segmented": 4}
KERNELS = {0: "none", 1: "lookback", 2: "reduce_then_scan", 3: "element", 4: "columns", 5: "compact",
           6: "pack", 7: "partition", 8: "segmented", 9: "columns_lookback", 10: "resident",
           11: "compact_resident", 12: "partition_resident", 13: "rows"}


class ScanError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__(f"{fn} failed: {text} (status {status})")
        self.status = status


class Tuning(ctypes.Structure):
    _fields_ = [("block_size", ctypes.c_int32), ("items_per_thread", ctypes.c_int32),
                ("local_mem_bytes", ctypes.c_int64), ("algo", ctypes.c_int32),
                ("rts_blocks", ctypes.c_int32), ("spin_limit", ctypes.c_int32),
                ("grid_blocks", ctypes.c_int32), ("mode_limit", ctypes.c_int32),
                ("no_identity", ctypes.c_int32), ("delay_stride", ctypes.c_int32),
                ("delay_sleeps", ctypes.c_int32), ("resident_sweeps", ctypes.c_int32)]


class Plan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("items_per_thread", ctypes.c_int32), ("vec", ctypes.c_int32),
                ("tile_elems", ctypes.c_int64), ("num_tiles", ctypes.c_int64),
                ("lds_bytes", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
                ("launches", ctypes.c_int32), ("carry_words", ctypes.c_int32),
                ("tiles_per_block", ctypes.c_int32)]


EXPORTS = ["scan_plan", "scan_workspace_bytes", "scan_workspace_init", "scan_workspace_error", "scan_inclusive",
           "scan_inclusive_noalloc",
           "scan_exclusive", "scan_dim", "scan_segmented", "compact_if", "partition_if", "pack_offsets", "pack_emit_neighbors",
           "scan_copy", "scan_status_string", "scan_version"]

_lib = None
_lock = threading.Lock()


def load_library(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                               "(python -m stream_compaction_wave64_amd.build)")
        lib = ctypes.CDLL(path)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        tp = ctypes.POINTER(Tuning)
        sig = {
            "scan_plan": ([i32, i32, i32, i64, i64, i64, tp, ctypes.POINTER(Plan)], i32),
            "scan_workspace_bytes": ([i32, i64], sz),
            "scan_workspace_init": ([vp, sz, vp], i32),
            "scan_workspace_error": ([vp, ctypes.POINTER(ctypes.c_int32), vp], i32),
            "scan_inclusive": ([vp, vp, i64, i32, i32, i32, vp, sz, tp, vp], i32),
            "scan_inclusive_noalloc": ([vp, vp, i64, i32, i32, i32, tp, vp], i32),
            "scan_exclusive": ([vp, vp, i64, i32, i32, i32, vp, sz, tp, vp], i32),
            "scan_dim": ([vp, vp, i64, i64, i64, i32, i32, i32, vp, sz, tp, vp], i32),
            "compact_if": ([vp, i64, i32, i32, ctypes.c_double, vp, vp, vp, sz, tp, vp], i32),
            "scan_segmented": ([vp, vp, i64, vp, i64, i32, i32, i32, vp, sz, tp, vp], i32),
            "partition_if": ([vp, i64, i32, i32, ctypes.c_double, vp, vp, vp, vp, sz, tp, vp], i32),
            "pack_offsets": ([vp, i64, vp, vp, sz, tp, vp], i32),
            "pack_emit_neighbors": ([vp, i64, vp, vp], i32),
            "scan_copy": ([vp, vp, sz, vp], i32),
            "scan_status_string": ([i32], ctypes.c_char_p),
            "scan_version": ([], ctypes.c_char_p),
        }
        for name, (args, res) in sig.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = res
        _lib = lib
        return lib


def _check(fn, status):
    if status != 0:
        raise ScanError(fn, status, load_library().scan_status_string(status).decode())


def _tuning(t):
    if t is None:
        return None
    if isinstance(t, Tuning):
        return ctypes.byref(t)
    t = dict(t)
    if "algo" in t and isinstance(t["algo"], str):
        t["algo"] = ALGOS[t["algo"]]
    return ctypes.byref(Tuning(**t))


def _dtype(x: torch.Tensor) -> int:
    try:
        return DTYPES[x.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {x.dtype}") from None


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need_cuda(*tensors):
    for t in tensors:
        if not t.is_cuda:
            raise ValueError("tensors must live on a HIP device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


# ------------------------------------------------------------- workspaces

class _Workspaces:
    """One zero-initialised workspace per (device, stream), grown on demand.

    The library keeps its descriptors self-resetting, so a workspace is only
    zeroed when it is (re)allocated.  Distinct streams get distinct
    workspaces because calls on different streams may overlap in time."""

    def __init__(self):
        self._ws = {}

    def get(self, device: torch.device, nbytes: int) -> torch.Tensor:
        key = (device.index, _stream(device))
        ws = self._ws.get(key)
        if ws is None or ws.numel() < nbytes:
            nbytes = max(nbytes, 1 << 16, 0 if ws is None else 2 * ws.numel())
            ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
            self._ws[key] = ws
        return ws

    def clear(self):
        self._ws.clear()


workspaces = _Workspaces()


def plan(call: str, dtype: torch.dtype, op: str, outer: int, length: int, inner: int = 1, tuning=None) -> dict:
    """The launch a call would enqueue (host only, no device needed)."""
    lib = load_library()
    p = Plan()
    _check("scan_plan", lib.scan_plan(CALLS[call], DTYPES[dtype], OPS[op], outer, length, inner,
                                      _tuning(tuning), ctypes.byref(p)))
    d = {f: getattr(p, f) for f, _ in Plan._fields_}
    d["kernel"] = KERNELS.get(d["kernel"], d["kernel"])
    return d


def _workspace_for(call, x, op, outer, length, inner, tuning):
    p = plan(call, x.dtype, op, outer, length, inner, tuning)
    nbytes = int(p["workspace_bytes"])
    ws = workspaces.get(x.device, nbytes)
    return ws, ws.numel()


# ------------------------------------------------------------------ scans

def _scan(fn_name, x, op, out, width, tuning):
    lib = load_library()
    _need_cuda(x)
    if out is None:
        out = torch.empty_like(x)
    _need_cuda(out)
    if out.dtype != x.dtype or out.numel() != x.numel():
        raise ValueError("out must match x in dtype and size")
    if width < 1 or x.numel() % width:
        raise ValueError("width must divide the element count")
    n = x.numel() // width
    ws, wsb = _workspace_for("scan", x, op, 1, n, width, tuning)
    fn = getattr(lib, fn_name)
    _check(fn_name, fn(x.data_ptr(), out.data_ptr(), n, _dtype(x), OPS[op], width, ws.data_ptr(), wsb,
                       _tuning(tuning), _stream(x.device)))
    return out


def scan_inclusive(x: torch.Tensor, op: str = "sum", out=None, width: int = 1, tuning=None) -> torch.Tensor:
    """out[i] = x[0] (+) ... (+) x[i] over the flattened tensor (structs of
    `width` components scanned component-wise)."""
    return _scan("scan_inclusive", x, op, out, width, tuning)


def scan_inclusive_noalloc(x: torch.Tensor, out: torch.Tensor, op: str = "sum", width: int = 1,
                           tuning=None) -> torch.Tensor:
    """scan_inclusive on the library's own per-GPU workspace: no allocation,
    so `out` must be given.  Calls that may overlap on one GPU race."""
    lib = load_library()
    _need_cuda(x, out)
    if out.dtype != x.dtype or out.numel() != x.numel():
        raise ValueError("out must match x in dtype and size")
    if width < 1 or x.numel() % width:
        raise ValueError("width must divide the element count")
    n = x.numel() // width
    _check("scan_inclusive_noalloc", lib.scan_inclusive_noalloc(x.data_ptr(), out.data_ptr(), n, _dtype(x), OPS[op],
                                                                width, _tuning(tuning), _stream(x.device)))
    return out


def scan_exclusive(x: torch.Tensor, op: str = "sum", out=None, width: int = 1, tuning=None) -> torch.Tensor:
    """out[0] = identity, out[i] = x[0] (+) ... (+) x[i-1]."""
    return _scan("scan_exclusive", x, op, out, width, tuning)


def scan_dim(x: torch.Tensor, dim: int, op: str = "sum", exclusive: bool = False, out=None,
             tuning=None) -> torch.Tensor:
    """Scan of a contiguous tensor along `dim`."""
    lib = load_library()
    _need_cuda(x)
    dim = dim % max(x.dim(), 1)
    shape = list(x.shape) or [1]
    outer = 1
    for s in shape[:dim]:
        outer *= s
    length = shape[dim]
    inner = 1
    for s in shape[dim + 1:]:
        inner *= s
    if out is None:
        out = torch.empty_like(x)
    _need_cuda(out)
    ws, wsb = _workspace_for("scan", x, op, outer, length, inner, tuning)
    _check("scan_dim", lib.scan_dim(x.data_ptr(), out.data_ptr(), outer, length, inner, _dtype(x), OPS[op],
                                    int(exclusive), ws.data_ptr(), wsb, _tuning(tuning), _stream(x.device)))
    return out


def scan_segmented(x: torch.Tensor, offsets: torch.Tensor, op: str = "sum", exclusive: bool = False, out=None,
                   tuning=None) -> torch.Tensor:
    """Each ragged segment x[offsets[s] .. offsets[s+1]) scanned on its own
    (offsets: int32 device tensor of nseg + 1 non-decreasing values from 0 to
    x.numel(), as pack_offsets writes them)."""
    lib = load_library()
    _need_cuda(x, offsets)
    if offsets.dtype != torch.int32 or offsets.dim() != 1 or offsets.numel() < 1:
        raise ValueError("offsets must be a 1-D int32 tensor of nseg + 1 entries")
    if out is None:
        out = torch.empty_like(x)
    _need_cuda(out)
    if out.dtype != x.dtype or out.numel() != x.numel():
        raise ValueError("out must match x in dtype and size")
    n, nseg = x.numel(), offsets.numel() - 1
    ws, wsb = _workspace_for("segmented", x, op, nseg, n, 1, tuning)
    _check("scan_segmented", lib.scan_segmented(x.data_ptr(), out.data_ptr(), n, offsets.data_ptr(), nseg, _dtype(x),
                                                OPS[op], int(exclusive), ws.data_ptr(), wsb, _tuning(tuning),
                                                _stream(x.device)))
    return out


def compact_if(x: torch.Tensor, cmp: str = "gt", threshold: float = 0.5, out=None, count=None, tuning=None):
    """Indices i with x[i] <cmp> threshold, in order.  Returns (out, count):
    out has x.numel() int32 slots of which the first count[0] are written;
    count is a 1-element int32 device tensor (no synchronisation here)."""
    lib = load_library()
    _need_cuda(x)
    n = x.numel()
    if out is None:
        out = torch.empty(max(n, 1), dtype=torch.int32, device=x.device)
    if count is None:
        count = torch.empty(1, dtype=torch.int32, device=x.device)
    _need_cuda(out, count)
    if out.dtype != torch.int32 or out.numel() < n:
        raise ValueError("out must be int32 with n entries")
    ws, wsb = _workspace_for("compact", x, "sum", 1, n, 1, tuning)
    _check("compact_if", lib.compact_if(x.data_ptr(), n, _dtype(x), CMPS[cmp], float(threshold), out.data_ptr(),
                                        count.data_ptr(), ws.data_ptr(), wsb, _tuning(tuning), _stream(x.device)))
    return out, count


def partition_if(x: torch.Tensor, cmp: str = "gt", threshold: float = 0.5, out=None, out_idx=None,
                 with_idx: bool = True, count=None, tuning=None):
    """Stable partition of x: the elements with x[i] <cmp> threshold first,
    then the others, each part in input order.  Returns (out, out_idx,
    count): out_idx holds each output's source index (None when with_idx is
    False and no out_idx is given); count is a 1-element int32 device tensor
    (no synchronisation here).  bit_clear / bit_set test bit `threshold` of
    an integer key (one pass of an LSD radix sort)."""
    lib = load_library()
    _need_cuda(x)
    n = x.numel()
    if out is None:
        out = torch.empty(max(n, 1), dtype=x.dtype, device=x.device)
    if out_idx is None and with_idx:
        out_idx = torch.empty(max(n, 1), dtype=torch.int32, device=x.device)
    if count is None:
        count = torch.empty(1, dtype=torch.int32, device=x.device)
    _need_cuda(out, count)
    if out.dtype != x.dtype or out.numel() < n:
        raise ValueError("out must match x in dtype and hold n values")
    if out_idx is not None:
        _need_cuda(out_idx)
        if out_idx.dtype != torch.int32 or out_idx.numel() < n:
            raise ValueError("out_idx must be int32 with n entries")
    ws, wsb = _workspace_for("partition", x, "sum", 1, n, 1, tuning)
    _check("partition_if", lib.partition_if(x.data_ptr(), n, _dtype(x), CMPS[cmp], float(threshold), out.data_ptr(),
                                            out_idx.data_ptr() if out_idx is not None else None, count.data_ptr(),
                                            ws.data_ptr(), wsb, _tuning(tuning), _stream(x.device)))
    return out, out_idx, count


def pack_offsets(counts: torch.Tensor, out=None, tuning=None) -> torch.Tensor:
    """offsets[0..n]: exclusive scan of int32 counts with the total at offsets[n]."""
    lib = load_library()
    _need_cuda(counts)
    if counts.dtype != torch.int32:
        raise TypeError("counts must be int32")
    n = counts.numel()
    if out is None:
        out = torch.empty(n + 1, dtype=torch.int32, device=counts.device)
    _need_cuda(out)
    ws, wsb = _workspace_for("pack", counts, "sum", 1, n, 1, tuning)
    _check("pack_offsets", lib.pack_offsets(counts.data_ptr(), n, out.data_ptr(), ws.data_ptr(), wsb,
                                            _tuning(tuning), _stream(counts.device)))
    return out


def pack_emit_neighbors(offsets: torch.Tensor, total: int, out=None) -> torch.Tensor:
    """Records of every object at its offset: object i, record j -> (i+1+j) mod n."""
    lib = load_library()
    _need_cuda(offsets)
    n = offsets.numel() - 1
    if out is None:
        out = torch.empty(max(int(total), 1), dtype=torch.int32, device=offsets.device)
    _need_cuda(out)
    _check("pack_emit_neighbors", lib.pack_emit_neighbors(offsets.data_ptr(), n, out.data_ptr(),
                                                          _stream(offsets.device)))
    return out


def scan_copy(x: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """Copy-ceiling kernel: same 128-bit tile access pattern as the fp32 scan."""
    lib = load_library()
    _need_cuda(x, out)
    nbytes = x.numel() * x.element_size()
    _check("scan_copy", lib.scan_copy(x.data_ptr(), out.data_ptr(), nbytes, _stream(x.device)))
    return out


def scan_workspace_init(ws: torch.Tensor) -> None:
    lib = load_library()
    _need_cuda(ws)
    _check("scan_workspace_init", lib.scan_workspace_init(ws.data_ptr(), ws.numel() * ws.element_size(),
                                                          _stream(ws.device)))


def scan_workspace_error(ws: torch.Tensor) -> int:
    """Error word of a workspace (synchronizes the current stream)."""
    lib = load_library()
    _need_cuda(ws)
    err = ctypes.c_int32(0)
    _check("scan_workspace_error", lib.scan_workspace_error(ws.data_ptr(), ctypes.byref(err), _stream(ws.device)))
    return err.value


def scan_workspace_bytes(dtype: torch.dtype, count: int) -> int:
    return int(load_library().scan_workspace_bytes(DTYPES[dtype], count))


def version() -> str:
    return load_library().scan_version().decode()
