"""Sequential CPU oracle for scan, compaction and packing (ctypes over oracle.c).

TEST INFRASTRUCTURE ONLY: tests/, the smoke check in __graft_entry__.py and the
cpu_baseline leg of bench.py may import this package; the library under
stream_compaction_wave64_amd/ never does, and this package never imports it.

Every function takes and returns numpy arrays.  Scans work on a dense
row-major (outer, len, inner) array and scan along the middle axis, following
the exclusive / inclusive prefix-sum definitions on Merry's "Prefix sums on
GPUs" slides; floating-point results are returned in fp64 (fp32 inputs are
accumulated in fp64, fp64 inputs in double-double).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OPS = {"sum": 0, "prod": 1, "max": 2, "min": 3}
CMPS = {"gt": 0, "ge": 1, "lt": 2, "le": 3, "eq": 4, "ne": 5, "bit_clear": 6, "bit_set": 7}

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc -O2 (no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        for name in ("oracle_scan_i32", "oracle_scan_u32", "oracle_scan_i64",
                     "oracle_scan_f32", "oracle_scan_f64"):
            f = getattr(lib, name)
            f.argtypes = [vp, vp, i64, i64, i64, i32, i32]
            f.restype = i32
        for name in ("oracle_scan_noid_i32", "oracle_scan_noid_u32", "oracle_scan_noid_i64",
                     "oracle_scan_noid_f32", "oracle_scan_noid_f64"):
            f = getattr(lib, name)
            f.argtypes = [vp, vp, i64, i64, i64, i32]
            f.restype = i32
        for name in ("oracle_abs_prefix_f32", "oracle_abs_prefix_f64"):
            f = getattr(lib, name)
            f.argtypes = [vp, vp, i64, i64, i64, i32]
            f.restype = i32
        lib.oracle_compact_f32.argtypes = [vp, i64, i32, ctypes.c_float, vp]
        lib.oracle_compact_f32.restype = i64
        lib.oracle_compact_i32.argtypes = [vp, i64, i32, ctypes.c_int32, vp]
        lib.oracle_compact_i32.restype = i64
        lib.oracle_compact_u32.argtypes = [vp, i64, i32, ctypes.c_uint32, vp]
        lib.oracle_compact_u32.restype = i64
        lib.oracle_partition_f32.argtypes = [vp, i64, i32, ctypes.c_float, vp, vp]
        lib.oracle_partition_i32.argtypes = [vp, i64, i32, ctypes.c_int32, vp, vp]
        lib.oracle_partition_u32.argtypes = [vp, i64, i32, ctypes.c_uint32, vp, vp]
        for name in ("oracle_partition_f32", "oracle_partition_i32", "oracle_partition_u32"):
            getattr(lib, name).restype = i64
        for name in ("oracle_segscan_i32", "oracle_segscan_u32", "oracle_segscan_i64",
                     "oracle_segscan_f32", "oracle_segscan_f64"):
            f = getattr(lib, name)
            f.argtypes = [vp, vp, vp, i64, i32, i32]
            f.restype = i32
        lib.oracle_pack_offsets.argtypes = [vp, i64, vp]
        lib.oracle_pack_offsets.restype = i64
        lib.oracle_pack_emit.argtypes = [vp, i64, vp]
        lib.oracle_pack_emit.restype = i32
        lib.oracle_block_size.argtypes = [i64, i64, i64, i64]
        lib.oracle_block_size.restype = i64
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _dims(x: np.ndarray, dims):
    if dims is None:
        return 1, x.size, 1
    outer, length, inner = (int(d) for d in dims)
    if outer * length * inner != x.size:
        raise ValueError(f"dims {dims} do not match size {x.size}")
    return outer, length, inner


_SCAN = {
    np.dtype(np.int32): ("oracle_scan_i32", np.int32),
    np.dtype(np.uint32): ("oracle_scan_u32", np.uint32),
    np.dtype(np.int64): ("oracle_scan_i64", np.int64),
    np.dtype(np.float32): ("oracle_scan_f32", np.float64),
    np.dtype(np.float64): ("oracle_scan_f64", np.float64),
}


def scan(x: np.ndarray, op: str = "sum", exclusive: bool = False, dims=None) -> np.ndarray:
    """Scan of x along the middle axis of (outer, len, inner).

    Integers: same dtype, wrapping arithmetic.  fp32 / fp64: fp64 result.
    """
    lib = _load()
    x = np.ascontiguousarray(x)
    name, out_t = _SCAN[x.dtype]
    outer, length, inner = _dims(x, dims)
    y = np.empty(x.size, dtype=out_t)
    if x.size:
        rc = getattr(lib, name)(_ptr(x), _ptr(y), outer, length, inner, OPS[op], int(exclusive))
        if rc != 0:
            raise ValueError("oracle scan rejected its arguments")
    return y.reshape(x.shape)


def scan_noid(x: np.ndarray, op: str = "sum", dims=None) -> np.ndarray:
    """Inclusive scan that never uses the operator's identity: each column
    starts from its first element (AcceleratedKernels.jl PR #208's Optional
    partials for operators without a neutral element).  Result types as for
    scan()."""
    lib = _load()
    x = np.ascontiguousarray(x)
    name, out_t = _SCAN[x.dtype]
    outer, length, inner = _dims(x, dims)
    y = np.empty(x.size, dtype=out_t)
    if x.size:
        rc = getattr(lib, name.replace("oracle_scan_", "oracle_scan_noid_"))(_ptr(x), _ptr(y), outer, length,
                                                                              inner, OPS[op])
        if rc != 0:
            raise ValueError("oracle scan rejected its arguments")
    return y.reshape(x.shape)


def scan_segmented(x: np.ndarray, offsets: np.ndarray, op: str = "sum", exclusive: bool = False) -> np.ndarray:
    """Each ragged segment x[offsets[s] .. offsets[s+1]) scanned on its own
    (offsets: int32, non-decreasing, offsets[0] = 0, offsets[-1] = x.size).
    Result types as for scan()."""
    lib = _load()
    x = np.ascontiguousarray(x)
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    if off.size < 1 or off[0] != 0 or off[-1] != x.size or np.any(np.diff(off.astype(np.int64)) < 0):
        raise ValueError("offsets must be non-decreasing from 0 to x.size")
    name, out_t = _SCAN[x.dtype]
    y = np.empty(x.size, dtype=out_t)
    if x.size:
        rc = getattr(lib, name.replace("oracle_scan_", "oracle_segscan_"))(
            _ptr(x), _ptr(y), _ptr(off), off.size - 1, OPS[op], int(exclusive))
        if rc != 0:
            raise ValueError("oracle segmented scan rejected its arguments")
    return y


def segment_abs_prefix(x: np.ndarray, offsets: np.ndarray, exclusive: bool = False) -> np.ndarray:
    """P_i of a segmented scan, in fp64: the sum of |x_j| over the inputs
    output i depends on (the segmented scan of |x| itself, so each segment's
    sum starts from zero with no cancellation)."""
    return scan_segmented(np.abs(np.ascontiguousarray(x)), offsets, "sum", exclusive)


def abs_prefix(x: np.ndarray, exclusive: bool = False, dims=None) -> np.ndarray:
    """P_i: sum of |x_j| over the inputs output i depends on, in fp64."""
    lib = _load()
    x = np.ascontiguousarray(x)
    outer, length, inner = _dims(x, dims)
    p = np.empty(x.size, dtype=np.float64)
    if x.size:
        fn = {np.dtype(np.float32): lib.oracle_abs_prefix_f32,
              np.dtype(np.float64): lib.oracle_abs_prefix_f64}[x.dtype]
        fn(_ptr(x), _ptr(p), outer, length, inner, int(exclusive))
    return p.reshape(x.shape)


def _threshold(x: np.ndarray, cmp: str, threshold):
    if cmp.startswith("bit_"):
        if x.dtype == np.float32:
            raise TypeError("bit predicates take integer keys")
        return int(threshold) & 31
    return float(np.float32(threshold)) if x.dtype == np.float32 else int(threshold)


def compact(x: np.ndarray, cmp: str = "gt", threshold=0.5) -> np.ndarray:
    """Ascending int32 indices i with x[i] <cmp> threshold (in x's precision;
    bit_clear / bit_set test bit `threshold` of an integer key)."""
    lib = _load()
    x = np.ascontiguousarray(x)
    idx = np.empty(max(x.size, 1), dtype=np.int32)
    fn = {np.dtype(np.float32): lib.oracle_compact_f32, np.dtype(np.int32): lib.oracle_compact_i32,
          np.dtype(np.uint32): lib.oracle_compact_u32}.get(x.dtype)
    if fn is None:
        raise TypeError(x.dtype)
    cnt = fn(_ptr(x), x.size, CMPS[cmp], _threshold(x, cmp, threshold), _ptr(idx))
    return idx[:cnt].copy()


def partition(x: np.ndarray, cmp: str = "gt", threshold=0.5):
    """Stable partition: (vals, idx, k) with the k elements that satisfy the
    predicate first, then the others, each part in input order; idx holds
    each output's source index (int32)."""
    lib = _load()
    x = np.ascontiguousarray(x)
    fn = {np.dtype(np.float32): lib.oracle_partition_f32, np.dtype(np.int32): lib.oracle_partition_i32,
          np.dtype(np.uint32): lib.oracle_partition_u32}.get(x.dtype)
    if fn is None:
        raise TypeError(x.dtype)
    vals = np.empty(max(x.size, 1), dtype=x.dtype)
    idx = np.empty(max(x.size, 1), dtype=np.int32)
    k = fn(_ptr(x), x.size, CMPS[cmp], _threshold(x, cmp, threshold), _ptr(vals), _ptr(idx))
    return vals[: x.size].copy(), idx[: x.size].copy(), int(k)


def pack_offsets(counts: np.ndarray):
    """(offsets[n+1] int32, total as a Python int computed in 64 bits)."""
    lib = _load()
    c = np.ascontiguousarray(counts, dtype=np.int32)
    off = np.empty(c.size + 1, dtype=np.int32)
    total = lib.oracle_pack_offsets(_ptr(c), c.size, _ptr(off))
    return off, int(total)


def pack_emit(offsets: np.ndarray) -> np.ndarray:
    """Records of every object packed at its offset: object i, record j -> (i+1+j) mod n."""
    lib = _load()
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    n = off.size - 1
    out = np.empty(max(int(off[-1]), 1), dtype=np.int32)
    if n > 0:
        lib.oracle_pack_emit(_ptr(off), n, _ptr(out))
    return out[: int(off[-1])].copy()


def block_size(esize: int, budget: int, explicit: int = 0, default: int = 256) -> int:
    """Block size for elements of esize bytes under a local-memory budget."""
    return int(_load().oracle_block_size(esize, budget, explicit, default))
