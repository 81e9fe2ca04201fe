"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers (numpy PCG64 via default_rng); it holds
none of the scan, compaction or packing arithmetic, and imports neither the
HIP binding nor the oracle.  The workloads stand in for the arrays the pages
time (synthetic arrays only; no dataset is involved):

  int32 scans   integers uniform in [0, 100] (both ends included), seed 0
  fp32 scans    uniform [0, 1) float32 (multiples of 2^-24), seed 1
  fp64 scans    uniform [-1, 1) float64 (multiples of 2^-52), seed 1
  2-D scans     uniform [0, 1) float32, seed 3, drawn in the order
                4096x4096, 1e6x8, 2x1e7
  compaction    uniform [0, 1) float32 of 1e7, then Poisson(3) int32 counts
                of 1e7, seed 4
  structs       uniform [-1, 1) 17 x fp64 per element, then 24 x fp32 per
                element as 2*u - 1 (exact, multiples of 2^-23), seed 5
  segments      the compaction draw's Poisson(3) counts as segment lengths,
                then one uniform [0, 1) float32 value per record, seed 4

Each generator takes the element count so the tests can draw smaller arrays
of the same distribution.
"""
from __future__ import annotations

import numpy as np


def int32_uniform_0_100(n: int = 2 ** 20, seed: int = 0) -> np.ndarray:
    return np.random.default_rng(seed).integers(0, 101, n, dtype=np.int32)


def f32_uniform_01(n: int = 10 ** 8, seed: int = 1) -> np.ndarray:
    return np.random.default_rng(seed).random(n, dtype=np.float32)


def f64_uniform_pm1(n: int = 10 ** 7, seed: int = 1) -> np.ndarray:
    return np.random.default_rng(seed).uniform(-1.0, 1.0, n)


def dims_arrays(seed: int = 3, square: int = 4096, tall=(10 ** 6, 8), wide=(2, 10 ** 7)):
    """(square x square, tall, wide) float32 arrays drawn in that order."""
    rng = np.random.default_rng(seed)
    a = rng.random((square, square), dtype=np.float32)
    b = rng.random(tall, dtype=np.float32)
    c = rng.random(wide, dtype=np.float32)
    return a, b, c


def compaction_inputs(n: int = 10 ** 7, seed: int = 4, lam: float = 3.0):
    """(x float32 uniform [0,1), counts int32 Poisson(lam)) drawn in that order."""
    rng = np.random.default_rng(seed)
    x = rng.random(n, dtype=np.float32)
    counts = rng.poisson(lam, n).astype(np.int32)
    return x, counts


def struct_inputs(n: int = 10 ** 6, seed: int = 5, w64: int = 17, w32: int = 24):
    """(n x w64 float64 in [-1,1), n x w32 float32 in [-1,1)) drawn in that order."""
    rng = np.random.default_rng(seed)
    s64 = rng.uniform(-1.0, 1.0, (n, w64))
    s32 = (np.float32(2.0) * rng.random((n, w32), dtype=np.float32) - np.float32(1.0)).astype(np.float32)
    return s64, s32


def generic(dtype, n: int, seed: int, kind: str = "default") -> np.ndarray:
    """Small arrays for parity sweeps: values chosen per dtype so that sums stay
    exactly representable where the tests rely on it."""
    rng = np.random.default_rng(seed)
    dt = np.dtype(dtype)
    if dt == np.int32:
        if kind == "wide":
            return rng.integers(-2 ** 31, 2 ** 31, n, dtype=np.int64).astype(np.int32)
        return rng.integers(-100, 101, n, dtype=np.int32)
    if dt == np.uint32:
        if kind == "wide":
            return rng.integers(0, 2 ** 32, n, dtype=np.uint64).astype(np.uint32)
        return rng.integers(0, 101, n, dtype=np.uint32)
    if dt == np.int64:
        if kind == "wide":
            return rng.integers(-2 ** 63, 2 ** 63 - 1, n, dtype=np.int64)
        return rng.integers(-10 ** 6, 10 ** 6 + 1, n, dtype=np.int64)
    if dt == np.float32:
        if kind == "near1":
            return (np.float32(0.999) + np.float32(0.002) * rng.random(n, dtype=np.float32)).astype(np.float32)
        return (np.float32(2.0) * rng.random(n, dtype=np.float32) - np.float32(1.0)).astype(np.float32)
    if dt == np.float64:
        if kind == "near1":
            return 0.999 + 0.002 * rng.random(n)
        return rng.uniform(-1.0, 1.0, n)
    raise TypeError(dt)


def segmented_inputs(nseg: int = 10 ** 7, seed: int = 4, lam: float = 3.0):
    """(counts int32, values float32): the Poisson(lam) counts of
    compaction_inputs(nseg, seed) as segment lengths, then one uniform [0, 1)
    value per record, drawn next from the same generator."""
    rng = np.random.default_rng(seed)
    rng.random(nseg, dtype=np.float32)  # the compaction draw comes first
    counts = rng.poisson(lam, nseg).astype(np.int32)
    values = rng.random(int(counts.sum(dtype=np.int64)), dtype=np.float32)
    return counts, values
