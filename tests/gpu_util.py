"""Shared helpers for the GPU parity tests: device transfer and the comparison
rules (bit-exact for integers and for max/min; the stated tolerance for fp
sums; a relative bound for fp products)."""
import numpy as np
import torch

import oracle

DEV = "cuda:0"

# fp32 sums: |gpu - ref| <= 1e-5 * P_i + 1e-6 against the fp64 oracle, with P_i
# the prefix of |x|; fp64 sums: |gpu - ref| <= 1e-12 * P_i.
F32_REL, F32_ABS = 1e-5, 1e-6
F64_REL = 1e-12
# products: a product of k floating-point factors evaluated in any order
# with k - 1 roundings has relative error at most about (k - 1) * u, u the
# unit roundoff of the working precision (every rounding scales the whole
# product); the kernel carries prefixes between tiles in fp64, so this bound
# is loose for it.  Bit-exactness of products is checked separately on
# powers of two, where no rounding occurs.
UNIT_ROUNDOFF = {np.float32: 2.0 ** -24, np.float64: 2.0 ** -53}

TORCH = {np.dtype(np.int32): torch.int32, np.dtype(np.uint32): torch.uint32, np.dtype(np.int64): torch.int64,
         np.dtype(np.float32): torch.float32, np.dtype(np.float64): torch.float64}


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:  # torch has no uint32 <- numpy path on every version
        return torch.from_numpy(a.view(np.int32)).to(DEV).view(torch.uint32)
    return torch.from_numpy(a).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.uint32:
        return t.view(torch.int32).cpu().numpy().view(np.uint32)
    return t.cpu().numpy()


def assert_scan_matches(x: np.ndarray, got: np.ndarray, op: str, exclusive: bool, dims=None, what="", noid=False):
    """Compare a device result with the oracle under the rules above (noid:
    against the oracle's inclusive scan that never uses the identity)."""
    if noid:
        assert not exclusive
        ref = oracle.scan_noid(x, op, dims=dims)
    else:
        ref = oracle.scan(x, op, exclusive=exclusive, dims=dims)
    got = np.asarray(got).reshape(ref.shape)
    if np.issubdtype(x.dtype, np.integer) or op in ("max", "min"):
        if np.issubdtype(x.dtype, np.floating):
            ref = ref.astype(x.dtype)
        bad = np.flatnonzero(got.ravel() != ref.ravel())
        assert bad.size == 0, (f"{what}: {bad.size} mismatches, first at {bad[0]}: "
                               f"got {got.ravel()[bad[0]]} want {ref.ravel()[bad[0]]}")
        return
    g = got.astype(np.float64).ravel()
    r = ref.ravel()
    if op == "sum":
        p = oracle.abs_prefix(x, exclusive=exclusive, dims=dims).ravel()
        if x.dtype == np.float32:
            tol = F32_REL * p + F32_ABS
        else:
            tol = F64_REL * p
    else:  # prod
        length = ref.shape[-1] if dims is None else int(dims[1])
        pos = np.arange(r.size).reshape(-1) if dims is None else \
            np.broadcast_to(np.arange(length)[None, :, None], (int(dims[0]), length, int(dims[2]))).ravel()
        factors = pos + (0 if exclusive else 1)
        tol = 1.01 * factors * UNIT_ROUNDOFF[x.dtype.type] * np.abs(r) + \
            (1e-37 if x.dtype == np.float32 else 1e-300)
    err = np.abs(g - r)
    bad = np.flatnonzero(~(err <= tol))
    assert bad.size == 0, (f"{what}: {bad.size} outside tolerance, worst at "
                           f"{int(np.argmax(err - tol))}: err {err.max():.3e}")


def assert_segscan_matches(x: np.ndarray, off: np.ndarray, got: np.ndarray, op: str, exclusive: bool, what=""):
    """A device segmented scan against the oracle, under the same rules as a
    plain scan with P_i and the product's rounding counted within each
    segment."""
    ref = oracle.scan_segmented(x, off, op, exclusive=exclusive)
    got = np.asarray(got).ravel()
    if np.issubdtype(x.dtype, np.integer) or op in ("max", "min"):
        if np.issubdtype(x.dtype, np.floating):
            ref = ref.astype(x.dtype)
        bad = np.flatnonzero(got != ref)
        assert bad.size == 0, (f"{what}: {bad.size} mismatches, first at {bad[0]}: "
                               f"got {got[bad[0]]} want {ref[bad[0]]}")
        return
    g = got.astype(np.float64)
    if op == "sum":
        p = oracle.segment_abs_prefix(x, off, exclusive=exclusive)
        tol = F32_REL * p + F32_ABS if x.dtype == np.float32 else F64_REL * p
    else:  # prod: one rounding per factor within the segment
        start = np.repeat(off[:-1].astype(np.int64), np.diff(off.astype(np.int64)))
        factors = np.arange(x.size) - start + (0 if exclusive else 1)
        tol = 1.01 * factors * UNIT_ROUNDOFF[x.dtype.type] * np.abs(ref) + \
            (1e-37 if x.dtype == np.float32 else 1e-300)
    err = np.abs(g - ref)
    bad = np.flatnonzero(~(err <= tol))
    assert bad.size == 0, (f"{what}: {bad.size} outside tolerance, worst at "
                           f"{int(np.argmax(err - tol))}: err {err.max():.3e}")
