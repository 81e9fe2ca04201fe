"""Pins for the CPU oracle (runs without a GPU).

Each check ties the oracle to something other than itself: the worked examples
printed on the pages (tests/golden/), closed forms, brute force from the
definition on tiny inputs, invariants, independent numpy routines, and an exact
integer shadow of the floating-point scans.
"""
from fractions import Fraction
from itertools import accumulate

import numpy as np
import pytest

from conftest import read_golden, read_golden_table
from stream_compaction_wave64_amd import inputs

INT_TYPES = [np.int32, np.uint32, np.int64]
ALL_TYPES = INT_TYPES + [np.float32, np.float64]
OPS = ["sum", "prod", "max", "min"]


def _bits(dt):
    return np.dtype(dt).itemsize * 8


def _wrap(v, dt):
    """Python int -> value of integer dtype dt with two's-complement wrap."""
    b = _bits(dt)
    v %= 1 << b
    if np.issubdtype(dt, np.signedinteger) and v >= 1 << (b - 1):
        v -= 1 << b
    return v


def _identity(op, dt):
    if op == "sum":
        return 0
    if op == "prod":
        return 1
    if np.issubdtype(dt, np.integer):
        info = np.iinfo(dt)
        return info.min if op == "max" else info.max
    return -np.inf if op == "max" else np.inf


def _brute(x, op, exclusive, dt):
    """O(n^2) scan straight from the definition, in exact arithmetic."""
    n = len(x)
    out = []
    is_int = np.issubdtype(dt, np.integer)
    for i in range(n):
        terms = x[:i] if exclusive else x[: i + 1]
        if is_int:
            vals = [int(v) for v in terms]
        else:
            vals = [Fraction(float(v)) for v in terms]
        if not vals:
            r = _identity(op, dt)
        elif op == "sum":
            r = sum(vals)
        elif op == "prod":
            r = 1
            for v in vals:
                r *= v
        elif op == "max":
            r = max(vals)
        else:
            r = min(vals)
        if is_int:
            out.append(_wrap(int(r), dt))
        else:
            out.append(float(r))
    return out


# ------------------------------------------------------------ golden examples


@pytest.mark.parametrize("dt", ALL_TYPES)
def test_merry_prefix_sum_example(oracle_lib, dt):
    g = read_golden("merry_prefix_sum_example.txt")
    x = np.array(g["input"], dtype=dt)
    assert list(oracle_lib.scan(x, "sum")) == g["inclusive"]
    assert list(oracle_lib.scan(x, "sum", exclusive=True)) == g["exclusive"]


@pytest.mark.parametrize("dt", ALL_TYPES)
def test_merry_kogge_stone_states(oracle_lib, dt):
    # The state after the round of stride t is the sum of the 2t inputs ending at
    # i, i.e. incl[i] - incl[i - 2t]; the printed rows pin the oracle's scan.
    g = read_golden("merry_kogge_stone_example.txt")
    x = np.array(g["input"], dtype=dt)
    incl = [int(v) for v in oracle_lib.scan(x, "sum")]
    for t, key in ((1, "stride1"), (2, "stride2"), (4, "stride4")):
        window = [incl[i] - (incl[i - 2 * t] if i - 2 * t >= 0 else 0) for i in range(len(x))]
        assert window == g[key], key
    assert incl == g["stride4"]


@pytest.mark.parametrize("dt", ALL_TYPES)
def test_merry_brent_kung_example(oracle_lib, dt):
    g = read_golden("merry_brent_kung_example.txt")
    x = np.array(g["input"], dtype=dt)
    incl = [int(v) for v in oracle_lib.scan(x, "sum")]
    excl = [int(v) for v in oracle_lib.scan(x, "sum", exclusive=True)]
    assert excl == g["exclusive"]
    pairs = [incl[2 * i + 1] - (incl[2 * i - 1] if i else 0) for i in range(4)]
    quads = [incl[4 * i + 3] - (incl[4 * i - 1] if i else 0) for i in range(2)]
    assert pairs == g["pairs"] and quads == g["quads"] and incl[-1] == g["total"][0]


@pytest.mark.parametrize("dt", ALL_TYPES)
def test_merry_radix4_example(oracle_lib, dt):
    g = read_golden("merry_radix4_example.txt")
    x = np.array(g["input"], dtype=dt)
    incl = [int(v) for v in oracle_lib.scan(x, "sum")]
    excl = [int(v) for v in oracle_lib.scan(x, "sum", exclusive=True)]
    assert incl == g["inclusive"]
    assert [incl[4 * b + 3] - excl[4 * b] for b in range(4)] == g["blocksums"]
    assert [excl[4 * b] for b in range(4)] == g["bases"]
    assert incl[-1] == g["total"][0]
    # scanning the block sums gives the same bases (the tree's recursion step)
    bs = np.array(g["blocksums"], dtype=dt)
    assert [int(v) for v in oracle_lib.scan(bs, "sum", exclusive=True)] == g["bases"]


def test_merry_output_packing_example(oracle_lib):
    g = read_golden("merry_output_packing_example.txt")
    off, total = oracle_lib.pack_offsets(np.array(g["counts"], dtype=np.int32))
    assert list(off) == g["offsets"] and total == g["offsets"][-1]
    n = len(g["counts"])
    rec = oracle_lib.pack_emit(off)
    expect = [(o + 1 + r) % n for o, r in zip(g["owner"], g["rank"])]
    assert list(rec) == expect


def test_pr208_block_size_rule(oracle_lib):
    for esize, budget, explicit, default, expected in read_golden_table("pr208_block_size_rule.txt"):
        assert oracle_lib.block_size(esize, budget, explicit, default) == expected, (esize, budget)


# ------------------------------------------------------------- closed forms


@pytest.mark.parametrize("dt", ALL_TYPES)
def test_all_ones_gives_i_plus_1(oracle_lib, dt):
    n = 5000
    y = oracle_lib.scan(np.ones(n, dtype=dt), "sum")
    assert np.array_equal(y, np.arange(1, n + 1))
    y = oracle_lib.scan(np.ones(n, dtype=dt), "sum", exclusive=True)
    assert np.array_equal(y, np.arange(0, n))


def test_iota_gives_triangular_int32_wraps(oracle_lib):
    n = 100_000  # beyond i = 65535 the int32 triangle wraps mod 2^32
    y = oracle_lib.scan(np.arange(n, dtype=np.int32), "sum")
    i = np.arange(n, dtype=np.int64)
    expect = ((i * (i + 1) // 2) % (1 << 32)).astype(np.uint32).view(np.int32)
    assert np.array_equal(y, expect)


@pytest.mark.parametrize("dt", [np.int64, np.float32, np.float64])
def test_iota_gives_triangular(oracle_lib, dt):
    n = 5793 if dt == np.float32 else 100_000  # fp32 inputs/outputs exact up to i=5792
    y = oracle_lib.scan(np.arange(n, dtype=dt), "sum")
    i = np.arange(n, dtype=np.int64)
    assert np.array_equal(y, i * (i + 1) // 2)


@pytest.mark.parametrize("dt", ALL_TYPES)
def test_constant_and_extrema_closed_forms(oracle_lib, dt):
    n = 777
    c = 3
    assert np.array_equal(oracle_lib.scan(np.full(n, c, dtype=dt), "sum"), c * np.arange(1, n + 1))
    iota = np.arange(n, dtype=dt)
    assert np.array_equal(oracle_lib.scan(iota, "max"), np.arange(n))
    assert np.array_equal(oracle_lib.scan(iota[::-1].copy(), "min"), np.arange(n)[::-1])
    assert np.all(oracle_lib.scan(iota, "min") == 0)
    ex = oracle_lib.scan(iota, "max", exclusive=True)
    assert ex[0] == _identity("max", dt) and np.array_equal(ex[1:], np.arange(n - 1))


def test_prod_powers_of_two_wrap(oracle_lib):
    y = oracle_lib.scan(np.full(40, 2, dtype=np.int32), "prod")
    expect = [_wrap(2 ** (i + 1), np.int32) for i in range(40)]
    assert list(y) == expect
    y = oracle_lib.scan(np.full(40, 2, dtype=np.float64), "prod")
    assert list(y) == [2.0 ** (i + 1) for i in range(40)]


# ----------------------------------------------------------- brute force


@pytest.mark.parametrize("dt", ALL_TYPES)
@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("n", [1, 2, 3, 7, 64, 65, 127, 300])
def test_brute_force_small(oracle_lib, dt, op, n):
    rng = np.random.default_rng(1000 + n)
    if np.issubdtype(dt, np.integer):
        info = np.iinfo(dt)
        x = rng.integers(max(info.min, -2 ** 62), min(info.max, 2 ** 62), n, dtype=np.int64)
        x = x.astype(dt) if dt != np.uint32 else (x % (1 << 32)).astype(np.uint32)
    else:
        # dyadic values so the exact prefix of sums is representable; prod uses
        # values near 1 and is compared after exact rounding below
        x = (rng.integers(-64, 65, n) / 16.0).astype(dt)
        if op == "prod":
            x = (1.0 + rng.integers(-8, 9, n) / 1024.0).astype(dt)
    for excl in (False, True):
        got = oracle_lib.scan(x, op, exclusive=excl)
        exp = _brute(x, op, excl, dt)
        if np.issubdtype(dt, np.integer) or op != "prod":
            assert list(got) == exp, (op, excl)
        else:
            # products of n dyadic factors are not representable: the oracle is
            # within its accumulator's rounding of the exact value
            rel = 2.0 ** -50 if dt == np.float32 else 2.0 ** -100
            for g, e in zip(got, exp):
                assert abs(g - e) <= rel * n * abs(e) + 1e-300


# ------------------------------------- inclusive scans without a neutral element
# AcceleratedKernels.jl PR #208, description, first bullet: operators with no
# neutral element keep Optional partials.  The oracle's scan_noid starts each
# column from its first element and never forms an identity.


@pytest.mark.parametrize("dt", ALL_TYPES, ids=lambda d: np.dtype(d).name)
@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("n", [1, 2, 3, 17, 64])
def test_noid_brute_force_small(oracle_lib, dt, op, n):
    rng = np.random.default_rng(2000 + n)
    if np.issubdtype(dt, np.integer):
        info = np.iinfo(dt)
        x = rng.integers(max(info.min, -2 ** 62), min(info.max, 2 ** 62), n, dtype=np.int64)
        x = x.astype(dt) if dt != np.uint32 else (x % (1 << 32)).astype(np.uint32)
    else:
        x = (rng.integers(-64, 65, n) / 16.0).astype(dt)
        if op == "prod":
            x = (1.0 + rng.integers(-8, 9, n) / 1024.0).astype(dt)
    got = oracle_lib.scan_noid(x, op)
    exp = _brute(x, op, False, dt)  # inclusive: every term is an input, no identity involved
    if np.issubdtype(dt, np.integer) or op != "prod":
        assert list(got) == exp
    else:
        rel = 2.0 ** -50 if dt == np.float32 else 2.0 ** -100
        for g, e in zip(got, exp):
            assert abs(g - e) <= rel * n * abs(e)


@pytest.mark.parametrize("dt", ALL_TYPES, ids=lambda d: np.dtype(d).name)
@pytest.mark.parametrize("op", OPS)
def test_noid_equals_identity_scan_inclusive(oracle_lib, dt, op):
    # with no signed zero in the data, combining the identity first changes
    # nothing: both scans must agree bit for bit, 1-D and along a middle axis
    kind = "near1" if op == "prod" and np.issubdtype(dt, np.floating) else "wide"
    x = inputs.generic(dt, 3 * 257 * 5, 31, kind)
    if np.issubdtype(dt, np.floating):
        x[x == 0] = 1
    a, b = oracle_lib.scan_noid(x, op), oracle_lib.scan(x, op)
    assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    d = (3, 257, 5)
    a, b = oracle_lib.scan_noid(x, op, dims=d), oracle_lib.scan(x, op, dims=d)
    assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("dt", [np.float32, np.float64])
def test_noid_keeps_negative_zero(oracle_lib, dt):
    # IEEE addition: -0.0 + -0.0 = -0.0, but 0.0 + -0.0 = +0.0.  A scan of
    # negative zeros that never uses the identity stays -0.0 everywhere; one
    # that starts from the identity 0.0 is +0.0 everywhere.
    z = np.full(100, -0.0, dtype=dt)
    got = oracle_lib.scan_noid(z, "sum")
    assert np.all(got == 0) and np.all(np.signbit(got))
    ident = oracle_lib.scan(z, "sum")
    assert np.all(ident == 0) and not np.any(np.signbit(ident))
    x = np.array([-0.0, 1.5, -1.5, 2.0], dtype=dt)
    got = oracle_lib.scan_noid(x, "sum")
    assert np.signbit(got[0]) and list(got) == [0.0, 1.5, 0.0, 2.0]
    # products: -0.0 * 2 = -0.0 and 1 * -0.0 = -0.0, with or without the identity
    p = np.array([-0.0, 2.0, 3.0], dtype=dt)
    for r in (oracle_lib.scan_noid(p, "prod"), oracle_lib.scan(p, "prod")):
        assert np.all(r == 0) and np.all(np.signbit(r))
    # along the middle axis: each of the 6 columns starts from its own -0.0
    got = oracle_lib.scan_noid(np.full((2, 50, 3), -0.0, dtype=dt), "sum", dims=(2, 50, 3))
    assert np.all(np.signbit(got))


# ----------------------------------------------------- independent routines


def test_matches_numpy_accumulate_int32(oracle_lib):
    x = inputs.int32_uniform_0_100(2 ** 20, seed=0)
    assert np.array_equal(oracle_lib.scan(x, "sum"), np.cumsum(x, dtype=np.int32))
    w = inputs.generic(np.int32, 100_000, 7, "wide")
    assert np.array_equal(oracle_lib.scan(w, "sum"), np.cumsum(w, dtype=np.int32))
    assert np.array_equal(oracle_lib.scan(w, "max"), np.maximum.accumulate(w))
    assert np.array_equal(oracle_lib.scan(w, "min"), np.minimum.accumulate(w))
    assert np.array_equal(oracle_lib.scan(w, "prod"), np.multiply.accumulate(w, dtype=np.int32))


def test_matches_numpy_accumulate_u32_i64(oracle_lib):
    u = inputs.generic(np.uint32, 50_000, 8, "wide")
    assert np.array_equal(oracle_lib.scan(u, "sum"), np.cumsum(u, dtype=np.uint32))
    assert np.array_equal(oracle_lib.scan(u, "max"), np.maximum.accumulate(u))
    assert np.array_equal(oracle_lib.scan(u, "min"), np.minimum.accumulate(u))
    v = inputs.generic(np.int64, 50_000, 9, "wide")
    with np.errstate(over="ignore"):
        assert np.array_equal(oracle_lib.scan(v, "sum"), np.cumsum(v, dtype=np.int64))
        assert np.array_equal(oracle_lib.scan(v, "prod"), np.multiply.accumulate(v, dtype=np.int64))


def test_float_max_min_match_numpy_exactly(oracle_lib):
    x = inputs.generic(np.float32, 10_000, 3)
    assert np.array_equal(oracle_lib.scan(x, "max"), np.maximum.accumulate(x).astype(np.float64))
    y = inputs.generic(np.float64, 10_000, 4)
    assert np.array_equal(oracle_lib.scan(y, "min"), np.minimum.accumulate(y))


# ----------------------------------------------------------------- invariants


@pytest.mark.parametrize("dt", INT_TYPES)
def test_scan_invariants_int(oracle_lib, dt):
    x = inputs.generic(dt, 20_000, 11, "wide")
    inc = oracle_lib.scan(x, "sum")
    exc = oracle_lib.scan(x, "sum", exclusive=True)
    with np.errstate(over="ignore"):
        assert np.array_equal(exc[1:], inc[:-1])
        assert exc[0] == 0
        assert np.array_equal((inc - exc).astype(dt), x)
        assert inc[-1] == np.sum(x, dtype=dt)


def test_scan_invariants_float(oracle_lib):
    x = inputs.f32_uniform_01(100_000, seed=1)
    inc = oracle_lib.scan(x, "sum")
    exc = oracle_lib.scan(x, "sum", exclusive=True)
    assert np.array_equal(exc[1:], inc[:-1]) and exc[0] == 0.0
    assert np.array_equal(inc - exc, x.astype(np.float64))  # exact on the 2^-24 grid
    assert np.all(np.diff(inc) >= 0)
    p = oracle_lib.abs_prefix(x)
    assert np.array_equal(p, inc)  # non-negative inputs: P_i equals the prefix
    pe = oracle_lib.abs_prefix(x, exclusive=True)
    assert np.array_equal(pe, exc)
    m = oracle_lib.scan(x, "max")
    assert np.all(np.diff(m) >= 0) and np.all(m >= x)


# ------------------------------------------- tolerance weights, signed inputs
# P_i = sum of |x_j| over the inputs output i depends on scales every fp
# tolerance, so it is pinned on signed data, where a dropped absolute value
# or a swapped inclusive/exclusive form changes the result.


@pytest.mark.parametrize("dt", [np.float32, np.float64])
def test_abs_prefix_alternating_signs_closed_form(oracle_lib, dt):
    # +1, -1, +1, ...: the prefix alternates 1, 0, 1, ... while P_i = i + 1
    # (inclusive) and i (exclusive), exactly.
    n = 1001
    x = np.where(np.arange(n) % 2 == 0, 1.0, -1.0).astype(dt)
    i = np.arange(n, dtype=np.float64)
    assert np.array_equal(oracle_lib.abs_prefix(x), i + 1)
    assert np.array_equal(oracle_lib.abs_prefix(x, exclusive=True), i)
    # the scan itself cancels: the weight is what keeps the tolerance honest
    assert np.array_equal(oracle_lib.scan(x, "sum"), (i % 2 == 0).astype(np.float64))


@pytest.mark.parametrize("dt,q", [(np.float32, 23), (np.float64, 30)])
@pytest.mark.parametrize("exclusive", [False, True])
def test_abs_prefix_signed_integer_shadow(oracle_lib, dt, q, exclusive):
    # signed values on the 2^-q grid: |x_j| * 2^q are integers whose int64
    # prefix is exact, and every partial sum stays below 2^53, so the
    # oracle's fp64 accumulation must reproduce it bit for bit
    rng = np.random.default_rng(7)
    k = rng.integers(-(2 ** q), 2 ** q, 50_000, dtype=np.int64)
    x = (k.astype(np.float64) * 2.0 ** -q).astype(dt)
    assert np.array_equal(x.astype(np.float64) * 2.0 ** q, k.astype(np.float64))
    a = np.abs(k)
    shadow = np.cumsum(a) - (a if exclusive else 0)
    assert np.array_equal(oracle_lib.abs_prefix(x, exclusive=exclusive), shadow.astype(np.float64) * 2.0 ** -q)


@pytest.mark.parametrize("dt,q", [(np.float32, 23), (np.float64, 30)])
@pytest.mark.parametrize("exclusive", [False, True])
def test_abs_prefix_signed_dims(oracle_lib, dt, q, exclusive):
    # (outer, len, inner) = (3, 257, 5): each of the 15 columns along the
    # middle axis gets its own weight, exact on the grid
    rng = np.random.default_rng(8)
    k = rng.integers(-(2 ** q), 2 ** q, (3, 257, 5), dtype=np.int64)
    x = (k.astype(np.float64) * 2.0 ** -q).astype(dt)
    a = np.abs(k)
    shadow = np.cumsum(a, axis=1) - (a if exclusive else 0)
    got = oracle_lib.abs_prefix(x, exclusive=exclusive, dims=(3, 257, 5))
    assert np.array_equal(got, shadow.astype(np.float64) * 2.0 ** -q)


# ------------------------------------------------------- exact integer shadow


def test_fp32_exact_integer_shadow(oracle_lib):
    # values on the 2^-24 grid: k_i = x_i * 2^24 are integers and their int64
    # prefix is exact; the fp64 accumulation must reproduce it bit for bit.
    x = inputs.f32_uniform_01(10 ** 7, seed=1)
    k = (x.astype(np.float64) * 2.0 ** 24).astype(np.int64)
    assert np.array_equal(k.astype(np.float64) / 2.0 ** 24, x.astype(np.float64))
    exact = np.cumsum(k, dtype=np.int64)
    assert int(exact[-1]) < 2 ** 53
    got = oracle_lib.scan(x, "sum")
    assert np.array_equal(got, exact.astype(np.float64) / 2.0 ** 24)


def test_fp64_exact_integer_shadow(oracle_lib):
    # values on the 2^-52 grid; the exact prefix (Python integers) rounded once
    # to double must equal the oracle's double-double result rounded to double.
    x = inputs.f64_uniform_pm1(40_000, seed=1)
    k = [int(v * 2.0 ** 52) for v in x]
    assert all(kk / 2.0 ** 52 == v for kk, v in zip(k[:1000], x[:1000]))
    exact = list(accumulate(k))
    expect = np.array([e / 2 ** 52 for e in exact])  # int / int is correctly rounded
    got = oracle_lib.scan(x, "sum")
    assert np.array_equal(got, expect)
    # the same inputs all positive: |prefix| grows and the rounding still matches
    xa = np.abs(x)
    ka = [abs(kk) for kk in k]
    expect = np.array([e / 2 ** 52 for e in accumulate(ka)])
    assert np.array_equal(oracle_lib.scan(xa, "sum"), expect)


# ------------------------------------------------------------------- dims


@pytest.mark.parametrize("dt", [np.int32, np.float32])
def test_dims_layouts_agree(oracle_lib, dt):
    rng = np.random.default_rng(5)
    a = (rng.integers(0, 50, (37, 53))).astype(dt)
    # along rows (contiguous) == 1-D scans of each row
    rows = oracle_lib.scan(a.ravel(), "sum", dims=(37, 53, 1)).reshape(37, 53)
    for r in range(37):
        assert np.array_equal(rows[r], oracle_lib.scan(a[r].copy(), "sum"))
    # along columns (stride 53) == row scans of the transpose, transposed back
    cols = oracle_lib.scan(a.ravel(), "sum", dims=(1, 37, 53)).reshape(37, 53)
    t = oracle_lib.scan(a.T.copy().ravel(), "sum", dims=(53, 37, 1)).reshape(53, 37).T
    assert np.array_equal(cols, t)
    assert np.array_equal(cols, np.cumsum(a, axis=0, dtype=np.float64 if dt == np.float32 else np.int32))
    # 3-D: (outer, len, inner)
    b = rng.integers(0, 9, (4, 6, 5)).astype(dt)
    got = oracle_lib.scan(b.ravel(), "sum", dims=(4, 6, 5)).reshape(4, 6, 5)
    assert np.array_equal(got, np.cumsum(b, axis=1, dtype=np.float64 if dt == np.float32 else np.int32))


# ------------------------------------------------------------- compaction


def test_compaction_brute_and_numpy(oracle_lib):
    x, _ = inputs.compaction_inputs(200_000, seed=4)
    idx = oracle_lib.compact(x, "gt", 0.5)
    assert np.array_equal(idx, np.flatnonzero(x > np.float32(0.5)).astype(np.int32))
    small = x[:300]
    assert list(oracle_lib.compact(small, "gt", 0.5)) == [i for i in range(300) if small[i] > 0.5]
    assert np.all(np.diff(idx) > 0) and np.all(x[idx] > 0.5)
    rest = np.setdiff1d(np.arange(x.size), idx)
    assert np.all(x[rest] <= 0.5)
    for cmp, fn in (("ge", np.greater_equal), ("lt", np.less), ("le", np.less_equal),
                    ("eq", np.equal), ("ne", np.not_equal)):
        assert np.array_equal(oracle_lib.compact(x, cmp, 0.5), np.flatnonzero(fn(x, np.float32(0.5))))


def test_compaction_closed_forms(oracle_lib):
    n = 1001
    assert np.array_equal(oracle_lib.compact(np.ones(n, np.float32), "gt", 0.5), np.arange(n))
    assert oracle_lib.compact(np.zeros(n, np.float32), "gt", 0.5).size == 0
    alt = np.tile(np.array([0.0, 1.0], np.float32), n)
    assert np.array_equal(oracle_lib.compact(alt, "gt", 0.5), 2 * np.arange(n) + 1)
    ties = np.full(10, 0.5, np.float32)
    assert oracle_lib.compact(ties, "gt", 0.5).size == 0 and oracle_lib.compact(ties, "ge", 0.5).size == 10
    xi = np.arange(-5, 6, dtype=np.int32)
    assert list(oracle_lib.compact(xi, "gt", 0)) == list(range(6, 11))


def test_compaction_special_floats(oracle_lib):
    # IEEE 754 comparisons: an unordered operand (NaN) makes every relation
    # false except "not equal"; -0.0 == +0.0; infinities are ordered.
    x = np.array([np.nan, -0.0, 0.0, np.inf, -np.inf, 0.5, np.nan], np.float32)
    assert list(oracle_lib.compact(x, "gt", 0.0)) == [3, 5]
    assert list(oracle_lib.compact(x, "ge", 0.0)) == [1, 2, 3, 5]
    assert list(oracle_lib.compact(x, "lt", 0.0)) == [4]
    assert list(oracle_lib.compact(x, "le", 0.0)) == [1, 2, 4]
    assert list(oracle_lib.compact(x, "eq", 0.0)) == [1, 2]
    assert list(oracle_lib.compact(x, "ne", 0.0)) == [0, 3, 4, 5, 6]
    assert list(oracle_lib.compact(x, "lt", np.inf)) == [1, 2, 4, 5]
    vals, idx, k = oracle_lib.partition(x, "ne", 0.0)
    assert k == 5 and list(idx) == [0, 3, 4, 5, 6, 1, 2]
    assert np.array_equal(vals.view(np.uint32), x[idx].view(np.uint32))  # raw bits move, NaNs included


def test_compaction_bit_predicates(oracle_lib):
    keys = np.arange(64, dtype=np.uint32)
    for b in range(6):
        assert np.array_equal(oracle_lib.compact(keys, "bit_set", b), np.flatnonzero((keys >> b) & 1))
        assert np.array_equal(oracle_lib.compact(keys, "bit_clear", b), np.flatnonzero(((keys >> b) & 1) == 0))
    neg = np.array([-1, 0, 5, -8], np.int32)  # bit 31 is the sign bit
    assert list(oracle_lib.compact(neg, "bit_set", 31)) == [0, 3]


# ------------------------------------------------------------- partition


def _check_partition(x, pred, vals, idx, k):
    """Stable partition by the boolean mask `pred` (True first)."""
    n = x.size
    assert k == int(pred.sum())
    assert np.array_equal(np.sort(idx), np.arange(n))           # a permutation
    assert np.array_equal(vals, x[idx])                           # values follow indices
    assert pred[idx[:k]].all() and not pred[idx[k:]].any()        # the split
    assert np.all(np.diff(idx[:k]) > 0) and np.all(np.diff(idx[k:]) > 0)  # each part in order


def test_partition_invariants(oracle_lib):
    x, _ = inputs.compaction_inputs(50_000, seed=6)
    for cmp, fn in (("gt", np.greater), ("le", np.less_equal), ("eq", np.equal)):
        vals, idx, k = oracle_lib.partition(x, cmp, 0.5)
        _check_partition(x, fn(x, np.float32(0.5)), vals, idx, k)
    rng = np.random.default_rng(7)
    xi = rng.integers(-1000, 1000, 30_000).astype(np.int32)
    vals, idx, k = oracle_lib.partition(xi, "lt", 17)
    _check_partition(xi, xi < 17, vals, idx, k)
    keys = rng.integers(0, 2 ** 32, 30_000, dtype=np.uint64).astype(np.uint32)
    for b in (0, 13, 31):
        vals, idx, k = oracle_lib.partition(keys, "bit_clear", b)
        _check_partition(keys, ((keys >> np.uint32(b)) & 1) == 0, vals, idx, k)
    # small: brute force
    small = x[:200]
    vals, idx, k = oracle_lib.partition(small, "gt", 0.5)
    want = [i for i in range(200) if small[i] > 0.5] + [i for i in range(200) if not small[i] > 0.5]
    assert list(idx) == want and k == sum(1 for v in small if v > 0.5)


def test_partition_closed_forms(oracle_lib):
    n = 1001
    for x, k_want in ((np.ones(n, np.float32), n), (np.zeros(n, np.float32), 0)):
        vals, idx, k = oracle_lib.partition(x, "gt", 0.5)
        assert k == k_want and np.array_equal(idx, np.arange(n)) and np.array_equal(vals, x)
    alt = np.tile(np.array([0.0, 1.0], np.float32), n)
    vals, idx, k = oracle_lib.partition(alt, "gt", 0.5)
    assert k == n
    assert np.array_equal(idx, np.concatenate([2 * np.arange(n) + 1, 2 * np.arange(n)]))
    assert np.array_equal(vals, np.concatenate([np.ones(n, np.float32), np.zeros(n, np.float32)]))


def test_radix_sort_from_stable_bit_partitions(oracle_lib):
    # LSD radix sort is repeated stable partitioning by one-bit digits: the
    # composed permutation must be numpy's stable argsort
    rng = np.random.default_rng(8)
    keys = rng.integers(0, 2 ** 32, 5000, dtype=np.uint64).astype(np.uint32)
    keys[::7] = keys[3]                                           # many equal keys
    cur, perm = keys.copy(), np.arange(keys.size)
    for b in range(32):
        cur, idx, _ = oracle_lib.partition(cur, "bit_clear", b)
        perm = perm[idx]
    assert np.array_equal(cur, np.sort(keys))
    assert np.array_equal(perm, np.argsort(keys, kind="stable"))
    # signed keys: the sign bit's pass puts set bits (negatives) first
    sk = rng.integers(-2 ** 31, 2 ** 31, 5000, dtype=np.int64).astype(np.int32)
    cur, perm = sk.copy(), np.arange(sk.size)
    for b in range(32):
        cur, idx, _ = oracle_lib.partition(cur, "bit_set" if b == 31 else "bit_clear", b)
        perm = perm[idx]
    assert np.array_equal(cur, np.sort(sk)) and np.array_equal(perm, np.argsort(sk, kind="stable"))


# ------------------------------------------------------- segmented scan


def test_segmented_packing_example(oracle_lib):
    g = read_golden("segmented_scan_packing_example.txt")
    off = np.array(g["offsets"], np.int32)
    for dt in (np.int32, np.int64, np.float32, np.float64):
        x = np.array(g["values"], dt)
        assert list(oracle_lib.scan_segmented(x, off, "sum")) == g["incl_sum"]
        assert list(oracle_lib.scan_segmented(x, off, "sum", exclusive=True)) == g["excl_sum"]
        assert list(oracle_lib.scan_segmented(x, off, "max")) == g["incl_max"]
        assert list(oracle_lib.scan_segmented(x, off, "prod")) == g["incl_prod"]


def _random_offsets(rng, n, mean):
    lens = rng.poisson(mean, n)                          # includes empty segments
    off = np.concatenate([[0], np.cumsum(lens)])
    off = off[off <= n]
    return np.concatenate([off, [n]]).astype(np.int32)


def test_segmented_brute_force(oracle_lib):
    rng = np.random.default_rng(60)
    for n, mean in ((1, 1.0), (37, 2.0), (200, 5.0), (300, 0.7)):
        x = rng.integers(-9, 10, n).astype(np.int64)
        off = _random_offsets(rng, n, mean)
        seg = np.repeat(np.arange(off.size - 1), np.diff(off))
        for op, f, ident in (("sum", lambda a, b: a + b, 0), ("max", max, np.iinfo(np.int64).min)):
            incl = oracle_lib.scan_segmented(x, off, op)
            excl = oracle_lib.scan_segmented(x, off, op, exclusive=True)
            for i in range(n):
                acc = ident
                for j in range(off[seg[i]], i):
                    acc = f(acc, x[j])
                assert excl[i] == acc
                assert incl[i] == f(acc, x[i])


def test_segmented_closed_forms_and_invariants(oracle_lib):
    rng = np.random.default_rng(61)
    n = 50_000
    off = _random_offsets(rng, n, 6.0)
    start = np.repeat(off[:-1], np.diff(off))
    ones = np.ones(n, np.int32)
    assert np.array_equal(oracle_lib.scan_segmented(ones, off, "sum"), np.arange(n) - start + 1)
    assert np.array_equal(oracle_lib.scan_segmented(ones, off, "sum", exclusive=True), np.arange(n) - start)
    x = rng.random(n, dtype=np.float32)
    # one segment is the plain scan; one-element segments return x (identity when exclusive)
    assert np.array_equal(oracle_lib.scan_segmented(x, np.array([0, n], np.int32), "sum"), oracle_lib.scan(x))
    each = np.arange(n + 1, dtype=np.int32)
    assert np.array_equal(oracle_lib.scan_segmented(x, each, "sum"), x.astype(np.float64))
    assert not oracle_lib.scan_segmented(x, each, "sum", exclusive=True).any()
    # empty segments change nothing
    dup = np.sort(np.concatenate([off, off[::3], off[::7]])).astype(np.int32)
    assert np.array_equal(oracle_lib.scan_segmented(x, dup, "max"), oracle_lib.scan_segmented(x, off, "max"))
    # the last output of each non-empty segment is the segment total
    incl = oracle_lib.scan_segmented(x, off, "sum")
    ends = off[1:][np.diff(off) > 0] - 1
    starts = off[:-1][np.diff(off) > 0]
    totals = np.add.reduceat(x.astype(np.float64), starts)
    assert np.allclose(incl[ends], totals, rtol=1e-12)


# ---------------------------------------------------------------- packing


def test_pack_offsets_and_emit(oracle_lib):
    _, counts = inputs.compaction_inputs(100_000, seed=4)
    off, total = oracle_lib.pack_offsets(counts)
    assert off[0] == 0 and total == int(counts.sum()) and off[-1] == total
    assert np.array_equal(np.diff(off), counts)
    n = counts.size
    owner = np.repeat(np.arange(n), counts)
    rank = np.arange(total) - np.repeat(off[:-1], counts)
    rec = oracle_lib.pack_emit(off)
    assert np.array_equal(rec, (owner + 1 + rank) % n)


def test_pack_closed_forms(oracle_lib):
    off, total = oracle_lib.pack_offsets(np.ones(500, np.int32))
    assert np.array_equal(off, np.arange(501)) and total == 500
    off, total = oracle_lib.pack_offsets(np.zeros(500, np.int32))
    assert not off.any() and total == 0
    assert oracle_lib.pack_emit(off).size == 0
    big = np.array([0, 0, 1000, 0], np.int32)
    off, total = oracle_lib.pack_offsets(big)
    assert list(off) == [0, 0, 0, 1000, 1000]
    assert np.array_equal(oracle_lib.pack_emit(off), (3 + np.arange(1000)) % 4)
    # 64-bit total exposes int32 overflow
    off, total = oracle_lib.pack_offsets(np.full(3, 2 ** 30, np.int32))
    assert total == 3 * 2 ** 30
