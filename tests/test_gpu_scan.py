"""GPU parity of the single-pass look-back scan against the CPU oracle.

Sizes span one partial tile, exact tile multiples, several tiles with a
ragged tail, and many tiles forced by a small explicit tile shape; every
dtype x op x inclusive/exclusive; aligned (128-bit) and misaligned
(element-wide) access; in-place; the full-size metric and fp64 configs."""
import numpy as np
import pytest
import torch

import stream_compaction_wave64_amd as sw
from stream_compaction_wave64_amd import inputs
from gpu_util import DEV, TORCH, assert_scan_matches, to_dev, to_host

pytestmark = pytest.mark.gpu

DTYPES = [np.int32, np.uint32, np.int64, np.float32, np.float64]
OPS = ["sum", "prod", "max", "min"]


def _input(dt, n, seed, op):
    kind = "near1" if op == "prod" and np.issubdtype(dt, np.floating) else "wide"
    if op == "sum" and np.issubdtype(dt, np.floating):
        kind = "default"
    return inputs.generic(dt, n, seed, kind)


def _run(x, op, exclusive, tuning=None, offset=0):
    """Scan x on the device; offset > 0 shifts the data off 16-byte alignment."""
    if offset:
        buf = to_dev(np.concatenate([np.zeros(offset, x.dtype), x]))
        xd = buf[offset:]
        outbuf = torch.empty(x.size + offset, dtype=xd.dtype, device=DEV)
        out = outbuf[offset:]
    else:
        xd = to_dev(x)
        out = None
    fn = sw.scan_exclusive if exclusive else sw.scan_inclusive
    res = fn(xd, op=op, out=out, tuning=tuning)
    torch.cuda.synchronize()
    return to_host(res)


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: np.dtype(d).name)
@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
def test_parity_default_tiles(dt, op, exclusive):
    # Sizes around the small-array look-back tiles (448 x 5 rows of 128-bit
    # vectors), each run with the planner's choice (the resident pass for
    # whole vectors, the element-wide pipeline otherwise) and with that tile
    # shape pinned through the tuning (the look-back pipeline).
    vec = 16 // np.dtype(dt).itemsize
    small = {"block_size": 512, "items_per_thread": 5 * vec}
    p = sw.plan("scan", TORCH[np.dtype(dt)], op, 1, 10 ** 6, tuning=small)
    assert p["kernel"] == "lookback"
    tile = p["tile_elems"]
    for i, n in enumerate([1, 2, 3, 63, 64, 65, 1000, tile - 4, tile, tile + 4, 3 * tile + 12,
                           64 * tile - 4, 65 * tile + 4, 200_003]):
        x = _input(dt, n, 100 + i, op)
        assert_scan_matches(x, _run(x, op, exclusive), op, exclusive, what=f"n={n}")
        assert_scan_matches(x, _run(x, op, exclusive, small), op, exclusive, what=f"n={n} small tiles")


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: np.dtype(d).name)
@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("exclusive", [False, True], ids=["incl", "excl"])
def test_parity_whole_array_default_shape(dt, op, exclusive):
    # the shape large whole arrays get (the planner's choice at 1e8, beyond
    # the small-array rule and the resident pass), pinned through the tuning
    # so that sizes of a few tiles run it too
    p = sw.plan("scan", TORCH[np.dtype(dt)], op, 1, 10 ** 8)
    assert p["kernel"] == "lookback"
    tuning = {"block_size": p["block_size"], "items_per_thread": p["items_per_thread"]}
    tile = p["tile_elems"]
    assert sw.plan("scan", TORCH[np.dtype(dt)], op, 1, 1000, tuning=tuning)["tile_elems"] == tile
    for i, n in enumerate([5, tile - 4, tile + 4, 3 * tile + 12, 300 * tile - 4]):
        x = _input(dt, n, 300 + i, op)
        assert_scan_matches(x, _run(x, op, exclusive, tuning), op, exclusive, what=f"n={n}")


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: np.dtype(d).name)
@pytest.mark.parametrize("op", OPS)
def test_parity_across_shape_switches(dt, op):
    # Whole arrays of 128-bit rows: the resident single pass (one register
    # tile of 960 data threads x rows per compute unit, at most 256 tiles, 17
    # rows for 4-byte and 21 for 8-byte elements; two tiles per workgroup
    # from 28 MiB, 40 MiB for 8-byte elements) up to its capacity, the
    # smallest arrays included; past it the default look-back shape.  Both
    # sides of the switch.
    es = np.dtype(dt).itemsize
    vec = 16 // es
    big = sw.plan("scan", TORCH[np.dtype(dt)], op, 1, 10 ** 8)
    res_min = (8 << 20) // es
    # capacity: 256 tiles of 17 rows (4-byte), 512 tiles of 11 rows two per
    # workgroup (8-byte)
    cap = 256 * 17 * 960 * vec if es == 4 else 512 * 11 * 960 * vec
    cases = [(res_min - vec, "resident", None), (res_min, "resident", None), (cap, "resident", None),
             (cap + vec, "lookback", big["tile_elems"])]
    for i, (n, kernel, tile) in enumerate(cases):
        p = sw.plan("scan", TORCH[np.dtype(dt)], op, 1, n)
        assert p["kernel"] == kernel, (n, p)
        if tile is not None:
            assert p["tile_elems"] == tile, (n, p)
        else:
            blocks = -(-p["num_tiles"] // p["tiles_per_block"])
            assert blocks <= 256 and p["block_size"] == 1024, (n, p)
        if op not in ("sum", "max") and n > res_min:
            continue  # the two largest sizes: sum and max only (time)
        x = _input(dt, n, 400 + i, op)
        for excl in (False, True):
            assert_scan_matches(x, _run(x, op, excl), op, excl, what=f"n={n} excl={excl}")


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: np.dtype(d).name)
@pytest.mark.parametrize("op", OPS)
def test_parity_resident(dt, op):
    # the resident pass at row counts 3 and 7 with a ragged last tile (a
    # partial row, then a partial vector row), and a tile count that leaves
    # compute units idle
    es = np.dtype(dt).itemsize
    vec = 16 // es
    re = 960 * vec  # elements per tile row
    for i, (rows, n) in enumerate([(3, 3 * re * 200 + 5 * vec), (7, 7 * re * 255 + re + 3 * vec),
                                   (3, 3 * re * 181)]):
        p = sw.plan("scan", TORCH[np.dtype(dt)], op, 1, n)
        assert p["kernel"] == "resident", (n, p)
        x = _input(dt, n, 500 + i, op)
        for excl in (False, True):
            assert_scan_matches(x, _run(x, op, excl), op, excl, what=f"n={n} rows={p['items_per_thread'] // vec}")


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: np.dtype(d).name)
@pytest.mark.parametrize("op", OPS)
def test_parity_resident_two_tiles(dt, op):
    # The resident pass with two tiles per workgroup (whole arrays from 28
    # MiB, 40 MiB for 8-byte elements; workgroup w holds tiles w and w + G):
    # an odd tile count (the last
    # workgroup has no second tile) with a ragged last tile, an even count
    # ending in a partial vector row, the form's capacity (512 full tiles),
    # and a forced two-tile plan below the threshold (two rows per tile).
    es = np.dtype(dt).itemsize
    vec = 16 // es
    re = 960 * vec
    rows = 8 if es == 4 else 11
    even = 436 * 6 * re - 3 * vec if es == 4 else 10 ** 7
    # just past the planner's switch to two tiles, stepped until the tile
    # count is odd, with a ragged last tile
    odd = ((28 << 20) if es == 4 else (40 << 20)) // es + 3 * vec
    while sw.plan("scan", TORCH[np.dtype(dt)], op, 1, odd)["num_tiles"] % 2 == 0:
        odd += 997 * vec
    sizes = [(odd, None), (even, None), (512 * rows * re, None),
             ((8 << 20) // es, {"resident_sweeps": 2})]
    if op not in ("sum", "max"):
        sizes = sizes[:1] + sizes[3:]  # time: the other operators at the small sizes
    counts = set()
    for i, (n, tuning) in enumerate(sizes):
        p = sw.plan("scan", TORCH[np.dtype(dt)], op, 1, n, tuning=tuning)
        assert p["kernel"] == "resident" and p["tiles_per_block"] == 2, (n, p)
        assert -(-p["num_tiles"] // 2) <= 256, (n, p)
        counts.add(p["num_tiles"] % 2)
        x = _input(dt, n, 520 + i, op)
        for excl in (False, True):
            assert_scan_matches(x, _run(x, op, excl, tuning), op, excl,
                                what=f"n={n} tiles={p['num_tiles']} rows={p['items_per_thread'] // vec}")
    assert counts == {0, 1}, "odd and even tile counts"


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: np.dtype(d).name)
@pytest.mark.parametrize("op", OPS)
def test_parity_many_small_tiles(dt, op):
    # one row per tile: tile = 192 x vec elements (256 threads less the
    # look-back wave), so 1e5 elements make
    # hundreds of tiles and the look-back walks windows of 64
    vec = 16 // np.dtype(dt).itemsize
    tuning = {"block_size": 256, "items_per_thread": vec}
    for n, seed in ((100_000, 1), (256 * vec * 70 + 8, 2)):
        x = _input(dt, n, seed, op)
        for excl in (False, True):
            assert_scan_matches(x, _run(x, op, excl, tuning), op, excl, what=f"n={n} excl={excl}")


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: np.dtype(d).name)
@pytest.mark.parametrize("grid", [1, 2, 3, 7, 64])
def test_parity_small_persistent_grid(dt, grid):
    # a grid of a few workgroups makes each one scan many tiles in turn,
    # exercising the prefetch alternation and look-back across rounds
    vec = 16 // np.dtype(dt).itemsize
    tuning = {"block_size": 256, "items_per_thread": vec, "grid_blocks": grid}
    for n, seed in ((256 * vec * 37 + 4 * vec, 3), (256 * vec * 2, 4), (5 * vec, 5)):
        x = _input(dt, n, seed, "sum")
        for excl in (False, True):
            assert_scan_matches(x, _run(x, "sum", excl, tuning), "sum", excl, what=f"n={n} excl={excl}")


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: np.dtype(d).name)
@pytest.mark.parametrize("grid", [513, 514, 0])
def test_parity_lookback_either_side_of_gap_grid(dt, grid):
    # grids of up to 513 workgroups use the aggregate-only look-back (each
    # workgroup reads the G - 1 aggregates since its own previous tile);
    # larger ones (514, or the resident count of one-row tiles) the windowed
    # look-back over published prefixes; 1501 tiles either way
    vec = 16 // np.dtype(dt).itemsize
    tuning = {"block_size": 256, "items_per_thread": vec, "grid_blocks": grid}
    n = 192 * vec * 1500 + 3 * vec
    assert sw.plan("scan", TORCH[np.dtype(dt)], "sum", 1, n, tuning=tuning)["num_tiles"] == 1501
    for op, seed in (("sum", 11), ("max", 12)):
        x = _input(dt, n, seed, op)
        for excl in (False, True):
            assert_scan_matches(x, _run(x, op, excl, tuning), op, excl, what=f"grid={grid} {op} excl={excl}")


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: np.dtype(d).name)
def test_parity_misaligned_elementwise(dt):
    for n in (1, 5, 3001, 100_001):
        x = _input(dt, n, 7, "sum")
        for excl in (False, True):
            assert_scan_matches(x, _run(x, "sum", excl, offset=1), "sum", excl, what=f"n={n}")
            assert_scan_matches(x, _run(x, "max", excl, offset=1), "max", excl, what=f"n={n}")


@pytest.mark.parametrize("dt", [np.float32, np.float64], ids=["float32", "float64"])
def test_prod_of_powers_of_two_bit_exact(dt):
    # factors 2^d with d in {-1, 0, 1} steered to keep the exponent walk inside
    # [-60, 60]: every partial product is exact, so any association must give
    # the oracle's value bit for bit (a dropped or repeated factor shows).
    rng = np.random.default_rng(31)
    n = 300_001
    d = rng.integers(-1, 2, n)
    e = 0
    for i in range(n):
        if abs(e + d[i]) > 60:
            d[i] = -d[i]
        e += d[i]
    x = np.ldexp(np.ones(n), d).astype(dt)
    for excl in (False, True):
        for tuning in (None, {"block_size": 256, "items_per_thread": 16 // np.dtype(dt).itemsize}):
            got = _run(x, "prod", excl, tuning)
            ref = __import__("oracle").scan(x, "prod", exclusive=excl).astype(dt)
            assert np.array_equal(got, ref), f"excl={excl} tuning={tuning}"


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: np.dtype(d).name)
@pytest.mark.parametrize("op", OPS)
def test_parity_reduce_then_scan(dt, op):
    vec = 16 // np.dtype(dt).itemsize
    for n, tuning in ((1, {}), (1000, {}), (3_000_001, {}), (1_000_003, {"rts_blocks": 7}),
                      (256 * vec * 50 + 4, {"block_size": 256, "items_per_thread": vec, "rts_blocks": 3}),
                      (123_457, {"block_size": 256, "items_per_thread": vec, "rts_blocks": 1000})):
        x = _input(dt, n, 60, op)
        tu = dict(tuning, algo="reduce_then_scan")
        for excl in (False, True):
            assert_scan_matches(x, _run(x, op, excl, tu), op, excl, what=f"n={n} {tuning} excl={excl}")


def test_reduce_then_scan_leaves_workspace_clean():
    # its partials share the descriptor area: a look-back call right after must
    # see only untagged words
    x = inputs.generic(np.float32, 2_000_000, 61)
    for _ in range(3):
        a = _run(x, "sum", False, {"algo": "reduce_then_scan"})
        b = _run(x, "sum", False)
        assert_scan_matches(x, a, "sum", False)
        assert_scan_matches(x, b, "sum", False)


def test_config_fp32_1e8_reduce_then_scan():
    x = inputs.f32_uniform_01(10 ** 8, seed=1)
    r = sw.scan_inclusive(to_dev(x), tuning={"algo": "reduce_then_scan"})
    torch.cuda.synchronize()
    assert_scan_matches(x, to_host(r), "sum", False, what="fp32 1e8 rts")


def test_in_place():
    x = inputs.generic(np.int32, 300_001, 9, "wide")
    xd = to_dev(x)
    sw.scan_inclusive(xd, out=xd)
    torch.cuda.synchronize()
    assert_scan_matches(x, to_host(xd), "sum", False)
    y = inputs.generic(np.float32, 123_457 * 4, 10)
    yd = to_dev(y)
    sw.scan_exclusive(yd, out=yd)
    torch.cuda.synchronize()
    assert_scan_matches(y, to_host(yd), "sum", True)


def test_repeated_calls_reuse_workspace():
    # descriptors are tagged with a per-workspace epoch: back-to-back calls of
    # different sizes and types on one workspace must not see each other's
    x = inputs.generic(np.int32, 500_000, 11, "wide")
    xd = to_dev(x)
    f = inputs.generic(np.float64, 77_777, 12)
    fd = to_dev(f)
    for k in range(20):
        a = sw.scan_inclusive(xd if k % 2 == 0 else xd[: 100_000 + k])
        b = sw.scan_exclusive(fd, op="sum")
        torch.cuda.synchronize()
        assert_scan_matches(x if k % 2 == 0 else x[: 100_000 + k], to_host(a), "sum", False, what=f"k={k}")
        assert_scan_matches(f, to_host(b), "sum", True, what=f"k={k}")


def test_shrinking_call_clears_stale_descriptors():
    # Descriptor tags carry the epoch mod 256.  A large call at epoch 2 leaves
    # its words tagged 2.  A small call at epoch 257 must clear the words above
    # its own up to the high-water mark: the next call runs at epoch 258,
    # which is 2 mod 256, and a large call there would otherwise accept the
    # stale tag-2 words as published.
    from stream_compaction_wave64_amd import binding
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    hdr = ws[:16].view(torch.int32)  # [0] epoch, [1] error, [2:4] high-water mark
    words = ws[4096:].view(torch.int64)
    big1 = inputs.generic(np.int32, 2_000_003, 13, "wide")
    big2 = inputs.generic(np.int32, 2_000_003, 16, "wide")
    small = inputs.generic(np.int32, 50_000, 14, "wide")
    tiles_big = -(-big1.size // sw.plan("scan", torch.int32, "sum", 1, big1.size)["tile_elems"])
    tiles_small = -(-small.size // sw.plan("scan", torch.int32, "sum", 1, small.size)["tile_elems"])
    assert tiles_small > 1 and tiles_big > 2 * tiles_small
    key = (torch.device(DEV).index, binding._stream(torch.device(DEV)))
    saved = binding.workspaces._ws.get(key)
    binding.workspaces._ws[key] = ws
    try:
        hdr[0] = 2
        r = sw.scan_inclusive(to_dev(big1))
        torch.cuda.synchronize()
        assert_scan_matches(big1, to_host(r), "sum", False, what="big at epoch 2")
        assert int(hdr[0].item()) == 3 and int(hdr[2].item()) == tiles_big
        assert words[tiles_small:tiles_big].ne(0).all().item()  # tagged words left behind
        hdr[0] = 257
        r = sw.scan_inclusive(to_dev(small))
        torch.cuda.synchronize()
        assert_scan_matches(small, to_host(r), "sum", False, what="small at epoch 257")
        assert int(hdr[0].item()) == 258 and int(hdr[2].item()) == tiles_small
        assert not words[tiles_small:tiles_big].any().item()
        r = sw.scan_inclusive(to_dev(big2))
        torch.cuda.synchronize()
        assert_scan_matches(big2, to_host(r), "sum", False, what="big at epoch 258")
        assert int(hdr[1].item()) == 0  # no error and no fallback along the way
    finally:
        if saved is None:
            binding.workspaces._ws.pop(key, None)
        else:
            binding.workspaces._ws[key] = saved


def test_shrinking_ws_bytes_on_one_buffer():
    # A buffer initialised with scan_workspace_init records its size, so calls
    # that pass only their own plan's ws_bytes on it still clear what a larger
    # call left tagged beyond their range.  A large call, then 300 small calls
    # (more than the 256 epochs after which a tag repeats) each passing its
    # own smaller size, then a large call again: every result exact, no error.
    import ctypes
    from stream_compaction_wave64_amd import binding
    lib = binding.load_library()
    nbytes = 1 << 22
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    sw.scan_workspace_init(ws)
    stream = binding._stream(torch.device(DEV))
    big1 = inputs.generic(np.int32, 2_000_003, 17, "wide")
    big2 = inputs.generic(np.int32, 2_000_003, 18, "wide")
    small = inputs.generic(np.int32, 60_000, 19, "wide")
    p_big = sw.plan("scan", torch.int32, "sum", 1, big1.size)
    p_small = sw.plan("scan", torch.int32, "sum", 1, small.size)
    assert p_small["num_tiles"] > 1 and p_big["num_tiles"] > 2 * p_small["num_tiles"]
    assert p_big["workspace_bytes"] <= nbytes

    def run(x, ws_bytes):
        xd, out = to_dev(x), torch.empty(x.size, dtype=torch.int32, device=DEV)
        rc = lib.scan_inclusive(xd.data_ptr(), out.data_ptr(), x.size, 0, 0, 1, ws.data_ptr(), ws_bytes, None,
                                stream)
        assert rc == 0, rc
        return out

    r = run(big1, p_big["workspace_bytes"])
    torch.cuda.synchronize()
    assert_scan_matches(big1, to_host(r), "sum", False, what="first large call")
    xs = to_dev(small)
    outs = torch.empty(small.size, dtype=torch.int32, device=DEV)
    for k in range(300):
        rc = lib.scan_inclusive(xs.data_ptr(), outs.data_ptr(), small.size, 0, 0, 1, ws.data_ptr(),
                                p_small["workspace_bytes"], None, stream)
        assert rc == 0, rc
    torch.cuda.synchronize()
    assert_scan_matches(small, to_host(outs), "sum", False, what="small calls")
    r = run(big2, p_big["workspace_bytes"])
    torch.cuda.synchronize()
    assert_scan_matches(big2, to_host(r), "sum", False, what="large call after 300 small ones")
    assert sw.scan_workspace_error(ws) == 0


def test_empty_and_degenerate():
    e = torch.empty(0, dtype=torch.float32, device=DEV)
    assert sw.scan_inclusive(e).numel() == 0
    one = to_dev(np.array([2.5], np.float32))
    assert to_host(sw.scan_inclusive(one))[0] == 2.5
    assert to_host(sw.scan_exclusive(one))[0] == 0.0
    assert to_host(sw.scan_exclusive(one, op="max"))[0] == -np.inf
    assert to_host(sw.scan_exclusive(to_dev(np.array([7], np.int32)), op="min"))[0] == np.iinfo(np.int32).max


def test_config_int32_2pow20_bit_exact():
    x = inputs.int32_uniform_0_100(2 ** 20, seed=0)
    xd = to_dev(x)
    for excl in (False, True):
        fn = sw.scan_exclusive if excl else sw.scan_inclusive
        r = fn(xd)
        torch.cuda.synchronize()
        assert_scan_matches(x, to_host(r), "sum", excl, what=f"C1 excl={excl}")


def test_config_fp32_1e8_within_tolerance():
    x = inputs.f32_uniform_01(10 ** 8, seed=1)
    r = sw.scan_inclusive(to_dev(x))
    torch.cuda.synchronize()
    assert_scan_matches(x, to_host(r), "sum", False, what="fp32 1e8")


def test_config_fp64_1e7_within_tolerance():
    x = inputs.f64_uniform_pm1(10 ** 7, seed=1)
    r = sw.scan_inclusive(to_dev(x))
    torch.cuda.synchronize()
    assert_scan_matches(x, to_host(r), "sum", False, what="fp64 1e7")


def test_beyond_2pow31_elements_sampled():
    # int32 all-ones over 2^31 + 1027 elements: element i is (i + 1) mod 2^32;
    # exercises 64-bit element offsets; checked on samples and the tail.
    n = 2 ** 31 + 1027
    x = torch.ones(n, dtype=torch.int32, device=DEV)
    out = sw.scan_inclusive(x)
    torch.cuda.synchronize()
    del x
    rng = np.random.default_rng(15)
    idx = np.concatenate([rng.integers(0, n, 200_000), np.arange(n - 5000, n), np.arange(2 ** 31 - 10, 2 ** 31 + 10)])
    got = to_host(out[torch.from_numpy(idx).to(DEV)])
    want = ((idx + 1) % (1 << 32)).astype(np.uint32).view(np.int32)
    assert np.array_equal(got, want)
