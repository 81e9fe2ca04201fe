"""Host-side checks of the C ABI (no GPU): the library builds and loads, it
exports every function include/scan_wave64.h declares, the planner's tile
arithmetic, and argument errors that are rejected before any launch."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "scan_wave64.h")


@pytest.fixture(scope="module")
def lib():
    from stream_compaction_wave64_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from stream_compaction_wave64_amd import build
        build.build()
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("scan_inclusive", "scan_exclusive", "scan_dim", "compact_if", "pack_offsets",
                     "pack_emit_neighbors", "scan_plan", "scan_workspace_bytes", "scan_workspace_init",
                     "scan_status_string"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    from stream_compaction_wave64_amd import binding
    assert set(binding.EXPORTS) == set(declared_functions())


def test_header_compiles_as_c():
    import subprocess
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "t.c")
        open(src, "w").write('#include "scan_wave64.h"\nint main(void){scan_plan_t p; (void)p; return 0;}\n')
        subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), "-c", src,
                               "-o", os.path.join(d, "t.o")])


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.scan_status_string(code)
    assert b"unknown" in lib.scan_status_string(-99)
    assert b"gfx950" in lib.scan_version()


def test_plan_fp32_metric_shape():
    from stream_compaction_wave64_amd import binding
    import torch
    p = binding.plan("scan", torch.float32, "sum", 1, 10 ** 8)
    assert p["kernel"] == "lookback" and p["vec"] == 4
    # the look-back kernels give one wave of each workgroup to the look-back
    assert p["tile_elems"] == (p["block_size"] - 64) * p["items_per_thread"]
    assert p["num_tiles"] == -(-10 ** 8 // p["tile_elems"])
    assert p["carry_words"] == 1  # fp32 sums carry in fp64 between tiles, packed into one word
    assert p["launches"] == 1
    assert p["workspace_bytes"] >= 4096 + p["num_tiles"] * 8 * p["carry_words"]


def test_plan_segments_and_types():
    from stream_compaction_wave64_amd import binding
    import torch
    p = binding.plan("scan", torch.int32, "sum", 64, 20_000)
    assert p["kernel"] == "lookback" and p["num_tiles"] == 64 * -(-20_000 // p["tile_elems"])
    assert p["carry_words"] == 1
    p = binding.plan("scan", torch.float64, "max", 1, 10 ** 7)
    assert p["carry_words"] == 2 and p["vec"] == 2
    p = binding.plan("scan", torch.float32, "max", 1, 1000)
    assert p["carry_words"] == 1
    p = binding.plan("scan", torch.float32, "sum", 1, 1000, tuning={"block_size": 256, "items_per_thread": 4})
    assert p["tile_elems"] == 192 * 4
    p = binding.plan("scan", torch.float32, "sum", 1, 1000, tuning={"block_size": 256, "items_per_thread": 4,
                                                                     "algo": "reduce_then_scan"})
    assert p["tile_elems"] == 256 * 4
    with pytest.raises(binding.ScanError):
        binding.plan("scan", torch.float32, "sum", 1, 1000, tuning={"block_size": 192, "items_per_thread": 4})


def test_plan_rows_that_fit_one_tile():
    # Two or more rows of whole 128-bit vectors, each at least one wave's
    # vectors and at most 256 threads x 8 rows of them: one workgroup per row
    # (the fewest tile rows that hold it), no workspace, one launch.
    from stream_compaction_wave64_amd import binding
    import torch
    p = binding.plan("scan", torch.float32, "sum", 4096, 4096)
    assert (p["kernel"], p["block_size"], p["items_per_thread"], p["num_tiles"], p["workspace_bytes"],
            p["launches"]) == ("rows", 256, 16, 4096, 0, 1)
    for dt, vec in ((torch.float32, 4), (torch.int32, 4), (torch.float64, 2), (torch.int64, 2)):
        for r in (1, 2, 4, 8):
            for length in (256 * (r // 2) * vec + vec, 256 * r * vec):
                if length < 64 * vec:
                    continue
                p = binding.plan("scan", dt, "max", 3, length)
                assert (p["kernel"], p["items_per_thread"]) == ("rows", r * vec), (dt, r, length)
        assert binding.plan("scan", dt, "sum", 3, 2048 * vec + vec)["kernel"] == "lookback"  # longer than 8 rows
        assert binding.plan("scan", dt, "sum", 3, 64 * vec - vec)["kernel"] == "lookback"   # under one wave
        assert binding.plan("scan", dt, "sum", 3, 4096 + 1)["kernel"] == "lookback"         # not whole vectors
    assert binding.plan("scan", torch.float32, "sum", 1, 4096)["kernel"] == "resident"        # one array
    for tu in ({"grid_blocks": 8}, {"block_size": 512, "items_per_thread": 8}, {"no_identity": 1},
               {"algo": "reduce_then_scan"}):
        if tu.get("algo"):
            with pytest.raises(binding.ScanError):  # reduce-then-scan: whole arrays only
                binding.plan("scan", torch.float32, "sum", 4096, 4096, tuning=tu)
            continue
        assert binding.plan("scan", torch.float32, "sum", 4096, 4096, tuning=tu)["kernel"] == "lookback", tu


def test_plan_small_arrays_take_short_tiles():
    # Whole arrays of 128-bit rows take the resident pass at every size up to
    # its capacity, the smallest included.  With a grid cap (no resident
    # pass) those that 448 x 5-row tiles cover in at most 256 tiles (one per
    # CU) take those tiles; rows of a 2-D array take the resident pass from
    # 8 MiB; explicit shapes, the element-wide path and reduce-then-scan keep
    # their own (arrays within one default tile follow the short-segment rule
    # instead).
    from stream_compaction_wave64_amd import binding
    import torch
    cap = {"grid_blocks": 64}
    for dt, vec, big_ipt in ((torch.int32, 4, 28), (torch.float32, 4, 28), (torch.float64, 2, 16)):
        small_tile = 448 * 5 * vec
        big_tile = 448 * big_ipt if vec == 2 else 704 * big_ipt
        below = (8 << 20) // (16 // vec) - vec  # the largest array under 8 MiB
        for n in (vec, 64 * vec, 2 * big_tile, 128 * small_tile, below, below + vec, 256 * small_tile + vec):
            p = binding.plan("scan", dt, "sum", 1, n)
            assert p["kernel"] == "resident" and p["num_tiles"] <= 256 and p["block_size"] == 1024, (dt, n, p)
        for n in (2 * big_tile, 128 * small_tile, below):
            p = binding.plan("scan", dt, "sum", 1, n, tuning=cap)
            assert (p["kernel"], p["block_size"], p["items_per_thread"]) == ("lookback", 512, 5 * vec), (dt, n, p)
            assert p["num_tiles"] <= 256
        p = binding.plan("scan", dt, "sum", 1, 256 * small_tile + vec, tuning=cap)  # past 256 small tiles
        assert (p["kernel"], p["items_per_thread"]) == ("lookback", big_ipt), (dt, p)
        row8 = ((8 << 20) // (16 // vec) // 3 // vec + 1) * vec  # 3 rows of this many: just over 8 MiB
        for n in (big_tile, row8 - 2 * vec):  # rows of a 2-D array under 8 MiB
            assert binding.plan("scan", dt, "sum", 3, n)["kernel"] != "resident", (dt, n)
        assert binding.plan("scan", dt, "sum", 3, row8)["kernel"] == "resident"
        p = binding.plan("scan", dt, "sum", 1, 64 * small_tile + 1)  # element-wide path: unchanged
        assert p["vec"] == 1 and p["items_per_thread"] == big_ipt // vec, (dt, p)
        p = binding.plan("scan", dt, "sum", 1, 1024 * small_tile + 1)  # element-wide, 8 MiB and more
        assert p["kernel"] == "lookback" and p["vec"] == 1, (dt, p)
        p = binding.plan("scan", dt, "sum", 1, 64 * small_tile, tuning={"block_size": 512, "items_per_thread": 3 * vec})
        assert p["items_per_thread"] == 3 * vec and p["kernel"] == "lookback"
        p = binding.plan("scan", dt, "sum", 2, 64 * small_tile)
        assert p["items_per_thread"] == big_ipt, (dt, p)
    p = binding.plan("scan", torch.float32, "sum", 1, 1 << 20, tuning={"algo": "reduce_then_scan"})
    assert p["kernel"] == "reduce_then_scan" and p["items_per_thread"] == 32
    # count-scan-emit's offsets follow the scan's plan
    assert binding.plan("pack", torch.int32, "sum", 1, 4096)["launches"] == 1


def test_plan_resident():
    # The resident pass: one 1024-thread workgroup (15 data waves and a
    # control wave) per tile of rows x 960 x vec elements, or per two tiles
    # for a whole array of 28 MiB or more (40 MiB for 8-byte elements); the fewest rows that keep the
    # workgroups within 256, up to 17 rows (4-byte elements) or 21 (8-byte)
    # with one tile, 8 or 11 per tile with two; one descriptor word per tile
    # (two for 64-bit carries); not with a grid cap or an explicit shape;
    # segments (rows of a 2-D array) when all fit, one tile per workgroup.
    from stream_compaction_wave64_amd import binding
    import torch
    one = {"resident_sweeps": 1}
    p = binding.plan("scan", torch.float32, "sum", 1, 10 ** 7, tuning=one)   # 11 rows of 3840: 237 tiles
    assert (p["kernel"], p["block_size"], p["items_per_thread"], p["num_tiles"]) == ("resident", 1024, 44, 237)
    assert p["workspace_bytes"] == 4096 + 2048 and p["launches"] == 1  # 237 words, in 256-byte units
    assert p["tiles_per_block"] == 1
    p = binding.plan("scan", torch.float32, "sum", 1, 10 ** 7)   # 6 rows of 3840: 435 tiles, 218 workgroups
    assert (p["kernel"], p["items_per_thread"], p["num_tiles"], p["tiles_per_block"]) == ("resident", 24, 435, 2)
    assert p["workspace_bytes"] == 4096 + 3584
    p = binding.plan("scan", torch.float64, "sum", 1, 10 ** 7, tuning=one)   # 21 rows of 1920: 249 tiles
    assert (p["kernel"], p["items_per_thread"], p["num_tiles"], p["carry_words"]) == ("resident", 42, 249, 2)
    p = binding.plan("scan", torch.float64, "sum", 1, 10 ** 7)   # 11 rows of 1920: 474 tiles, 237 workgroups
    assert (p["kernel"], p["items_per_thread"], p["num_tiles"], p["tiles_per_block"]) == ("resident", 22, 474, 2)
    # two tiles from 28 MiB (4-byte elements) or 40 MiB (8-byte), one below;
    # a forced two below the threshold
    below = (28 << 20) // 4 - 4
    assert binding.plan("scan", torch.int32, "sum", 1, below)["tiles_per_block"] == 1
    assert binding.plan("scan", torch.int32, "sum", 1, below + 4)["tiles_per_block"] == 2
    below = (40 << 20) // 8 - 2
    assert binding.plan("scan", torch.float64, "sum", 1, below)["tiles_per_block"] == 1
    assert binding.plan("scan", torch.float64, "sum", 1, below + 2)["tiles_per_block"] == 2
    assert binding.plan("scan", torch.int64, "max", 1, (32 << 20) // 8)["tiles_per_block"] == 1
    assert binding.plan("scan", torch.int32, "sum", 1, 1 << 21, tuning={"resident_sweeps": 2})["tiles_per_block"] == 2
    # capacities: 256 x 17 rows of 3840 with one tile (two tiles hold 512 x 8
    # rows, fewer); 512 x 11 rows of 1920 with two (one tile: 256 x 21)
    cap4, cap8 = 256 * 17 * 3840, 512 * 11 * 1920
    p = binding.plan("scan", torch.int32, "sum", 1, cap4)
    assert (p["kernel"], p["items_per_thread"], p["num_tiles"], p["tiles_per_block"]) == ("resident", 68, 256, 1)
    assert binding.plan("scan", torch.int32, "sum", 1, cap4 + 4)["kernel"] == "lookback"
    p = binding.plan("scan", torch.int64, "max", 1, cap8)
    assert (p["kernel"], p["items_per_thread"], p["num_tiles"], p["tiles_per_block"]) == ("resident", 22, 512, 2)
    assert binding.plan("scan", torch.int64, "max", 1, cap8 + 2)["kernel"] == "lookback"
    assert binding.plan("scan", torch.int64, "max", 1, 256 * 21 * 1920 + 2, tuning=one)["kernel"] == "lookback"
    p = binding.plan("scan", torch.float32, "sum", 4, 1 << 20)    # segments: 4 x 55 tiles of 5 rows
    assert (p["kernel"], p["num_tiles"], p["items_per_thread"]) == ("resident", 220, 20)
    p = binding.plan("scan", torch.float32, "sum", 4, 3 << 20)    # 48 MiB of segments: one tile per workgroup
    assert (p["kernel"], p["tiles_per_block"]) == ("resident", 1), p
    for tu in ({"grid_blocks": 8}, {"block_size": 768, "items_per_thread": 28}, {"algo": "reduce_then_scan"}):
        assert binding.plan("scan", torch.float32, "sum", 1, 10 ** 7, tuning=tu)["kernel"] != "resident", tu
        assert binding.plan("scan", torch.float32, "sum", 1, 10 ** 7, tuning=tu)["tiles_per_block"] == 0, tu
    # inclusive scans without an identity take it too (Optional partials)
    p = binding.plan("scan", torch.float32, "sum", 1, 10 ** 7, tuning={"no_identity": 1})
    assert (p["kernel"], p["num_tiles"], p["items_per_thread"]) == ("resident", 435, 24)
    p = binding.plan("scan", torch.float32, "sum", 1, 10 ** 7, tuning={"no_identity": 1, "resident_sweeps": 1})
    assert (p["kernel"], p["num_tiles"], p["items_per_thread"]) == ("resident", 237, 44)
    assert binding.plan("scan", torch.float32, "sum", 1, 10 ** 7,
                        tuning={"no_identity": 1, "grid_blocks": 8})["kernel"] == "lookback"
    assert binding.plan("pack", torch.int32, "sum", 1, 10 ** 7)["kernel"] == "pack"
    # compaction: the same tiles (rows of 960 x 4 keys, at most 17 rows so the
    # tile-local indices fit 16 bits), at any size of whole 128-bit vectors
    p = binding.plan("compact", torch.float32, "sum", 1, 10 ** 7)
    assert (p["kernel"], p["num_tiles"], p["items_per_thread"], p["launches"]) == ("compact_resident", 237, 44, 1)
    assert binding.plan("compact", torch.int32, "sum", 1, 256 * 17 * 3840)["kernel"] == "compact_resident"
    assert binding.plan("compact", torch.int32, "sum", 1, 256 * 17 * 3840 + 4)["kernel"] == "compact"
    assert binding.plan("compact", torch.int32, "sum", 1, 4096)["kernel"] == "compact_resident"
    assert binding.plan("compact", torch.int32, "sum", 1, 4097)["kernel"] == "compact"  # element-wide
    assert binding.plan("compact", torch.float32, "sum", 1, 10 ** 7, tuning={"grid_blocks": 4})["kernel"] == "compact"
    p = binding.plan("partition", torch.float32, "sum", 1, 10 ** 7)  # one launch, no count pass
    assert (p["kernel"], p["num_tiles"], p["launches"]) == ("partition_resident", 237, 1)
    p = binding.plan("partition", torch.float32, "sum", 1, 10 ** 7, tuning={"grid_blocks": 4})
    assert (p["kernel"], p["launches"]) == ("partition", 2)


def test_plan_columns_single_pass():
    # Wide inner extents take the one-pass column kernel when the array makes
    # at most 256 register tiles of 256 rows x (64 x vec) columns (one per
    # compute unit) and at most 64 row blocks per strip; its workspace holds
    # one descriptor word per column of every tile (two for 64-bit carries).
    from stream_compaction_wave64_amd import binding
    import torch
    p = binding.plan("scan", torch.float32, "sum", 1, 4096, 4096)
    assert (p["kernel"], p["launches"], p["block_size"], p["vec"]) == ("columns_lookback", 1, 1024, 4)
    assert p["num_tiles"] == 16 * 16 and p["tile_elems"] == 256 * 256
    assert p["workspace_bytes"] == 4096 + 256 * 256 * 8
    p = binding.plan("scan", torch.float64, "sum", 1, 4096, 4096)  # 512 tiles of 128 columns
    assert (p["kernel"], p["launches"]) == ("columns", 3)
    p = binding.plan("scan", torch.float64, "max", 2, 1024, 1024)   # 2 x 4 x 8 tiles
    assert (p["kernel"], p["num_tiles"], p["carry_words"]) == ("columns_lookback", 64, 2)
    assert p["workspace_bytes"] == 4096 + 64 * 128 * 2 * 8
    p = binding.plan("scan", torch.int32, "sum", 1, 16384, 256)      # 64 row blocks: the most
    assert p["kernel"] == "columns_lookback"
    p = binding.plan("scan", torch.int32, "sum", 1, 16385, 256)      # 65 row blocks
    assert p["kernel"] == "columns"
    p = binding.plan("scan", torch.float32, "sum", 1, 4096, 4096, tuning={"algo": "reduce_then_scan"})
    assert (p["kernel"], p["launches"]) == ("columns", 3)
    p = binding.plan("scan", torch.float32, "sum", 1, 4096, 100)      # strips less than half full
    assert p["kernel"] != "columns_lookback"


def _call_scan(lib, fn, inp, out, n, dt=3, op=0, width=1, ws=None, wsb=0):
    return getattr(lib, fn)(inp, out, n, dt, op, width, ws, wsb, None, None)


def test_argument_errors_before_launch(lib):
    fake = ctypes.c_void_p(1 << 20)
    ws = ctypes.c_void_p(1 << 24)
    for fn in ("scan_inclusive", "scan_exclusive"):
        assert _call_scan(lib, fn, None, None, 0) == 0           # n == 0: no-op
        assert _call_scan(lib, fn, None, fake, 10) == -1         # NULL input
        assert _call_scan(lib, fn, fake, None, 10) == -1         # NULL output
        assert _call_scan(lib, fn, fake, fake, -1) == -1         # negative size
        assert _call_scan(lib, fn, fake, fake, 10, dt=9) == -1   # bad dtype
        assert _call_scan(lib, fn, fake, fake, 10, op=7) == -1   # bad op
        assert _call_scan(lib, fn, fake, fake, 10, width=0) == -1
        assert _call_scan(lib, fn, fake, fake, 10, ws=None, wsb=0) == -3        # no workspace
        assert _call_scan(lib, fn, fake, fake, 10 ** 6, ws=ws, wsb=300) == -3   # too small
        assert _call_scan(lib, fn, fake, fake, 10, ws=ctypes.c_void_p((1 << 24) + 8), wsb=1 << 20) == -3
    assert lib.scan_dim(fake, fake, 2, 3, 0, 3, 0, 0, ws, 1 << 20, None, None) == -1  # inner < 1
    assert lib.scan_dim(fake, fake, 0, 3, 1, 3, 0, 0, None, 0, None, None) == 0       # empty
    assert lib.pack_offsets(fake, -1, fake, ws, 1 << 20, None, None) == -1
    assert lib.pack_offsets(fake, 1 << 31, fake, ws, 1 << 20, None, None) == -5     # int32 overflow
    assert lib.scan_copy(fake, fake, 17, None) == -1
    d = ctypes.c_double
    for fn in ("compact_if", "partition_if"):
        extra = (fake,) if fn == "partition_if" else ()
        call = lambda dt, cmp, t, n=10: getattr(lib, fn)(fake, n, dt, cmp, d(t), fake, *extra, fake, ws, 1 << 20,
                                                         None, None)
        assert call(3, 9, 0.5) == -1          # bad predicate
        assert call(3, 6, 3) == -1            # bit predicate on fp32 keys
        assert call(0, 6, 32) == -1           # bit index past 31
        assert call(1, 7, 2.5) == -1          # fractional bit index
        assert call(2, 0, 0.5) == -2          # int64 keys are not built
        assert call(1, 0, 0.5, n=1 << 31) == -5
    assert lib.partition_if(fake, 10, 3, 0, d(0.5), None, None, fake, ws, 1 << 20, None, None) == -1  # NULL out


def test_segmented_argument_errors_and_plan(lib):
    from stream_compaction_wave64_amd import binding
    import torch
    fake = ctypes.c_void_p(1 << 20)
    ws = ctypes.c_void_p(1 << 24)
    seg = lambda n, nseg, off=fake, dt=3, op=0: lib.scan_segmented(fake, fake, n, off, nseg, dt, op, 0, ws, 1 << 20,
                                                                   None, None)
    assert seg(0, 0) == 0            # empty: no-op
    assert seg(-1, 1) == -1
    assert seg(10, -1) == -1
    assert seg(10, 0) == -1          # elements but no segment
    assert seg(10, 2, off=None) == -1
    assert seg(10, 2, dt=9) == -1
    assert seg(10, 2, op=7) == -1
    assert seg(1 << 31, 2) == -5
    for dt in (torch.int32, torch.float32, torch.float64, torch.int64):
        for n in (1, 1000, 10 ** 7, 3 * 10 ** 7):
            # reduce-then-scan by default; single pass (map, heads, look-back scan) on request
            for algo, launches in ((None, 4), ("reduce_then_scan", 4), ("lookback", 3)):
                tu = {"algo": algo} if algo else None
                p = binding.plan("segmented", dt, "sum", n // 3 + 1, n, tuning=tu)
                assert p["kernel"] == "segmented" and p["launches"] == launches
                assert p["num_tiles"] == -(-n // p["tile_elems"])
                # map words and head planes at least (descriptors too in one pass)
                assert 4096 + p["num_tiles"] * 8 + n // 4 <= p["workspace_bytes"]
                assert p["workspace_bytes"] <= binding.scan_workspace_bytes(dt, n)


def test_plan_partition():
    from stream_compaction_wave64_amd import binding
    import torch
    for dt in (torch.float32, torch.int32, torch.uint32):
        for n in (1000, 10 ** 7):  # whole vectors within 256 register tiles: one launch, no count words
            p = binding.plan("partition", dt, "sum", 1, n)
            assert p["kernel"] == "partition_resident" and p["launches"] == 1
            assert p["workspace_bytes"] == 4096 + -(-p["num_tiles"] * 8 // 256) * 256
        for n in (1, 1001, 10 ** 8, 2 ** 31 - 1):
            p = binding.plan("partition", dt, "sum", 1, n)
            assert p["kernel"] == "partition" and p["launches"] == 2
            # tile descriptors, then at most 1024 count words
            tiles = -(-n // p["tile_elems"])
            assert p["num_tiles"] == tiles
            assert 4096 + (tiles + 1) * 8 <= p["workspace_bytes"] <= 4096 + (tiles + 1024) * 8 + 256
            assert p["workspace_bytes"] <= binding.scan_workspace_bytes(dt, n)


def test_workspace_bound_covers_plans():
    from stream_compaction_wave64_amd import binding
    import torch
    for dt in (torch.int32, torch.float32, torch.float64, torch.int64):
        for n in (4, 1000, 10 ** 6, 10 ** 8):
            for tuning in (None, {"block_size": 256, "items_per_thread": 16 // torch.empty(0, dtype=dt).element_size()}):
                p = binding.plan("scan", dt, "sum", 1, n, tuning=tuning)
                assert p["workspace_bytes"] <= binding.scan_workspace_bytes(dt, n)


def test_element_block_rule_matches_oracle():
    # The planner applies the large-element block rule (AcceleratedKernels.jl
    # PR #208) on the HIP side; the oracle implements the same rule
    # independently.  Widths whose rule lands on 64..256 use the element kernel.
    import oracle
    from stream_compaction_wave64_amd import binding
    import torch
    oracle.build(force=False)
    for dt, esz in ((torch.float32, 4), (torch.float64, 8)):
        for w in (2, 3, 4, 8, 16, 17, 24):
            for budget in (0, 32768, 65536, 49152):
                tun = {"local_mem_bytes": budget} if budget else None
                expect = oracle.block_size(w * esz, budget or 32768, 0, 256)
                if expect < 64:
                    continue
                p = binding.plan("scan", dt, "sum", 1, 10 ** 6, w, tuning=tun)
                assert p["kernel"] == "element" and p["block_size"] == expect, (dt, w, budget, p)
    # explicit block size is kept
    p = binding.plan("scan", torch.float64, "sum", 1, 10 ** 6, 17, tuning={"block_size": 64})
    assert p["block_size"] == 64
    # the two struct configs: 136-byte duals and 96-byte structs at the PR's 32 KiB default
    assert binding.plan("scan", torch.float64, "sum", 1, 10 ** 6, 17)["block_size"] == 64
    assert binding.plan("scan", torch.float32, "sum", 1, 10 ** 6, 24)["block_size"] == 128
    # a budget below one wave's tile (2 * 64 * 192 B) falls through to the column kernel
    p = binding.plan("scan", torch.float64, "sum", 1, 10 ** 5, 24, tuning={"local_mem_bytes": 16384})
    assert p["kernel"] == "columns", p
    assert binding.plan("scan", torch.float64, "sum", 1, 10 ** 6, 17)["carry_words"] == 34
    assert binding.plan("scan", torch.float32, "sum", 1, 10 ** 6, 24)["carry_words"] == 48


def test_noalloc_rejects_before_any_device_work(lib):
    # Checked on the host before the library's array is touched: a plan
    # whose workspace exceeds the array, bad arguments, and the n == 0 no-op.
    # fp64 sums take two descriptor words per 7168-element tile, so 6e8
    # elements need more than 1 MiB.  The pointers are never dereferenced.
    assert lib.scan_inclusive_noalloc(16, 32, 600_000_000, 4, 0, 1, None, None) == -3  # SCAN_ERR_WORKSPACE
    assert lib.scan_inclusive_noalloc(None, None, 0, 4, 0, 1, None, None) == 0
    assert lib.scan_inclusive_noalloc(16, 32, 10, 4, 0, 0, None, None) == -1  # width 0
    assert lib.scan_inclusive_noalloc(16, 32, 10, 9, 0, 1, None, None) == -1  # unknown dtype
    assert lib.scan_inclusive_noalloc(16, 32, -1, 4, 0, 1, None, None) == -1
