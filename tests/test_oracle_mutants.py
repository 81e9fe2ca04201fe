"""Plant plausible mistakes in a copy of the oracle (CPU only) and check that the
pins in test_oracle.py catch each one.  This shows the pins are sensitive to a
dropped term, a wrong index, a swapped comparison or an off-by-one anywhere in
the oracle, rather than merely agreeing with it.

Each mutant runs in a child process: a planted index mistake writes outside
the oracle's output arrays, and that must not corrupt the test process."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import test_oracle as T

SRC = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()

MUTANTS = {
    "i32 exclusive written after combining": (
        "y[at] = (int32_t)acc;\n                    acc = i32_combine(op, acc, a);",
        "acc = i32_combine(op, acc, a);\n                    y[at] = (int32_t)acc;"),
    "scan index with len and inner swapped": (
        "int64_t at = (o * len + i) * inner + k;", "int64_t at = (o * inner + i) * len + k;"),
    "i32 max identity 0": ("case O_MAX: return (uint32_t)INT32_MIN;", "case O_MAX: return 0u;"),
    "u32 max compares the wrong way": ("case O_MAX: return (a > b) ? a : b;",
                                       "case O_MAX: return (a < b) ? a : b;"),
    "i64 prod adds": ("case O_PROD: return a * b;\n    case O_MAX: return ((int64_t)a",
                      "case O_PROD: return a + b;\n    case O_MAX: return ((int64_t)a"),
    "fp32 accumulated in fp32": ("acc = f64_combine(op, acc, a);\n                    y[at] = acc;",
                                 "acc = (float)f64_combine(op, acc, a);\n                    y[at] = acc;"),
    "fp64 TwoSum error term dropped": ("return dd_renorm(s, err + a.lo);", "return dd_renorm(s, a.lo);"),
    "fp64 prod ignores low word": ("return dd_renorm(p, err + a.lo * b);", "return dd_renorm(p, err);"),
    "abs prefix exclusive/inclusive swapped": (
        "if (exclusive) { p[at] = acc; acc += fabs((double)x[at]); }",
        "if (!exclusive) { p[at] = acc; acc += fabs((double)x[at]); }"),
    "abs prefix f64 exclusive/inclusive swapped": (
        "if (exclusive) { p[at] = acc; acc += fabs(x[at]); }",
        "if (!exclusive) { p[at] = acc; acc += fabs(x[at]); }"),
    "abs prefix f32 drops the absolute value": ("fabs((double)x[at])", "((double)x[at])"),
    "abs prefix f64 drops the absolute value": ("fabs(x[at])", "(x[at])"),
    "no-identity scan seeded with zero": (
        "if (i == 0) acc = LOAD(x[at]);                              \\",
        "if (i == 0) acc = COMBINE(op, LOAD(0), x[at]);              \\"),
    "no-identity scan drops x[0] from the fold": (
        "if (i == 0) acc = LOAD(x[at]);", "if (i <= 1) acc = LOAD(x[at]);"),
    "double-double turns -0.0 into +0.0": (
        "    if (e == 0.0) {          /* exact: s + 0.0 would turn a -0.0 into +0.0 */", "    if (0) {"),
    "compaction off by one": ("idx[count++] = (int32_t)i;", "idx[count++] = (int32_t)(i + 1);"),
    "compaction > taken as >=": ("case O_GT: return v > t;", "case O_GT: return v >= t;"),
    "partition rejected part not offset by k": (
        "int64_t at = k;                                                              \\",
        "int64_t at = 0;                                                              \\"),
    "partition keeps the rejected part's order reversed": (
        "for (int64_t i = 0; i < n; i++)                                              \\\n            if (!KEEP",
        "for (int64_t i = n - 1; i >= 0; i--)                                         \\\n            if (!KEEP"),
    "bit predicate tests the next bit": ("return ((v >> (t & 31u)) & 1u) == 0u;", "return ((v >> ((t + 1) & 31u)) & 1u) == 0u;"),
    "segmented scan drops each segment's last element": (
        "const int rc = SCAN(x + b, y + b, 1, e - b, 1, op, exclusive);",
        "const int rc = SCAN(x + b, y + b, 1, e - b - 1, 1, op, exclusive);"),
    "segmented scan skips the last segment": (
        "for (int64_t s = 0; s < nseg; s++) {                                            \\",
        "for (int64_t s = 0; s + 1 < nseg; s++) {                                        \\"),
    "pack offsets shifted": ("offsets[i + 1] = (int32_t)run;", "offsets[i] = (int32_t)run;"),
    "emit record drops the +1": ("(int32_t)((i + 1 + j) % n)", "(int32_t)((i + j) % n)"),
    "block rule without the per-thread totals": ("2 * b * esize > budget", "b * esize > budget"),
    "block rule floor 1": [("while (b > 2 &&", "while (b > 1 &&"), ("if (b < 2) b = 2;", "")],
}

PINS = [
    lambda o: [T.test_merry_prefix_sum_example(o, dt) for dt in T.ALL_TYPES],
    lambda o: [T.test_merry_kogge_stone_states(o, dt) for dt in T.ALL_TYPES],
    lambda o: [T.test_merry_brent_kung_example(o, dt) for dt in T.ALL_TYPES],
    lambda o: [T.test_merry_radix4_example(o, dt) for dt in T.ALL_TYPES],
    lambda o: T.test_merry_output_packing_example(o),
    lambda o: T.test_pr208_block_size_rule(o),
    lambda o: [T.test_constant_and_extrema_closed_forms(o, dt) for dt in T.ALL_TYPES],
    lambda o: T.test_prod_powers_of_two_wrap(o),
    lambda o: [T.test_brute_force_small(o, dt, op, 65) for dt in T.ALL_TYPES for op in T.OPS],
    lambda o: T.test_matches_numpy_accumulate_u32_i64(o),
    lambda o: T.test_scan_invariants_float(o),
    lambda o: [T.test_abs_prefix_alternating_signs_closed_form(o, dt) for dt in (np.float32, np.float64)],
    lambda o: [T.test_abs_prefix_signed_integer_shadow(o, dt, q, e)
               for dt, q in ((np.float32, 23), (np.float64, 30)) for e in (False, True)],
    lambda o: [T.test_abs_prefix_signed_dims(o, dt, q, e)
               for dt, q in ((np.float32, 23), (np.float64, 30)) for e in (False, True)],
    lambda o: [T.test_noid_brute_force_small(o, dt, op, n) for dt in T.ALL_TYPES for op in T.OPS for n in (3, 17)],
    lambda o: [T.test_noid_equals_identity_scan_inclusive(o, dt, op) for dt in T.ALL_TYPES for op in T.OPS],
    lambda o: [T.test_noid_keeps_negative_zero(o, dt) for dt in (np.float32, np.float64)],
    lambda o: T.test_fp64_exact_integer_shadow(o),
    lambda o: [T.test_dims_layouts_agree(o, dt) for dt in (np.int32, np.float32)],
    lambda o: T.test_compaction_brute_and_numpy(o),
    lambda o: T.test_compaction_closed_forms(o),
    lambda o: T.test_pack_offsets_and_emit(o),
    lambda o: T.test_compaction_bit_predicates(o),
    lambda o: T.test_partition_invariants(o),
    lambda o: T.test_partition_closed_forms(o),
    lambda o: T.test_radix_sort_from_stable_bit_partitions(o),
    lambda o: T.test_segmented_packing_example(o),
    lambda o: T.test_segmented_brute_force(o),
    lambda o: T.test_segmented_closed_forms_and_invariants(o),
]


def _caught(lib_path):
    saved = oracle._lib
    oracle._lib = None
    real = oracle._LIB
    try:
        oracle._LIB = lib_path
        oracle._load()
        for pin in PINS:
            try:
                pin(oracle)
            except Exception:
                return True
        return False
    finally:
        oracle._lib = saved
        oracle._LIB = real


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    edits = MUTANTS[name]
    if isinstance(edits, tuple):
        edits = [edits]
    text = SRC
    for old, new in edits:
        assert old in text, f"mutation anchor for {name!r} not found"
        text = text.replace(old, new)
    src = tmp_path / "mut.c"
    src.write_text(text)
    lib = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-w", "-o", str(lib), str(src), "-lm"])
    here = os.path.dirname(os.path.abspath(__file__))
    code = ("import sys; sys.path[:0] = [sys.argv[1], sys.argv[2]]\n"
            "import test_oracle_mutants as M\n"
            "print('CAUGHT' if M._caught(sys.argv[3]) else 'MISSED', flush=True)\n")
    r = subprocess.run([sys.executable, "-c", code, here, os.path.dirname(here), str(lib)],
                       capture_output=True, text=True, timeout=300)
    # a child killed by a signal ran into the mutant's own memory error
    caught = "CAUGHT" in r.stdout or r.returncode < 0
    assert caught and "MISSED" not in r.stdout, f"no pin caught the mutant: {name}\n{r.stdout}\n{r.stderr[-2000:]}"


def test_unmutated_oracle_passes_all_pins(oracle_lib):
    assert not _caught(oracle._LIB)
