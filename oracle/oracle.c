/*
 * oracle.c -- sequential CPU oracle for prefix scan, stream compaction and
 * count-scan-emit packing.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file: only tests/, the smoke check in __graft_entry__.py and the
 * cpu_baseline leg of bench.py use it.  It shares no code, header, table or
 * constant with the HIP library; it is plain C99 compiled with gcc -O2 and no
 * fast-math, so a reader can check every loop against the definitions by eye.
 *
 * Definitions followed (sources are the pages' titles and sections):
 *  - Merry, "Prefix sums on GPUs" (GPGPU2 Workshop 2014), slides "Exclusive
 *    Prefix Sum" and "Inclusive Prefix Sum": with an operator (+) and its
 *    identity I, the inclusive scan of (a0..a_{n-1}) has element i equal to
 *    a0 (+) ... (+) a_i; the exclusive scan has element i equal to
 *    a0 (+) ... (+) a_{i-1}, and I at i = 0.
 *  - same slides, "Other Applications": compaction selects the objects that
 *    satisfy a predicate; "visibility" uses max in place of +.
 *  - same slides, "Output Format" / "Solution": each object writes its count,
 *    a scan turns counts into start positions, each object then emits its
 *    records from its start position, packed contiguously.
 *  - AcceleratedKernels.jl PR #208 ("Fit the scans' tiles in local memory for
 *    large element types"), description, first bullet and first commit
 *    message: the block-size rule for large element types.
 *
 * Readings of points the pages leave open:
 *  - integer arithmetic wraps modulo 2^w (two's complement), done here in
 *    unsigned arithmetic of the same width;
 *  - fp32 inputs are accumulated in fp64 and the fp64 prefix is returned;
 *    fp64 inputs are accumulated in double-double (Knuth's TwoSum / an
 *    fma-based TwoProd) and the rounded double is returned;
 *  - identities: sum 0, prod 1, max the type's lowest value (-inf for
 *    floats), min the type's highest value (+inf for floats);
 *  - the record emitted by object i as its j-th record is (i + 1 + j) mod n
 *    (the pages leave record content open; only the layout is fixed).
 *
 * Array layout for every scan: a dense row-major (outer, len, inner) array,
 * scanned along the middle axis; element (o, i, k) sits at o*len*inner +
 * i*inner + k.  A 1-D scan is (1, n, 1); an array of n structs of w
 * components scanned component-wise is (1, n, w).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

enum { O_SUM = 0, O_PROD = 1, O_MAX = 2, O_MIN = 3 };
enum { O_GT = 0, O_GE = 1, O_LT = 2, O_LE = 3, O_EQ = 4, O_NE = 5, O_BIT_CLEAR = 6, O_BIT_SET = 7 };

/* ---------------------------------------------------------------- int32 -- */

static uint32_t i32_combine(int op, uint32_t a, uint32_t b) {
    switch (op) {
    case O_SUM: return a + b;                       /* wraps mod 2^32 */
    case O_PROD: return a * b;                      /* wraps mod 2^32 */
    case O_MAX: return ((int32_t)a > (int32_t)b) ? a : b;
    default: return ((int32_t)a < (int32_t)b) ? a : b;
    }
}

static uint32_t i32_identity(int op) {
    switch (op) {
    case O_SUM: return 0u;
    case O_PROD: return 1u;
    case O_MAX: return (uint32_t)INT32_MIN;
    default: return (uint32_t)INT32_MAX;
    }
}

int oracle_scan_i32(const int32_t *x, int32_t *y, int64_t outer, int64_t len,
                    int64_t inner, int op, int exclusive) {
    if (op < O_SUM || op > O_MIN) return -1;
    for (int64_t o = 0; o < outer; o++) {
        for (int64_t k = 0; k < inner; k++) {
            uint32_t acc = i32_identity(op);
            for (int64_t i = 0; i < len; i++) {
                int64_t at = (o * len + i) * inner + k;
                uint32_t a = (uint32_t)x[at];
                if (exclusive) {
                    y[at] = (int32_t)acc;
                    acc = i32_combine(op, acc, a);
                } else {
                    acc = i32_combine(op, acc, a);
                    y[at] = (int32_t)acc;
                }
            }
        }
    }
    return 0;
}

/* --------------------------------------------------------------- uint32 -- */

static uint32_t u32_combine(int op, uint32_t a, uint32_t b) {
    switch (op) {
    case O_SUM: return a + b;
    case O_PROD: return a * b;
    case O_MAX: return (a > b) ? a : b;
    default: return (a < b) ? a : b;
    }
}

static uint32_t u32_identity(int op) {
    switch (op) {
    case O_SUM: return 0u;
    case O_PROD: return 1u;
    case O_MAX: return 0u;
    default: return UINT32_MAX;
    }
}

int oracle_scan_u32(const uint32_t *x, uint32_t *y, int64_t outer, int64_t len,
                    int64_t inner, int op, int exclusive) {
    if (op < O_SUM || op > O_MIN) return -1;
    for (int64_t o = 0; o < outer; o++) {
        for (int64_t k = 0; k < inner; k++) {
            uint32_t acc = u32_identity(op);
            for (int64_t i = 0; i < len; i++) {
                int64_t at = (o * len + i) * inner + k;
                if (exclusive) {
                    y[at] = acc;
                    acc = u32_combine(op, acc, x[at]);
                } else {
                    acc = u32_combine(op, acc, x[at]);
                    y[at] = acc;
                }
            }
        }
    }
    return 0;
}

/* ---------------------------------------------------------------- int64 -- */

static uint64_t i64_combine(int op, uint64_t a, uint64_t b) {
    switch (op) {
    case O_SUM: return a + b;                       /* wraps mod 2^64 */
    case O_PROD: return a * b;
    case O_MAX: return ((int64_t)a > (int64_t)b) ? a : b;
    default: return ((int64_t)a < (int64_t)b) ? a : b;
    }
}

static uint64_t i64_identity(int op) {
    switch (op) {
    case O_SUM: return 0u;
    case O_PROD: return 1u;
    case O_MAX: return (uint64_t)INT64_MIN;
    default: return (uint64_t)INT64_MAX;
    }
}

int oracle_scan_i64(const int64_t *x, int64_t *y, int64_t outer, int64_t len,
                    int64_t inner, int op, int exclusive) {
    if (op < O_SUM || op > O_MIN) return -1;
    for (int64_t o = 0; o < outer; o++) {
        for (int64_t k = 0; k < inner; k++) {
            uint64_t acc = i64_identity(op);
            for (int64_t i = 0; i < len; i++) {
                int64_t at = (o * len + i) * inner + k;
                uint64_t a = (uint64_t)x[at];
                if (exclusive) {
                    y[at] = (int64_t)acc;
                    acc = i64_combine(op, acc, a);
                } else {
                    acc = i64_combine(op, acc, a);
                    y[at] = (int64_t)acc;
                }
            }
        }
    }
    return 0;
}

/* ------------------------------------------------- fp32 (fp64 accumulator) */

static double f64_combine(int op, double a, double b) {
    switch (op) {
    case O_SUM: return a + b;
    case O_PROD: return a * b;
    case O_MAX: return (a > b) ? a : b;
    default: return (a < b) ? a : b;
    }
}

static double f64_identity(int op) {
    switch (op) {
    case O_SUM: return 0.0;
    case O_PROD: return 1.0;
    case O_MAX: return -INFINITY;
    default: return INFINITY;
    }
}

/* y receives the fp64 prefix of the fp32 inputs (the reference the fp32
 * result is compared with). */
int oracle_scan_f32(const float *x, double *y, int64_t outer, int64_t len,
                    int64_t inner, int op, int exclusive) {
    if (op < O_SUM || op > O_MIN) return -1;
    for (int64_t o = 0; o < outer; o++) {
        for (int64_t k = 0; k < inner; k++) {
            double acc = f64_identity(op);
            for (int64_t i = 0; i < len; i++) {
                int64_t at = (o * len + i) * inner + k;
                double a = (double)x[at];
                if (exclusive) {
                    y[at] = acc;
                    acc = f64_combine(op, acc, a);
                } else {
                    acc = f64_combine(op, acc, a);
                    y[at] = acc;
                }
            }
        }
    }
    return 0;
}

/* --------------------------------------- fp64 (double-double accumulator) */

/* (hi, lo) represents hi + lo exactly, |lo| <= ulp(hi)/2 after renorm. */
typedef struct { double hi, lo; } dd_t;

static dd_t dd_renorm(double s, double e) {         /* Fast2Sum, |s| >= |e| */
    dd_t r;
    if (e == 0.0) {          /* exact: s + 0.0 would turn a -0.0 into +0.0 */
        r.hi = s;
        r.lo = 0.0;
        return r;
    }
    r.hi = s + e;
    r.lo = e - (r.hi - s);
    return r;
}

static dd_t dd_add(dd_t a, double b) {              /* Knuth TwoSum + carry */
    double s = a.hi + b;
    double bb = s - a.hi;
    double err = (a.hi - (s - bb)) + (b - bb);
    return dd_renorm(s, err + a.lo);
}

static dd_t dd_mul(dd_t a, double b) {              /* TwoProd via fma */
    double p = a.hi * b;
    double err = fma(a.hi, b, -p);
    return dd_renorm(p, err + a.lo * b);
}

static dd_t dd_combine(int op, dd_t acc, double b) {
    dd_t r;
    switch (op) {
    case O_SUM: return dd_add(acc, b);
    case O_PROD: return dd_mul(acc, b);
    case O_MAX:
        if (acc.hi > b || (acc.hi == b && acc.lo >= 0.0)) return acc;
        r.hi = b; r.lo = 0.0; return r;
    default:
        if (acc.hi < b || (acc.hi == b && acc.lo <= 0.0)) return acc;
        r.hi = b; r.lo = 0.0; return r;
    }
}

/* y receives the double nearest to the double-double prefix. */
int oracle_scan_f64(const double *x, double *y, int64_t outer, int64_t len,
                    int64_t inner, int op, int exclusive) {
    if (op < O_SUM || op > O_MIN) return -1;
    for (int64_t o = 0; o < outer; o++) {
        for (int64_t k = 0; k < inner; k++) {
            dd_t acc;
            acc.hi = f64_identity(op);
            acc.lo = 0.0;
            for (int64_t i = 0; i < len; i++) {
                int64_t at = (o * len + i) * inner + k;
                if (exclusive) {
                    y[at] = acc.hi;
                    acc = dd_combine(op, acc, x[at]);
                } else {
                    acc = dd_combine(op, acc, x[at]);
                    y[at] = acc.hi;
                }
            }
        }
    }
    return 0;
}

/* ---------------------------- inclusive scans without a neutral element --
 * AcceleratedKernels.jl PR #208, description, first bullet: the partial
 * results may be "Optional" when the operator has no neutral element.  The
 * inclusive scan needs none: element 0 of each scanned column is x[0] itself
 * and element i is element i-1 combined with x[i].  These loops start from
 * the first input and never form an identity, so for sums a -0.0 input keeps
 * its sign (an identity 0.0 would turn 0.0 + -0.0 into +0.0).  Exclusive
 * scans have no value at i = 0 without an identity and are not defined. */
#define NOID_SCAN(NAME, T, ACC_T, LOAD, COMBINE, STORE)                            \
    int NAME(const T *x, void *yv, int64_t outer, int64_t len, int64_t inner,   \
             int op) {                                                          \
        if (op < O_SUM || op > O_MIN) return -1;                                \
        for (int64_t o = 0; o < outer; o++) {                                   \
            for (int64_t k = 0; k < inner; k++) {                               \
                ACC_T acc;                                                      \
                for (int64_t i = 0; i < len; i++) {                             \
                    int64_t at = (o * len + i) * inner + k;                     \
                    if (i == 0) acc = LOAD(x[at]);                              \
                    else acc = COMBINE(op, acc, x[at]);                         \
                    STORE(yv, at, acc);                                         \
                }                                                               \
            }                                                                   \
        }                                                                       \
        return 0;                                                               \
    }

#define LD_U32(v) ((uint32_t)(v))
#define LD_U64(v) ((uint64_t)(v))
#define LD_F64(v) ((double)(v))
static dd_t dd_from(double v) { dd_t r; r.hi = v; r.lo = 0.0; return r; }
#define ST_I32(y, at, acc) (((int32_t *)(y))[at] = (int32_t)(acc))
#define ST_U32(y, at, acc) (((uint32_t *)(y))[at] = (acc))
#define ST_I64(y, at, acc) (((int64_t *)(y))[at] = (int64_t)(acc))
#define ST_F64(y, at, acc) (((double *)(y))[at] = (acc))
#define ST_DD(y, at, acc) (((double *)(y))[at] = (acc).hi)
#define CB_I32(op, acc, v) i32_combine(op, acc, (uint32_t)(v))
#define CB_I64(op, acc, v) i64_combine(op, acc, (uint64_t)(v))
#define CB_F64(op, acc, v) f64_combine(op, acc, (double)(v))

NOID_SCAN(oracle_scan_noid_i32, int32_t, uint32_t, LD_U32, CB_I32, ST_I32)
NOID_SCAN(oracle_scan_noid_u32, uint32_t, uint32_t, LD_U32, u32_combine, ST_U32)
NOID_SCAN(oracle_scan_noid_i64, int64_t, uint64_t, LD_U64, CB_I64, ST_I64)
NOID_SCAN(oracle_scan_noid_f32, float, double, LD_F64, CB_F64, ST_F64)   /* fp64 accumulator */
NOID_SCAN(oracle_scan_noid_f64, double, dd_t, dd_from, dd_combine, ST_DD) /* double-double */

/* ------------------------------------------- tolerance weight P_i (fp64) --
 * P_i = sum of |x_j| over the elements the i-th output depends on (j <= i
 * inclusive, j < i exclusive), in fp64.  It scales the fp tolerance. */
int oracle_abs_prefix_f32(const float *x, double *p, int64_t outer, int64_t len,
                          int64_t inner, int exclusive) {
    for (int64_t o = 0; o < outer; o++)
        for (int64_t k = 0; k < inner; k++) {
            double acc = 0.0;
            for (int64_t i = 0; i < len; i++) {
                int64_t at = (o * len + i) * inner + k;
                if (exclusive) { p[at] = acc; acc += fabs((double)x[at]); }
                else { acc += fabs((double)x[at]); p[at] = acc; }
            }
        }
    return 0;
}

int oracle_abs_prefix_f64(const double *x, double *p, int64_t outer, int64_t len,
                          int64_t inner, int exclusive) {
    for (int64_t o = 0; o < outer; o++)
        for (int64_t k = 0; k < inner; k++) {
            double acc = 0.0;
            for (int64_t i = 0; i < len; i++) {
                int64_t at = (o * len + i) * inner + k;
                if (exclusive) { p[at] = acc; acc += fabs(x[at]); }
                else { acc += fabs(x[at]); p[at] = acc; }
            }
        }
    return 0;
}

/* ------------------------------------------------------------ compaction --
 * Indices i (ascending, 0-based) whose element satisfies x[i] <cmp> t.  The
 * comparison is taken in the element's own precision. Returns the count. */
static int keep_f32(int cmp, float v, float t) {
    switch (cmp) {
    case O_GT: return v > t;
    case O_GE: return v >= t;
    case O_LT: return v < t;
    case O_LE: return v <= t;
    case O_EQ: return v == t;
    default: return v != t;
    }
}

/* Integer keys also take the bit predicates: bit t (0..31) of the key's
 * 32-bit pattern clear / set -- the one-bit digit of a radix sort pass. */
static int keep_i32(int cmp, int32_t v, int32_t t) {
    switch (cmp) {
    case O_GT: return v > t;
    case O_GE: return v >= t;
    case O_LT: return v < t;
    case O_LE: return v <= t;
    case O_EQ: return v == t;
    case O_BIT_CLEAR: return (((uint32_t)v >> (t & 31)) & 1u) == 0u;
    case O_BIT_SET: return (((uint32_t)v >> (t & 31)) & 1u) == 1u;
    default: return v != t;
    }
}

static int keep_u32(int cmp, uint32_t v, uint32_t t) {
    switch (cmp) {
    case O_GT: return v > t;
    case O_GE: return v >= t;
    case O_LT: return v < t;
    case O_LE: return v <= t;
    case O_EQ: return v == t;
    case O_BIT_CLEAR: return ((v >> (t & 31u)) & 1u) == 0u;
    case O_BIT_SET: return ((v >> (t & 31u)) & 1u) == 1u;
    default: return v != t;
    }
}

int64_t oracle_compact_f32(const float *x, int64_t n, int cmp, float t, int32_t *idx) {
    int64_t count = 0;
    for (int64_t i = 0; i < n; i++)
        if (keep_f32(cmp, x[i], t)) idx[count++] = (int32_t)i;
    return count;
}

int64_t oracle_compact_i32(const int32_t *x, int64_t n, int cmp, int32_t t, int32_t *idx) {
    int64_t count = 0;
    for (int64_t i = 0; i < n; i++)
        if (keep_i32(cmp, x[i], t)) idx[count++] = (int32_t)i;
    return count;
}

int64_t oracle_compact_u32(const uint32_t *x, int64_t n, int cmp, uint32_t t, int32_t *idx) {
    int64_t count = 0;
    for (int64_t i = 0; i < n; i++)
        if (keep_u32(cmp, x[i], t)) idx[count++] = (int32_t)i;
    return count;
}

/* ------------------------------------------------------------ partition --
 * Merry, "Prefix sums on GPUs", slide "Other Applications": partitioning
 * places the objects that satisfy a predicate before the others, and radix
 * sort is repeated partitioning -- which needs each part to keep the input
 * order (a stable partition).  Written out: every satisfying element in
 * increasing index order, then every other element in increasing index
 * order; vals gets the 32-bit element, idx its source index.  Returns the
 * number of satisfying elements. */
#define PARTITION(NAME, T, KEEP)                                                     \
    int64_t NAME(const T *x, int64_t n, int cmp, T t, T *vals, int32_t *idx) {       \
        int64_t k = 0;                                                               \
        for (int64_t i = 0; i < n; i++)                                              \
            if (KEEP(cmp, x[i], t)) { vals[k] = x[i]; idx[k] = (int32_t)i; k++; }    \
        int64_t at = k;                                                              \
        for (int64_t i = 0; i < n; i++)                                              \
            if (!KEEP(cmp, x[i], t)) { vals[at] = x[i]; idx[at] = (int32_t)i; at++; } \
        return k;                                                                    \
    }
PARTITION(oracle_partition_f32, float, keep_f32)
PARTITION(oracle_partition_i32, int32_t, keep_i32)
PARTITION(oracle_partition_u32, uint32_t, keep_u32)
#undef PARTITION

/* ------------------------------------------------------ segmented scan --
 * Ragged segments (the packed lists of Merry's "Output Format" and
 * "Solution" slides, AcceleratedKernels.jl PR #208's SliceScan generalised
 * to segments of any length): segment s is x[off[s] .. off[s+1]) and is
 * scanned on its own with the plain scan above, so an exclusive result
 * starts every segment at the identity.  Empty segments are allowed.
 * Returns -1 if the offsets decrease. */
#define SEGSCAN(NAME, SCAN, TX, TY)                                                     \
    int NAME(const TX *x, TY *y, const int32_t *off, int64_t nseg, int op, int exclusive) { \
        for (int64_t s = 0; s < nseg; s++) {                                            \
            const int64_t b = off[s], e = off[s + 1];                                   \
            if (e < b) return -1;                                                       \
            if (e > b) {                                                                \
                const int rc = SCAN(x + b, y + b, 1, e - b, 1, op, exclusive);          \
                if (rc != 0) return rc;                                                 \
            }                                                                           \
        }                                                                               \
        return 0;                                                                       \
    }
SEGSCAN(oracle_segscan_i32, oracle_scan_i32, int32_t, int32_t)
SEGSCAN(oracle_segscan_u32, oracle_scan_u32, uint32_t, uint32_t)
SEGSCAN(oracle_segscan_i64, oracle_scan_i64, int64_t, int64_t)
SEGSCAN(oracle_segscan_f32, oracle_scan_f32, float, double)
SEGSCAN(oracle_segscan_f64, oracle_scan_f64, double, double)
#undef SEGSCAN

/* --------------------------------------------------------------- packing --
 * offsets[0] = 0, offsets[i+1] = offsets[i] + counts[i]; returns the total
 * (offsets[n]) computed in 64 bits, so a caller can see int32 overflow. */
int64_t oracle_pack_offsets(const int32_t *counts, int64_t n, int32_t *offsets) {
    int64_t run = 0;
    offsets[0] = 0;
    for (int64_t i = 0; i < n; i++) {
        run += counts[i];
        offsets[i + 1] = (int32_t)run;
    }
    return run;
}

/* Object i writes its records at out[offsets[i] .. offsets[i+1]); record j
 * is (i + 1 + j) mod n. */
int oracle_pack_emit(const int32_t *offsets, int64_t n, int32_t *out) {
    for (int64_t i = 0; i < n; i++) {
        int64_t c = (int64_t)offsets[i + 1] - offsets[i];
        for (int64_t j = 0; j < c; j++) out[offsets[i] + j] = (int32_t)((i + 1 + j) % n);
    }
    return 0;
}

/* ----------------------------------------------------- block-size rule ----
 * AcceleratedKernels.jl PR #208, first bullet: an explicit block size is kept
 * as given; an unset one starts at the default and is lowered to the largest
 * power of two B whose tile of one item per thread plus one per-thread total
 * (2 * B * esize bytes) fits the local-memory budget, and never below 2. */
int64_t oracle_block_size(int64_t esize, int64_t budget, int64_t explicit_b,
                          int64_t default_b) {
    if (explicit_b > 0) return explicit_b;
    int64_t b = default_b;
    while (b > 2 && 2 * b * esize > budget) b /= 2;
    if (b < 2) b = 2;
    return b;
}
