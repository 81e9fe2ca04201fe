/*
 * scan_wave64.h -- C ABI of a device-wide prefix-scan library for AMD
 * Instinct MI355X (gfx950, CDNA4, 64-lane wavefronts).
 *
 * Operations (sources are the pages' titles and sections):
 *  - inclusive / exclusive scan with an associative, commutative operator
 *    and its identity: Merry, "Prefix sums on GPUs" (GPGPU2 2014), slides
 *    "Exclusive Prefix Sum" and "Inclusive Prefix Sum";
 *  - the single-pass decoupled look-back device scan with tile descriptors
 *    that move from X to A (aggregate) to P (inclusive prefix), and the
 *    reduce-then-scan alternative: The CUDA Handbook, ch. 13 "Scan", CUDA
 *    implementations, sections 13.3.3 (reduce-then-scan) and the decoupled
 *    look-back section with Figure 13-11 and Listings 13-13..13-16;
 *  - scans along one dimension and of large element types, with the block
 *    size lowered to fit a local-memory budget: AcceleratedKernels.jl PR
 *    #208 ("Fit the scans' tiles in local memory for large element types");
 *  - stream compaction, stable partitioning (one pass of a radix sort by a
 *    one-bit digit) and count-scan-emit packing: Merry's slides "Output
 *    Format", "Solution" and "Other Applications".
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers (hipMalloc'd or equivalent) on
 *    the current HIP device; the caller owns every buffer, including the
 *    workspace.  The library allocates nothing and keeps no state besides
 *    cached device properties.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every call only enqueues work on that stream and never synchronizes;
 *    results are ready when the stream has reached the call.
 *  - Return value: SCAN_OK or a negative status (see scan_status_string).
 *    Argument errors are detected on the host before anything is enqueued.
 *    Launch failures return SCAN_ERR_HIP.  Faults during execution surface
 *    at the caller's next synchronization.
 *  - n == 0 (or any zero extent) is a successful no-op, except where stated.
 *  - Integer arithmetic wraps modulo 2^bits (two's complement).
 *  - In-place use (out == in) is allowed for the scans; partial overlap is
 *    undefined.
 *  - 128-bit vector accesses are used when every array pointer is 16-byte
 *    aligned and the scanned extent keeps rows aligned; otherwise the same
 *    kernels run with element-wide accesses.
 *
 * Workspace: a caller-owned, 256-byte aligned device buffer of at least the
 * size returned by scan_plan (per call) or scan_workspace_bytes (an upper bound for any call
 * on arrays of up to `count` values).  Before its first use it must be zeroed
 * once, preferably with scan_workspace_init.  After that it is self-
 * resetting: the look-back kernels tag their tile descriptors with a per-
 * workspace epoch held in the workspace header, advance it at the end of
 * each call and clear the descriptor words a previous, larger call left
 * above their own, so no clearing launch is needed between calls.
 * scan_workspace_init records the buffer's size in the header: later calls
 * may then pass any ws_bytes (e.g. each call's own scan_plan size) on the
 * same buffer, and a call may write anywhere in the buffer so initialised
 * until it is initialised again.  A buffer zeroed by other means has no
 * recorded size; calls on it should pass the whole buffer each time (words a
 * larger call tagged beyond a smaller call's ws_bytes are then cleared only
 * by the next call that passes enough bytes to reach them).  Calls that may
 * overlap in time (different streams) need distinct workspaces.  Layout
 * (informative): bytes [0, 4096) header { uint32 epoch, uint32 error word,
 * uint64 descriptor high-water mark, uint32 mode, uint32 claim counter,
 * uint64 recorded capacity in descriptor words (byte 24), and sixteen
 * counters of started workgroups, one per 128-byte line from byte 128 },
 * then 64-bit descriptor words.
 */
#ifndef SCAN_WAVE64_H
#define SCAN_WAVE64_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SCAN_I32 = 0,
    SCAN_U32 = 1,
    SCAN_I64 = 2,
    SCAN_F32 = 3,
    SCAN_F64 = 4
} scan_dtype_t;

/* All four operators have an identity: sum 0, prod 1, max the type's lowest
 * value (-inf for floats), min the type's highest value (+inf).  Inputs with
 * NaN give unspecified results for max/min. */
typedef enum {
    SCAN_OP_SUM = 0,
    SCAN_OP_PROD = 1,
    SCAN_OP_MAX = 2,
    SCAN_OP_MIN = 3
} scan_op_t;

typedef enum {
    SCAN_ALGO_AUTO = 0,             /* the single-pass look-back (segmented: reduce-then-scan) */
    SCAN_ALGO_LOOKBACK = 1,         /* single-pass decoupled look-back */
    SCAN_ALGO_REDUCE_THEN_SCAN = 2  /* three launches, 3n traffic (comparison path) */
} scan_algo_t;

typedef enum {
    SCAN_CMP_GT = 0,
    SCAN_CMP_GE = 1,
    SCAN_CMP_LT = 2,
    SCAN_CMP_LE = 3,
    SCAN_CMP_EQ = 4,
    SCAN_CMP_NE = 5,
    SCAN_CMP_BIT_CLEAR = 6,  /* integer keys: bit `threshold` (0..31) of the 32-bit pattern is 0 */
    SCAN_CMP_BIT_SET = 7     /* integer keys: that bit is 1 */
} scan_cmp_t;

enum {
    SCAN_OK = 0,
    SCAN_ERR_INVALID_ARG = -1,  /* negative size, NULL pointer with work to do, bad enum */
    SCAN_ERR_UNSUPPORTED = -2,  /* dtype/op/tuning combination not built */
    SCAN_ERR_WORKSPACE = -3,    /* workspace NULL or smaller than required */
    SCAN_ERR_HIP = -4,          /* a HIP runtime call or launch failed */
    SCAN_ERR_OVERFLOW = -5      /* sizes exceed an index type (e.g. int32 indices) */
};

/* Optional tuning; pass NULL for the planner's defaults.  Zero fields also
 * mean "planner's choice".  block_size and items_per_thread mirror the
 * knobs of the same names in the PR; an explicit block_size is kept as
 * given (the LDS-budget rule only lowers an unset one). */
typedef struct {
    int32_t block_size;        /* threads per workgroup: 64..1024, multiple of 64 */
    int32_t items_per_thread;  /* elements per thread per tile (a multiple of
                                  the 128-bit vector width; the element-wide
                                  fallback snaps it to its nearest built shape) */
    int64_t local_mem_bytes;   /* LDS budget per workgroup for large elements
                                  (default 32 KiB, the PR's) */
    int32_t algo;              /* scan_algo_t */
    int32_t rts_blocks;        /* workgroup count C of reduce-then-scan */
    int32_t spin_limit;        /* polls of one look-back window before a tile
                                  gives up and flags an error (default 2^22,
                                  a few seconds); tests force tiny values */
    int32_t grid_blocks;       /* cap on the persistent look-back grid (default:
                                  every workgroup that can be resident) */
    int32_t mode_limit;        /* polls a call waits for all of its workgroups
                                  to start before it claims tiles dynamically
                                  instead (default 512); tests force tiny values */
    int32_t no_identity;       /* nonzero: compute without the operator's
                                  identity, as for an operator that has none
                                  (AcceleratedKernels.jl PR #208, description,
                                  first bullet: "Optional" partials): partial
                                  results carry a presence flag instead, so
                                  e.g. a sum of -0.0 values stays -0.0.
                                  Inclusive scans of whole arrays and of rows
                                  (scan_inclusive, scan_dim with inner == 1;
                                  single pass: the look-back pipeline, or the
                                  resident pass where the plain scan takes
                                  it); anything else returns
                                  SCAN_ERR_UNSUPPORTED, exclusive scans
                                  included (no value for element 0) */
    int32_t delay_stride;      /* test aid for the look-back's waits: with
                                  delay_stride > 0, every tile t with
                                  t % delay_stride == delay_stride - 1 waits
                                  delay_sleeps periods of about 1.7 us before
                                  publishing its aggregate (0: off) */
    int32_t delay_sleeps;
    int32_t resident_sweeps;   /* resident single pass over a whole array:
                                  1 holds one tile per workgroup (the look-back
                                  between all loads and all stores), 2 two
                                  where they fit (the second tile's loads and
                                  the first's stores overlapping the
                                  look-backs); 0: two from 28 MiB up
                                  for 4-byte elements, 40 MiB for 8-byte */
} scan_tuning_t;

/* Kernel family a call runs (reported by scan_plan). */
typedef enum {
    SCAN_KERNEL_NONE = 0,
    SCAN_KERNEL_LOOKBACK = 1,   /* scalar elements, segmented single-pass look-back */
    SCAN_KERNEL_RTS = 2,        /* reduce-then-scan, three launches */
    SCAN_KERNEL_ELEMENT = 3,    /* element = `inner` components, staged through LDS */
    SCAN_KERNEL_COLUMNS = 4,    /* wide inner extent: column strips, chunked rows */
    SCAN_KERNEL_COMPACT = 5,    /* fused predicate + scan + scatter */
    SCAN_KERNEL_PACK = 6,       /* exclusive int32 scan + total */
    SCAN_KERNEL_PARTITION = 7,  /* count pass, then fused predicate + scan + two-sided scatter */
    SCAN_KERNEL_SEGMENTED = 8,  /* ragged segments: tile map, then reduce-then-scan of (head, value) pairs */
    SCAN_KERNEL_COLUMNS_LOOKBACK = 9, /* wide inner extent in one pass: register tiles of 256 rows, each adding
                                         the column aggregates of the tiles above it */
    SCAN_KERNEL_RESIDENT = 10,        /* arrays of at most 256 register tiles (one per compute unit): each tile
                                         loaded once, every earlier tile's aggregate read in one round trip */
    SCAN_KERNEL_COMPACT_RESIDENT = 11, /* compaction of such arrays in the same way: counts by ballots, selected
                                          indices staged in LDS, one contiguous range written per tile */
    SCAN_KERNEL_PARTITION_RESIDENT = 12, /* stable partition of such arrays in one launch: every tile reads all
                                            tiles' counts, each element goes straight to its slot */
    SCAN_KERNEL_ROWS = 13                /* many rows that each fit one tile: one workgroup per row, no
                                            workspace traffic (scan_dim along the contiguous axis) */
} scan_kernel_t;

typedef struct {
    int32_t kernel;            /* scan_kernel_t */
    int32_t block_size;        /* threads per workgroup */
    int32_t items_per_thread;  /* elements (or components) per thread per tile */
    int32_t vec;               /* elements per vector access (1 = element-wide) */
    int64_t tile_elems;        /* elements per tile */
    int64_t num_tiles;         /* tiles of the main launch */
    int64_t lds_bytes;         /* LDS per workgroup of the main launch */
    int64_t workspace_bytes;   /* workspace this call needs */
    int32_t launches;          /* kernel launches the call enqueues */
    int32_t carry_words;       /* 64-bit descriptor words per tile (look-back kernels; carry
                                  values per partial for reduce-then-scan) */
    int32_t tiles_per_block;   /* resident pass: tiles each workgroup holds (1, or 2
                                  for a whole array, see resident_sweeps); 0 for
                                  the other kernels */
} scan_plan_t;

/* Which call scan_plan describes. */
typedef enum {
    SCAN_CALL_SCAN = 0,        /* scan_inclusive / scan_exclusive / scan_dim */
    SCAN_CALL_COMPACT = 1,     /* compact_if (dtype = x dtype) */
    SCAN_CALL_PACK = 2,        /* pack_offsets (dtype must be SCAN_I32) */
    SCAN_CALL_PARTITION = 3,   /* partition_if (dtype = x dtype) */
    SCAN_CALL_SEGMENTED = 4    /* scan_segmented (outer = segments, len = elements, inner = 1) */
} scan_call_t;

/* Host only: the launch a call with these arguments would enqueue. */
int scan_plan(scan_call_t call, scan_dtype_t dtype, scan_op_t op, int64_t outer,
              int64_t len, int64_t inner, const scan_tuning_t *tuning,
              scan_plan_t *plan);

/* Upper bound on the workspace bytes of any call on arrays of at most
 * `count` values (components) of `dtype`, with any op and tuning. */
size_t scan_workspace_bytes(scan_dtype_t dtype, int64_t count);

/* Zero a workspace and record its size in its header (one fill kernel).
 * Required once before first use (see the workspace notes above). */
int scan_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Diagnostic (synchronizes `stream`): copy the workspace's error word to
 * *error.  Bit 0 means a wait gave up after spin_limit polls (a look-back
 * window), e.g. because the workspace was not zeroed or was used by
 * overlapping calls: the results of that call are invalid and the workspace
 * must be re-initialised.  Bit 1 is not used.
 * Bit 2 means a call could not confirm that all of its workgroups were
 * resident and claimed tiles one by one instead (results valid, slower).
 * None is set in normal operation; the word stays set until re-init. */
int scan_workspace_error(const void *ws, int32_t *error, void *stream);

/* Inclusive scan of n elements of `width` components each (AoS structs;
 * width 1 for plain arrays); the op is applied component-wise.
 * out[i] = in[0] (+) ... (+) in[i]. */
int scan_inclusive(const void *in, void *out, int64_t n, scan_dtype_t dtype,
                   scan_op_t op, int32_t width, void *ws, size_t ws_bytes,
                   const scan_tuning_t *tuning, void *stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): scan_inclusive without a
 * workspace argument.  The call allocates nothing.  Its workspace is a
 * device array inside the library, SCAN_NOALLOC_SCRATCH_BYTES (1 MiB) on each
 * GPU, held from that GPU's first call until the process ends.  The first
 * call on a GPU zeroes the array with one extra fill kernel on `stream`.
 * A call whose plan (scan_plan) needs a larger workspace returns
 * SCAN_ERR_WORKSPACE before anything is enqueued: e.g. fp32 sums of up to
 * about 2.5e9 elements fit, fp64 sums of up to about 4.6e8.  Every call on
 * one GPU shares that GPU's array, which keeps the last call's contents:
 * calls that may overlap in time on one GPU (different streams, or several
 * host threads without ordering) race and give wrong results; order them on
 * one stream.  A call that reports a timed-out wait (see
 * scan_workspace_error) leaves the array unusable until the process ends. */
#define SCAN_NOALLOC_SCRATCH_BYTES (1u << 20)
int scan_inclusive_noalloc(const void *in, void *out, int64_t n, scan_dtype_t dtype,
                           scan_op_t op, int32_t width, const scan_tuning_t *tuning,
                           void *stream);

/* Exclusive scan: out[0] = identity, out[i] = in[0] (+) ... (+) in[i-1]. */
int scan_exclusive(const void *in, void *out, int64_t n, scan_dtype_t dtype,
                   scan_op_t op, int32_t width, void *ws, size_t ws_bytes,
                   const scan_tuning_t *tuning, void *stream);

/* Scan of a dense row-major array viewed as (outer, len, inner) along the
 * middle axis: element (o, i, k) at o*len*inner + i*inner + k.  A (R, C)
 * matrix scanned along each row is (R, C, 1); along each column (1, R, C). */
int scan_dim(const void *in, void *out, int64_t outer, int64_t len, int64_t inner,
             scan_dtype_t dtype, scan_op_t op, int exclusive, void *ws,
             size_t ws_bytes, const scan_tuning_t *tuning, void *stream);

/* Scan of ragged segments: segment s is in[offsets[s] .. offsets[s+1]) and
 * is scanned on its own, so an inclusive result restarts at every segment's
 * first element and an exclusive one puts the identity there (Merry,
 * "Prefix sums on GPUs", slides "Output Format" and "Solution": the packed
 * lists whose offsets pack_offsets writes; AcceleratedKernels.jl PR #208's
 * SliceScan with segments of any length).  offsets: nseg + 1 device int32,
 * non-decreasing, offsets[0] = 0, offsets[nseg] = n; empty segments are
 * allowed.  Offsets that break this give unspecified results (no access
 * outside in, out, offsets or the workspace).  out may equal in.  Default
 * (algo AUTO or REDUCE_THEN_SCAN): four launches (tile map, reduce,
 * partials, rescan; reduce-then-scan of (head flag, value) pairs).  algo
 * LOOKBACK: three launches (tile map, heads, then one pass on the look-back
 * pipeline whose tiles combine (flag, value) carries in tile order).
 * n > INT32_MAX -> SCAN_ERR_OVERFLOW; n == 0 is a no-op; n > 0 with
 * nseg == 0 -> SCAN_ERR_INVALID_ARG. */
int scan_segmented(const void *in, void *out, int64_t n, const int32_t *offsets,
                   int64_t nseg, scan_dtype_t dtype, scan_op_t op, int exclusive,
                   void *ws, size_t ws_bytes, const scan_tuning_t *tuning, void *stream);

/* Stream compaction: writes, in increasing order, every 0-based index i with
 * x[i] <cmp> threshold to out_idx, and the number written to *d_count (a
 * device int32).  x_dtype is SCAN_F32, SCAN_I32 or SCAN_U32; the threshold
 * is converted to x's type once (fp32 rounded, integers clamped to the
 * type's range and truncated) and compared in that precision.  The bit
 * predicates take integer keys and a threshold that is a bit index 0..31
 * (else SCAN_ERR_INVALID_ARG).  out_idx must hold n entries (the worst
 * case).  n > INT32_MAX -> SCAN_ERR_OVERFLOW.  n == 0 writes *d_count = 0. */
int compact_if(const void *x, int64_t n, scan_dtype_t x_dtype, scan_cmp_t cmp,
               double threshold, int32_t *out_idx, int32_t *d_count, void *ws,
               size_t ws_bytes, const scan_tuning_t *tuning, void *stream);

/* Stable partition (Merry, "Prefix sums on GPUs", slide "Other
 * Applications": partitioning puts the objects that satisfy a predicate
 * before the others; radix sort is repeated partitioning, which needs each
 * part in input order).  Writes the k elements with x[i] <cmp> threshold to
 * out_vals[0..k) and the others to out_vals[k..n), each part in increasing
 * i; out_idx (may be NULL) gets each output's source index i; *d_count = k.
 * x, out_vals: n 32-bit values of x_dtype (SCAN_F32, SCAN_I32, SCAN_U32);
 * predicates and threshold as for compact_if.  With SCAN_CMP_BIT_CLEAR and
 * bit b this is one pass of an LSD radix sort by a one-bit digit.  Two
 * launches (a count pass, then the scan-and-scatter pass); x must not
 * overlap the outputs.  n > INT32_MAX -> SCAN_ERR_OVERFLOW; n == 0 writes
 * *d_count = 0. */
int partition_if(const void *x, int64_t n, scan_dtype_t x_dtype, scan_cmp_t cmp,
                 double threshold, void *out_vals, int32_t *out_idx, int32_t *d_count,
                 void *ws, size_t ws_bytes, const scan_tuning_t *tuning, void *stream);

/* Count-scan-emit, step 2: offsets[i] = counts[0] + ... + counts[i-1] for
 * i <= n (offsets has n + 1 entries; offsets[n] is the total).  Counts must
 * be non-negative and their total must fit int32 (it wraps otherwise).
 * n == 0 writes offsets[0] = 0. */
int pack_offsets(const int32_t *counts, int64_t n, int32_t *offsets, void *ws,
                 size_t ws_bytes, const scan_tuning_t *tuning, void *stream);

/* Count-scan-emit, step 3 (synthetic records): object i writes its
 * offsets[i+1]-offsets[i] records at out[offsets[i] ...]; its j-th record is
 * (i + 1 + j) mod n.  offsets must be non-decreasing from offsets[0] >= 0
 * (as pack_offsets writes them); out must hold offsets[n] entries and needs
 * only int32 alignment.  Nothing outside out[offsets[0] .. offsets[n]) is
 * written. */
int pack_emit_neighbors(const int32_t *offsets, int64_t n, int32_t *out, void *stream);

/* Measurement aid: copy `bytes` (multiple of 16, 16-byte aligned pointers)
 * with the fastest plain copy measured on MI355X (one 128-bit nontemporal
 * load and store per thread, 4 KiB per workgroup): the attainable read+write
 * bandwidth that a one-read, one-write scan is compared with. */
int scan_copy(const void *in, void *out, size_t bytes, void *stream);

/* Static description of a status code. */
const char *scan_status_string(int status);

/* Library version string. */
const char *scan_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SCAN_WAVE64_H */
