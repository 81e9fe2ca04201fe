// launch.hpp -- host-side interface between the C ABI (api.hip) and the kernel
// translation units.  Each kernel family exposes a lookup that returns a
// launcher for a (dtype, op, shape) combination, or nullptr when that
// combination is not instantiated.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "pipeline.hpp"
#include "scan_wave64.h"

namespace sw64 {

// ---------------------------------------------------------------- look-back
// One launch of the persistent pipeline (pipeline.hpp): at most the resident
// capacity of workgroups of `block` threads; workgroup w scans tiles w, w+G,
// ... of block*rows*vec elements.  Segments (rows of an (outer, len, 1)
// array) are seg_len elements long; the look-back never crosses a segment
// start.
struct ScanArgs {
    PipeArgs pipe;
    const void *in;
    void *out;
    int64_t seg_len;          // elements per segment
    int32_t exclusive;        // 0 inclusive, 1 exclusive
    void *total_out;          // optional: per-segment total, written by its last tile
};
using LbLaunch = int (*)(const ScanArgs &, uint32_t grid_cap, hipStream_t);
LbLaunch find_lookback(scan_dtype_t dt, scan_op_t op, int block, int rows, int vec);
LbLaunch find_pack_lookback(int block, int rows, int vec);  // int32 sum, offsets kept cacheable

// The resident single pass (resident.hip): one 1024-thread workgroup (15
// data waves and a control wave) per `sweeps` tiles (1, or 2 for a whole
// array) of `rows` x 960 x vec elements (vec = 16 / element size), at most
// kResMaxTiles workgroups.
constexpr int kResWaves = 16;
constexpr int kResMaxRows4 = 17, kResMaxRows8 = 21;  // 68 and 84 data registers per thread
constexpr int kResMaxRows2x4 = 8, kResMaxRows2x8 = 11;  // rows per tile with two tiles: 64 and 88 registers
// Resident compactions, and resident scans with two tiles per workgroup,
// whose first tile has at most this many rows decide the residency after
// publishing it (their loads end before the decision would); longer tiles
// decide while they load.  Measured: compaction of 1e7 keys in 11-row tiles
// 18.1 us deciding early, 19.4 late; 2^21 keys in 3-row tiles 10.0 early,
// 9.1 late; scan of 1e7 fp32 in two 6-row tiles 18.6 early, 17.4 late.  A
// scan with one tile per workgroup decides late only with tiles of at most
// kResLateDecisionRows1 rows and at least kResLateDecisionTiles of them
// (graph replays, us, early against late: int32 2^18 in 69 1-row tiles 6.0
// against 5.3, 2^21 in 183 3-row tiles 9.0 against 8.3, fp32 1e6 in 131
// 2-row tiles 7.0 against 6.6; but int32 2^22 in 219 5-row tiles 10.9
// against 11.4, 2^14 in 5 tiles 4.1 against 4.6, fp64 2^16 in 35 tiles 4.7
// against 5.0).
constexpr int kResLateDecisionRows = 8;
constexpr int kResLateDecisionRows1 = 3, kResLateDecisionTiles = 64;
constexpr int64_t kResMaxTiles = 256;                // one per compute unit on MI355X
using ResLaunch = int (*)(const ScanArgs &, int rows, int sweeps, hipStream_t);
ResLaunch find_resident(scan_dtype_t dt, scan_op_t op);
ResLaunch find_resident_noid(scan_dtype_t dt, scan_op_t op);  // inclusive, no identity, no total
ResLaunch find_pack_resident();  // int32 sum, offsets kept cacheable

// Many rows that each fit one tile (rows.hip): one workgroup of kRowsBlock
// threads per row, ROWS (1, 2, 4 or 8) tile rows of kRowsBlock x vec
// elements; rows of whole 128-bit vectors.
constexpr int kRowsBlock = 256;
struct RowsArgs {
    const void *in;
    void *out;
    int64_t len;        // elements per row (a multiple of the vector width)
    uint64_t rows;      // rows (one workgroup each)
    int32_t exclusive;  // 0 inclusive, 1 exclusive
};
using RowsLaunch = int (*)(const RowsArgs &, hipStream_t);
RowsLaunch find_rows(scan_dtype_t dt, scan_op_t op, int rows);

// ---------------------------------------------------------- reduce-then-scan
// Three launches over `blocks` workgroups, each owning `chunk_tiles`
// consecutive tiles of block*rows*vec elements: reduce each chunk into a
// partial, scan the partials in one workgroup, rescan each chunk from its
// base.  `partials` (blocks carry values) lives in the workspace's
// descriptor area; the last launch zeroes it again, which leaves valid
// (untagged) descriptor words behind.
struct RtsArgs {
    const void *in;
    void *out;
    int64_t n;
    uint32_t num_tiles;
    uint32_t chunk_tiles;
    uint32_t blocks;
    int32_t exclusive;
    int32_t reverse;          // rescan the chunks in reverse (arrays larger than the caches)
    void *partials;
};
using RtsLaunch = int (*)(const RtsArgs &, hipStream_t);
RtsLaunch find_rts(scan_dtype_t dt, scan_op_t op, int block, int rows, int vec);

// ----------------------------------------------------------- segmented scan
// Ragged segments given by int32 offsets, reduce-then-scan over chunks of
// tiles with (head flag, value) pairs (segmented.hip).
struct SegArgs {
    PipeArgs pipe;            // single-pass path: the look-back pipeline (descriptors first in the workspace)
    const void *in;
    void *out;
    int64_t n;
    const int32_t *off;       // nseg + 1 offsets
    int64_t nseg;
    uint64_t *map;            // per tile: the segment holding its first element (workspace)
    uint64_t *heads;          // per tile: its head bits as planes, TILE / 4 bytes (workspace)
    void *partials;           // reduce-then-scan path: per chunk (carry value, head flag) (workspace)
    int64_t tile;             // elements per tile
    int32_t tile_log2;        // log2(tile) for a power of two, else -1
    uint32_t num_tiles;
    uint32_t chunk_tiles;
    uint32_t blocks;          // chunks (<= 8192)
    int32_t exclusive;
    uint32_t grid_cap;        // single-pass path: cap on the persistent grid (0: none)
};
using SegLaunch = int (*)(const SegArgs &, hipStream_t);
// reduce-then-scan (four launches) and single-pass (map, heads, look-back scan)
SegLaunch find_seg(scan_dtype_t dt, scan_op_t op, int block, int rows, int vec);
SegLaunch find_seg_pipe(scan_dtype_t dt, scan_op_t op, int block, int rows, int vec);

// ---------------------------------------------------------------- compaction
struct CompactArgs {
    PipeArgs pipe;
    const void *x;
    int64_t n;
    uint32_t threshold;       // bit pattern of the threshold in x's type
    int32_t *out_idx;
    int32_t *count;
};
using CompactLaunch = int (*)(const CompactArgs &, uint32_t grid_cap, hipStream_t);
CompactLaunch find_compact(scan_dtype_t x_dt, scan_cmp_t cmp, int block, int rows, int vec);
// Resident compaction (compact.hip): the resident pass's tiles of rows x 960 x
// 4 elements, at most kResCompactMaxRows rows (tile-local indices in 16 bits).
constexpr int kResCompactMaxRows = 17;
using ResCompactLaunch = int (*)(const CompactArgs &, int rows, hipStream_t);
ResCompactLaunch find_compact_resident(scan_dtype_t x_dt, scan_cmp_t cmp);
int launch_emit_neighbors(const int32_t *offsets, int64_t n, int32_t *out, hipStream_t s);

// Stable partition: a count pass, then the compaction's fused scan writing
// every element (compact.hip).
struct PartitionArgs {
    PipeArgs pipe;
    const void *x;
    int64_t n;
    uint32_t threshold;       // bit pattern of the threshold (bit index for the bit predicates)
    void *out_vals;           // n 32-bit values
    int32_t *out_idx;         // n source indices, or null
    int32_t *count;
    uint32_t count_base;      // descriptor word of the count pass's first count (after the tiles')
    uint32_t count_wgs;       // count-pass workgroups (<= 1024)
    int64_t count_chunk;      // elements per count-pass workgroup (a multiple of the vector width)
};
using PartitionLaunch = int (*)(const PartitionArgs &, uint32_t grid_cap, hipStream_t);
PartitionLaunch find_partition(scan_dtype_t x_dt, scan_cmp_t cmp, int block, int rows, int vec);
// Resident partition (compact.hip): the resident compaction's tiles; the
// count_* fields are unused.
constexpr int kResPartChunkRows = 6;  // rows staged in LDS at a time (values and 16-bit indices: 135 KiB)
using ResPartitionLaunch = int (*)(const PartitionArgs &, int rows, hipStream_t);
ResPartitionLaunch find_partition_resident(scan_dtype_t x_dt, scan_cmp_t cmp);

// ---------------------------------------------------------- large elements
// Elements of W components scanned component-wise along the middle axis of
// an (outer, len, W) array by reduce-then-scan over chunks of tiles; a tile
// is `threads` x E elements staged through LDS (element.hip).
struct ElemArgs {
    const void *in;
    void *out;
    uint32_t outer;            // segments
    int64_t len;               // elements per segment
    uint32_t chunks;           // chunks per segment (one workgroup each)
    uint32_t tiles_per_chunk;
    int32_t exclusive;
    void *partials;            // outer * chunks * W carry values, in the workspace
};
using ElemLaunch = int (*)(const ElemArgs &, int threads, hipStream_t);
// e: elements per thread (elem_e_max(width) or 1); vec: 16-byte accesses
ElemLaunch find_element(scan_dtype_t dt, scan_op_t op, int width, int e, bool vec);

// Elements per thread of an element kernel's wide variant: the largest power
// of two that keeps at most 32 component values per thread.
constexpr int elem_e_max(int w) { return w > 16 ? 1 : (w > 8 ? 2 : (w > 4 ? 4 : (w > 2 ? 8 : 16))); }

// ------------------------------------------------------------ wide columns
// (outer, len, inner) with a wide inner extent: reduce-then-scan over chunks
// of `rows` rows, workgroups of 256 threads over strips of 256 x vec columns.
struct ColArgs {
    const void *in;
    void *out;
    uint32_t outer;
    int64_t len;
    int64_t inner;
    int64_t rows;             // rows per chunk (R)
    uint32_t chunks;          // chunks per column (<= 256)
    uint32_t strips;          // column strips
    int32_t exclusive;
    void *partials;           // outer * chunks * inner carry values, in the workspace
};
using ColLaunch = int (*)(const ColArgs &, hipStream_t);
ColLaunch find_columns(scan_dtype_t dt, scan_op_t op, int vec);

// The single pass for wide inner extents (128-bit rows only): one register
// tile of kColTileRows rows x (64 x vec) columns per 1024-thread workgroup,
// grid = tiles; each tile publishes its column aggregates and adds those of
// the tiles above it in its strip (columns.hip).
constexpr int kColTileWaves = 16, kColTileRowsPerThread = 16;
constexpr int kColTileRows = kColTileWaves * kColTileRowsPerThread;
constexpr int64_t kColSingleMaxTiles = 256;     // one tile per compute unit on MI355X
constexpr int64_t kColSingleMaxRowBlocks = 64;  // tiles above a tile: at most 63 reads per column
struct ColSingleArgs {
    PipeArgs pipe;            // workspace protocol (num_tiles = tiles, the grid)
    const void *in;
    void *out;
    uint32_t outer;
    int64_t len;
    int64_t inner;
    uint32_t strips;          // column strips of 64 x vec columns
    uint32_t rblocks;         // row blocks of kColTileRows rows per strip
    int32_t exclusive;
};
using ColSingleLaunch = int (*)(const ColSingleArgs &, hipStream_t);
ColSingleLaunch find_columns_single(scan_dtype_t dt, scan_op_t op);

// -------------------------------------------------------------- utilities
// fill `words` 64-bit words with `value`; word `at` (when in range) gets `at_value`
int launch_fill_u64(void *p, uint64_t words, uint64_t value, hipStream_t s, uint64_t at = ~uint64_t(0),
                    uint64_t at_value = 0);
int launch_fill_i32(int32_t *p, int64_t count, int32_t value, hipStream_t s);
int launch_copy(const void *in, void *out, size_t bytes, hipStream_t s);

}  // namespace sw64
