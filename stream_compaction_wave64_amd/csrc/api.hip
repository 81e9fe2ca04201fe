// api.hip -- the C ABI (include/scan_wave64.h): argument checks, the tile
// planner and kernel selection.  Everything here runs on the host; every
// arithmetic step of a scan runs in the kernels.
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "launch.hpp"
#include "scan_wave64.h"

namespace sw64 {

#define SW64_DECLARE_PER_TYPE(name, ret)              \
    ret name##_i32(scan_op_t, int, int, int);       \
    ret name##_u32(scan_op_t, int, int, int);       \
    ret name##_i64(scan_op_t, int, int, int);       \
    ret name##_f32(scan_op_t, int, int, int);       \
    ret name##_f64(scan_op_t, int, int, int);
SW64_DECLARE_PER_TYPE(find_lookback, LbLaunch)
SW64_DECLARE_PER_TYPE(find_noid, LbLaunch)
SW64_DECLARE_PER_TYPE(find_rts, RtsLaunch)
SW64_DECLARE_PER_TYPE(find_seg, SegLaunch)
SW64_DECLARE_PER_TYPE(find_seg_pipe, SegLaunch)
#undef SW64_DECLARE_PER_TYPE
ElemLaunch find_element_i32(scan_op_t, int, int, bool);
ElemLaunch find_element_u32(scan_op_t, int, int, bool);
ElemLaunch find_element_i64(scan_op_t, int, int, bool);
ElemLaunch find_element_f32(scan_op_t, int, int, bool);
ElemLaunch find_element_f64(scan_op_t, int, int, bool);

CompactLaunch find_compact_i32(scan_cmp_t, int, int, int);
CompactLaunch find_compact_u32(scan_cmp_t, int, int, int);
CompactLaunch find_compact_f32(scan_cmp_t, int, int, int);
PartitionLaunch find_partition_i32(scan_cmp_t, int, int, int);
PartitionLaunch find_partition_u32(scan_cmp_t, int, int, int);
PartitionLaunch find_partition_f32(scan_cmp_t, int, int, int);

CompactLaunch find_compact(scan_dtype_t dt, scan_cmp_t cmp, int block, int rows, int vec) {
    if (dt == SCAN_F32) return find_compact_f32(cmp, block, rows, vec);
    if (dt == SCAN_I32) return find_compact_i32(cmp, block, rows, vec);
    if (dt == SCAN_U32) return find_compact_u32(cmp, block, rows, vec);
    return nullptr;
}

PartitionLaunch find_partition(scan_dtype_t dt, scan_cmp_t cmp, int block, int rows, int vec) {
    if (dt == SCAN_F32) return find_partition_f32(cmp, block, rows, vec);
    if (dt == SCAN_I32) return find_partition_i32(cmp, block, rows, vec);
    if (dt == SCAN_U32) return find_partition_u32(cmp, block, rows, vec);
    return nullptr;
}

ColLaunch find_columns_i32(scan_op_t, int);
ColLaunch find_columns_u32(scan_op_t, int);
ColLaunch find_columns_i64(scan_op_t, int);
ColLaunch find_columns_f32(scan_op_t, int);
ColLaunch find_columns_f64(scan_op_t, int);

ResCompactLaunch find_compact_resident_i32(scan_cmp_t);
ResCompactLaunch find_compact_resident_u32(scan_cmp_t);
ResCompactLaunch find_compact_resident_f32(scan_cmp_t);

ResCompactLaunch find_compact_resident(scan_dtype_t dt, scan_cmp_t cmp) {
    if (dt == SCAN_F32) return find_compact_resident_f32(cmp);
    if (dt == SCAN_I32) return find_compact_resident_i32(cmp);
    if (dt == SCAN_U32) return find_compact_resident_u32(cmp);
    return nullptr;
}

ResPartitionLaunch find_partition_resident_i32(scan_cmp_t);
ResPartitionLaunch find_partition_resident_u32(scan_cmp_t);
ResPartitionLaunch find_partition_resident_f32(scan_cmp_t);

ResPartitionLaunch find_partition_resident(scan_dtype_t dt, scan_cmp_t cmp) {
    if (dt == SCAN_F32) return find_partition_resident_f32(cmp);
    if (dt == SCAN_I32) return find_partition_resident_i32(cmp);
    if (dt == SCAN_U32) return find_partition_resident_u32(cmp);
    return nullptr;
}

ResLaunch find_resident_i32(scan_op_t);
ResLaunch find_resident_u32(scan_op_t);
ResLaunch find_resident_i64(scan_op_t);
ResLaunch find_resident_f32(scan_op_t);
ResLaunch find_resident_f64(scan_op_t);

ResLaunch find_resident(scan_dtype_t dt, scan_op_t op) {
    switch (dt) {
    case SCAN_I32: return find_resident_i32(op);
    case SCAN_U32: return find_resident_u32(op);
    case SCAN_I64: return find_resident_i64(op);
    case SCAN_F32: return find_resident_f32(op);
    case SCAN_F64: return find_resident_f64(op);
    }
    return nullptr;
}

RowsLaunch find_rows_i32(scan_op_t, int);
RowsLaunch find_rows_u32(scan_op_t, int);
RowsLaunch find_rows_i64(scan_op_t, int);
RowsLaunch find_rows_f32(scan_op_t, int);
RowsLaunch find_rows_f64(scan_op_t, int);

RowsLaunch find_rows(scan_dtype_t dt, scan_op_t op, int rows) {
    switch (dt) {
    case SCAN_I32: return find_rows_i32(op, rows);
    case SCAN_U32: return find_rows_u32(op, rows);
    case SCAN_I64: return find_rows_i64(op, rows);
    case SCAN_F32: return find_rows_f32(op, rows);
    case SCAN_F64: return find_rows_f64(op, rows);
    }
    return nullptr;
}

ResLaunch find_resident_noid_i32(scan_op_t);
ResLaunch find_resident_noid_u32(scan_op_t);
ResLaunch find_resident_noid_i64(scan_op_t);
ResLaunch find_resident_noid_f32(scan_op_t);
ResLaunch find_resident_noid_f64(scan_op_t);

ResLaunch find_resident_noid(scan_dtype_t dt, scan_op_t op) {
    switch (dt) {
    case SCAN_I32: return find_resident_noid_i32(op);
    case SCAN_U32: return find_resident_noid_u32(op);
    case SCAN_I64: return find_resident_noid_i64(op);
    case SCAN_F32: return find_resident_noid_f32(op);
    case SCAN_F64: return find_resident_noid_f64(op);
    }
    return nullptr;
}

ColSingleLaunch find_columns_single_i32(scan_op_t);
ColSingleLaunch find_columns_single_u32(scan_op_t);
ColSingleLaunch find_columns_single_i64(scan_op_t);
ColSingleLaunch find_columns_single_f32(scan_op_t);
ColSingleLaunch find_columns_single_f64(scan_op_t);

ColSingleLaunch find_columns_single(scan_dtype_t dt, scan_op_t op) {
    switch (dt) {
    case SCAN_I32: return find_columns_single_i32(op);
    case SCAN_U32: return find_columns_single_u32(op);
    case SCAN_I64: return find_columns_single_i64(op);
    case SCAN_F32: return find_columns_single_f32(op);
    case SCAN_F64: return find_columns_single_f64(op);
    }
    return nullptr;
}

ColLaunch find_columns(scan_dtype_t dt, scan_op_t op, int vec) {
    switch (dt) {
    case SCAN_I32: return find_columns_i32(op, vec);
    case SCAN_U32: return find_columns_u32(op, vec);
    case SCAN_I64: return find_columns_i64(op, vec);
    case SCAN_F32: return find_columns_f32(op, vec);
    case SCAN_F64: return find_columns_f64(op, vec);
    }
    return nullptr;
}

ElemLaunch find_element(scan_dtype_t dt, scan_op_t op, int width, int e, bool vec) {
    switch (dt) {
    case SCAN_I32: return find_element_i32(op, width, e, vec);
    case SCAN_U32: return find_element_u32(op, width, e, vec);
    case SCAN_I64: return find_element_i64(op, width, e, vec);
    case SCAN_F32: return find_element_f32(op, width, e, vec);
    case SCAN_F64: return find_element_f64(op, width, e, vec);
    }
    return nullptr;
}

LbLaunch find_lookback(scan_dtype_t dt, scan_op_t op, int block, int rows, int vec) {
    switch (dt) {
    case SCAN_I32: return find_lookback_i32(op, block, rows, vec);
    case SCAN_U32: return find_lookback_u32(op, block, rows, vec);
    case SCAN_I64: return find_lookback_i64(op, block, rows, vec);
    case SCAN_F32: return find_lookback_f32(op, block, rows, vec);
    case SCAN_F64: return find_lookback_f64(op, block, rows, vec);
    }
    return nullptr;
}

// the look-back scan that never uses the operator's identity (noid.hip)
LbLaunch find_noid(scan_dtype_t dt, scan_op_t op, int block, int rows, int vec) {
    switch (dt) {
    case SCAN_I32: return find_noid_i32(op, block, rows, vec);
    case SCAN_U32: return find_noid_u32(op, block, rows, vec);
    case SCAN_I64: return find_noid_i64(op, block, rows, vec);
    case SCAN_F32: return find_noid_f32(op, block, rows, vec);
    case SCAN_F64: return find_noid_f64(op, block, rows, vec);
    }
    return nullptr;
}

SegLaunch find_seg(scan_dtype_t dt, scan_op_t op, int block, int rows, int vec) {
    switch (dt) {
    case SCAN_I32: return find_seg_i32(op, block, rows, vec);
    case SCAN_U32: return find_seg_u32(op, block, rows, vec);
    case SCAN_I64: return find_seg_i64(op, block, rows, vec);
    case SCAN_F32: return find_seg_f32(op, block, rows, vec);
    case SCAN_F64: return find_seg_f64(op, block, rows, vec);
    }
    return nullptr;
}

SegLaunch find_seg_pipe(scan_dtype_t dt, scan_op_t op, int block, int rows, int vec) {
    switch (dt) {
    case SCAN_I32: return find_seg_pipe_i32(op, block, rows, vec);
    case SCAN_U32: return find_seg_pipe_u32(op, block, rows, vec);
    case SCAN_I64: return find_seg_pipe_i64(op, block, rows, vec);
    case SCAN_F32: return find_seg_pipe_f32(op, block, rows, vec);
    case SCAN_F64: return find_seg_pipe_f64(op, block, rows, vec);
    }
    return nullptr;
}

RtsLaunch find_rts(scan_dtype_t dt, scan_op_t op, int block, int rows, int vec) {
    switch (dt) {
    case SCAN_I32: return find_rts_i32(op, block, rows, vec);
    case SCAN_U32: return find_rts_u32(op, block, rows, vec);
    case SCAN_I64: return find_rts_i64(op, block, rows, vec);
    case SCAN_F32: return find_rts_f32(op, block, rows, vec);
    case SCAN_F64: return find_rts_f64(op, block, rows, vec);
    }
    return nullptr;
}

namespace {

constexpr size_t kHeader = kWsHeaderBytes;  // workspace header bytes (WsHeader)
constexpr uint32_t kDefaultSpinLimit = 1u << 22;
constexpr uint32_t kDefaultModeLimit = 512;
constexpr int kDefaultBlock = 512;  // threads per workgroup of the tiled kernels
constexpr int kDefaultRtsBlocks = 1024;               // C of reduce-then-scan
constexpr int64_t kDefaultLocalMem = 32 * 1024;       // LDS budget of the large-element rule (AcceleratedKernels.jl PR #208)
constexpr int64_t kSmallArrayTiles = 256;             // one tile per CU: the small-array shape rule
// Rows of a 2-D array take the resident single pass from this many bytes
// up (below it, when first measured, the small-array tiles won for whole
// arrays too); whole arrays take it at every size (graph replays of
// back-to-back calls, resident against small-array tiles, us: int32 2^14
// 3.9 against 7.4, 2^18 6.1 against 7.4, 2^20 7.2 against 8.5; fp32 1e6 7.2
// against 9.0; fp64 2^16 5.0 against 7.4, 2^19 6.9 against 9.5).
constexpr int64_t kResMinBytes = int64_t(8) << 20;
// whole arrays: two tiles per workgroup from here (4-byte and 8-byte
// elements; graph replays, us, one tile against two: int32 24 MiB 14.4
// against 15.4, 28 MiB 15.7 against 14.7; fp64 32 MiB 17.9 against 19.1,
// 36-40 MiB level, 48 MiB 24.3 against 23.3)
constexpr int64_t kResTwoTileBytes4 = int64_t(28) << 20, kResTwoTileBytes8 = int64_t(40) << 20;
constexpr int64_t kElemTileLocalMem = 64 * 1024;      // default bound on an element tile's E (default dynamic LDS limit)
constexpr int kElemDefaultBlock = 256;                // large elements: start of the rule
constexpr int64_t kElemChunks = 2048;  // large elements: workgroups per launch (<= 8192, the partials pass)

// AcceleratedKernels.jl PR #208, first bullet: an explicit block size is kept
// as given; an unset one starts at the default and is lowered to the largest
// power of two B whose one-item-per-thread tile plus one per-thread total
// (2 * B * esize bytes) fits the local-memory budget, never below 2.
int64_t element_block(int64_t esize, int64_t budget, int64_t explicit_b, int64_t default_b) {
    if (explicit_b > 0) return explicit_b;
    int64_t b = default_b;
    while (b > 2 && 2 * b * esize > budget) b /= 2;
    return b < 2 ? 2 : b;
}

bool valid_dtype(int dt) { return dt >= SCAN_I32 && dt <= SCAN_F64; }
bool valid_op(int op) { return op >= SCAN_OP_SUM && op <= SCAN_OP_MIN; }
bool valid_cmp(int c) { return c >= SCAN_CMP_GT && c <= SCAN_CMP_BIT_SET; }
bool bit_cmp(int c) { return c == SCAN_CMP_BIT_CLEAR || c == SCAN_CMP_BIT_SET; }

int dtype_bytes(scan_dtype_t dt) { return (dt == SCAN_I64 || dt == SCAN_F64) ? 8 : 4; }

// Bytes of the value a tile hands to its successors (see Carry in device.hpp).
int carry_bytes(scan_dtype_t dt, scan_op_t op) {
    if (dt == SCAN_F32 && (op == SCAN_OP_SUM || op == SCAN_OP_PROD)) return 8;
    return dtype_bytes(dt);
}

// 64-bit descriptor words per tile of a scalar look-back scan: one 32-bit
// chunk per word, except fp32 sums and products, whose fp64 carry packs into
// one word (DescTrunc in device.hpp).
int desc_words(scan_dtype_t dt, scan_op_t op) {
    if (dt == SCAN_F32 && (op == SCAN_OP_SUM || op == SCAN_OP_PROD)) return 1;
    return carry_bytes(dt, op) / 4;
}

size_t round_up(size_t x, size_t m) { return (x + m - 1) / m * m; }

scan_tuning_t tuning_or_default(const scan_tuning_t *t) {
    scan_tuning_t d;
    memset(&d, 0, sizeof(d));
    if (t) d = *t;
    return d;
}

// Plan of a tiled launch over scalar elements (look-back, reduce-then-scan
// or compaction).
struct TilePlan {
    int kernel;               // scan_kernel_t
    int block, rows, vec;
    int sweeps = 1;           // resident pass: tiles per workgroup
    int64_t tile;
    int64_t tiles_per_seg, num_tiles;
    int carry_words;
    int64_t rts_blocks, rts_chunk;
    size_t ws_bytes;
    int launches;
    int width;                // components per element (element kernel)
    int64_t col_rows, col_chunks, col_strips;  // column kernel
};

// Shape of a tile: the caller's default (block_default threads x rows_default
// rows of 128-bit vectors), or block_size / items_per_thread from the
// tuning.  The element-wide fallback (misaligned data or a length that
// breaks the vector alignment) is built for the default and one-row shapes:
// a tuned shape snaps to the nearer.  Kernels with a control wave (`ctrl`)
// give the tile block - 64 threads.
template <class Find>
int plan_shape(int esize, bool vec_ok, const scan_tuning_t &tu, TilePlan &p, Find find, bool ctrl,
               int rows_default, int block_default) {
    const int vmax = 16 / esize;
    p.vec = vec_ok ? vmax : 1;
    p.block = tu.block_size > 0 ? tu.block_size : block_default;
    int ipt = tu.items_per_thread > 0 ? tu.items_per_thread : rows_default * vmax;
    if (p.vec == 1 && tu.items_per_thread <= 0) ipt = rows_default;
    if (ipt % p.vec != 0) return SCAN_ERR_UNSUPPORTED;
    p.rows = ipt / p.vec;
    if (p.vec == 1 && !find(p.block, p.rows, 1)) {
        p.rows = p.rows >= rows_default ? rows_default : 1;
        p.block = p.rows == 1 ? 256 : block_default;
    }
    if (!find(p.block, p.rows, p.vec)) return SCAN_ERR_UNSUPPORTED;
    p.tile = int64_t(ctrl ? p.block - 64 : p.block) * p.rows * p.vec;
    return SCAN_OK;
}

int plan_scan(scan_dtype_t dt, scan_op_t op, int64_t outer, int64_t len, bool aligned, const scan_tuning_t &tu,
              TilePlan &p) {
    const int esize = dtype_bytes(dt);
    const bool rts = tu.algo == SCAN_ALGO_REDUCE_THEN_SCAN;
    if (rts && outer != 1) return SCAN_ERR_UNSUPPORTED;  // reduce-then-scan: whole arrays only
    if (rts && tu.no_identity) return SCAN_ERR_UNSUPPORTED;  // without an identity: the look-back only
    const bool vec_ok = aligned && len % (16 / esize) == 0;
    // the look-back kernels of this call: with or without the identity
    auto find_lb = [&](int b, int r, int v) {
        return tu.no_identity ? find_noid(dt, op, b, r, v) : find_lookback(dt, op, b, r, v);
    };
    // default shapes: reduce-then-scan 512 threads x 8 rows (4 for 8-byte
    // elements); look-back 768 x 7 (512 x 8 for 8-byte elements), its tiles
    // bounded by the two LDS stashes of the pipeline
    int rc = rts ? plan_shape(
                       esize, vec_ok, tu, p,
                       [&](int b, int r, int v) { return find_rts(dt, op, b, r, v) != nullptr; }, false,
                       esize == 8 ? 4 : 8, kDefaultBlock)
                 : plan_shape(
                       esize, vec_ok, tu, p,
                       [&](int b, int r, int v) { return find_lb(b, r, v) != nullptr; }, true,
                       esize == 8 ? 8 : 7, esize == 8 ? kDefaultBlock : 768);
    if (rc != SCAN_OK) return rc;
    const bool shape_free = !rts && tu.block_size <= 0 && tu.items_per_thread <= 0;
    if (shape_free && len < p.tile) {
        // Short segments: the fewest rows of a 512-thread tile that hold a
        // whole segment, so each segment is one tile (no look-back) with
        // little of it idle.
        for (int r : {1, 2, 3, 5}) {
            const int64_t t = int64_t(kDefaultBlock - 64) * r * p.vec;
            if (t < p.tile && t >= len && find_lb(kDefaultBlock, r, p.vec) != nullptr) {
                p.block = kDefaultBlock;
                p.rows = r;
                p.tile = t;
                break;
            }
        }
    } else if (shape_free && outer == 1 && p.vec > 1 && p.rows > 5) {
        // Small whole arrays: 512 x 5 tiles finish sooner while they cover
        // the array at no more than one tile per CU (more CUs reading, each a
        // shorter tile: int32 2^20 took 8.9 us against 11.2, fp64 2^20 12.1
        // against 12.8); past that the default's longer tiles win.
        const int64_t t = int64_t(kDefaultBlock - 64) * 5 * p.vec;
        if ((len + t - 1) / t <= kSmallArrayTiles && find_lb(kDefaultBlock, 5, p.vec) != nullptr) {
            p.block = kDefaultBlock;
            p.rows = 5;
            p.tile = t;
        }
    }
    p.tiles_per_seg = (len + p.tile - 1) / p.tile;
    p.num_tiles = outer * p.tiles_per_seg;
    if (p.num_tiles > int64_t(INT32_MAX)) return SCAN_ERR_OVERFLOW;  // grid x limit
    p.carry_words = rts ? carry_bytes(dt, op) / 4 : desc_words(dt, op);
    // Arrays that fit one register tile per compute unit: the resident single
    // pass, with the fewest rows per tile that keep the tiles within
    // kResMaxTiles (the most compute units reading).  Only for the default
    // shape, without a grid cap, scans of 128-bit rows (without an identity
    // too: inclusive, as everywhere).
    // A whole array of 28 MiB or more (4-byte elements; 40 MiB, 8-byte)
    // takes two tiles per workgroup where they fit (the second tile's loads
    // and the first's stores overlap the look-backs: fp32 1e7 20.4 -> 16.8
    // us, fp64 1e7 35.5 -> 34.0, int32 2^23 17.9 -> 16.2); below that the
    // fewer, longer workgroups lose (int32 2^22 10.6 -> 13.3 us).  The
    // tuning can ask for either.
    if (shape_free && tu.grid_blocks <= 0 && vec_ok && (outer == 1 || outer * len * esize >= kResMinBytes) &&
        (tu.no_identity ? find_resident_noid(dt, op) : find_resident(dt, op)) != nullptr) {
        const int64_t re = int64_t(kResWaves - 1) * kWave * (16 / esize);  // the data waves
        const bool two = outer == 1 && (tu.resident_sweeps == 2 ||
                                        (tu.resident_sweeps != 1 &&
                                         len * esize >= (esize == 8 ? kResTwoTileBytes8 : kResTwoTileBytes4)));
        for (int sw = two ? 2 : 1; sw >= 1; sw--) {
            const int maxr = sw == 2 ? (esize == 8 ? kResMaxRows2x8 : kResMaxRows2x4)
                                     : (esize == 8 ? kResMaxRows8 : kResMaxRows4);
            for (int r = 1; r <= maxr; r++) {
                const int64_t tps = (len + r * re - 1) / (r * re);
                if ((outer * tps + sw - 1) / sw <= kResMaxTiles) {
                    p.kernel = SCAN_KERNEL_RESIDENT;
                    p.block = kResWaves * kWave;
                    p.rows = r;
                    p.sweeps = sw;
                    p.vec = 16 / esize;
                    p.tile = r * re;
                    p.tiles_per_seg = tps;
                    p.num_tiles = outer * tps;
                    p.rts_blocks = p.rts_chunk = 0;
                    p.ws_bytes = kHeader + round_up(size_t(p.num_tiles) * p.carry_words * 8, 256);
                    p.launches = 1;
                    return SCAN_OK;
                }
            }
        }
    }
    // Many rows that each fit one tile of the rows kernel (256 threads x 1,
    // 2, 4 or 8 rows of 128-bit vectors, the fewest that hold a row; rows of
    // at least one wave's vectors): one workgroup per row and no look-back.
    // Identity scans of the default shape without a grid cap; two rows or
    // more, so that count-scan-emit's single array keeps its total.
    if (shape_free && tu.grid_blocks <= 0 && !tu.no_identity && vec_ok && outer >= 2 &&
        len >= int64_t(kWave) * (16 / esize)) {
        for (int r : {1, 2, 4, 8}) {
            const int64_t t = int64_t(kRowsBlock) * r * (16 / esize);
            if (len <= t && find_rows(dt, op, r) != nullptr) {
                p.kernel = SCAN_KERNEL_ROWS;
                p.block = kRowsBlock;
                p.rows = r;
                p.vec = 16 / esize;
                p.tile = t;
                p.tiles_per_seg = 1;
                p.num_tiles = outer;
                p.carry_words = 0;
                p.rts_blocks = p.rts_chunk = 0;
                p.ws_bytes = 0;  // no workspace
                p.launches = 1;
                return SCAN_OK;
            }
        }
    }
    if (rts) {
        p.kernel = SCAN_KERNEL_RTS;
        int64_t c = tu.rts_blocks > 0 ? tu.rts_blocks : kDefaultRtsBlocks;
        if (c > p.num_tiles) c = p.num_tiles;
        p.rts_chunk = (p.num_tiles + c - 1) / c;
        p.rts_blocks = (p.num_tiles + p.rts_chunk - 1) / p.rts_chunk;
        p.ws_bytes = kHeader + round_up(size_t(p.rts_blocks) * carry_bytes(dt, op), 256);
        p.launches = 3;
    } else {
        p.kernel = SCAN_KERNEL_LOOKBACK;
        p.rts_blocks = p.rts_chunk = 0;
        p.ws_bytes = kHeader + round_up(size_t(p.num_tiles) * p.carry_words * 8, 256);
        p.launches = 1;
    }
    return SCAN_OK;
}

// Large elements (inner > 1): `block` threads per workgroup from the PR's
// rule, each owning E elements of a tile: E = elem_e_max(inner) when that
// tile still fits (2 * block * E * esize bytes within the caller's budget,
// else within kElemTileLocalMem), else 1.  The rule's own budget only sizes
// the block: E is this kernel's blocking, not the PR's, and narrow elements
// (1e6 x 8 fp32: 256 threads x 4) lose a third of their rate at E = 1.
// Chunks of tiles give about kElemChunks workgroups per launch.
int plan_element(scan_dtype_t dt, scan_op_t op, int64_t outer, int64_t len, int64_t inner, bool aligned,
                 const scan_tuning_t &tu, TilePlan &p) {
    if (tu.algo == SCAN_ALGO_REDUCE_THEN_SCAN) return SCAN_ERR_UNSUPPORTED;
    if (inner > 64) return SCAN_ERR_UNSUPPORTED;
    const int esize = dtype_bytes(dt);
    const int64_t budget = tu.local_mem_bytes > 0 ? tu.local_mem_bytes : kDefaultLocalMem;
    const int64_t b = element_block(inner * esize, budget, tu.block_size, kElemDefaultBlock);
    if (b < 64 || b > 512 || b % 64 != 0) return SCAN_ERR_UNSUPPORTED;
    const bool vec = aligned && (inner * esize) % 16 == 0;
    int e = elem_e_max(int(inner));
    const int64_t e_budget = tu.local_mem_bytes > 0 ? tu.local_mem_bytes : kElemTileLocalMem;
    if (e > 1 && 2 * b * e * inner * esize > e_budget) e = 1;
    if (!find_element(dt, op, int(inner), e, vec)) return SCAN_ERR_UNSUPPORTED;
    p.kernel = SCAN_KERNEL_ELEMENT;
    p.block = int(b);
    p.rows = e;
    p.vec = vec ? 16 / esize : 1;
    p.width = int(inner);
    p.tile = b * e;
    p.tiles_per_seg = (len + p.tile - 1) / p.tile;
    p.num_tiles = outer * p.tiles_per_seg;
    if (p.num_tiles > int64_t(INT32_MAX)) return SCAN_ERR_OVERFLOW;
    const int64_t want = tu.rts_blocks > 0 ? (tu.rts_blocks < 8192 ? tu.rts_blocks : 8192) : kElemChunks;
    int64_t chunks = (want + outer - 1) / outer;
    if (chunks > p.tiles_per_seg) chunks = p.tiles_per_seg;
    if (chunks < 1) chunks = 1;
    p.rts_chunk = (p.tiles_per_seg + chunks - 1) / chunks;      // tiles per chunk
    p.rts_blocks = (p.tiles_per_seg + p.rts_chunk - 1) / p.rts_chunk;  // chunks per segment
    if (outer * p.rts_blocks > int64_t(INT32_MAX) || outer * inner > int64_t(INT32_MAX)) return SCAN_ERR_OVERFLOW;
    p.carry_words = int(inner) * carry_bytes(dt, op) / 4;
    p.ws_bytes = kHeader + round_up(size_t(outer * p.rts_blocks * inner) * carry_bytes(dt, op), 256);
    p.launches = 3;
    return SCAN_OK;
}

// Wide inner extents.  In one pass (k_col_single) when the rows allow
// 128-bit accesses, the strips are at least half full, the array makes at
// most kColSingleMaxTiles register tiles (one per compute unit) of at most
// kColSingleMaxRowBlocks per strip, and reduce-then-scan is not asked for.
// Otherwise reduce-then-scan over row chunks: about 512 workgroups over
// (outer, chunk, strip), at least 16 rows per chunk (so the partials stay
// within 0.5 byte per value) and at most 256 chunks (the partials kernel's
// LDS block).
int plan_columns(scan_dtype_t dt, scan_op_t op, int64_t outer, int64_t len, int64_t inner, bool aligned,
                 const scan_tuning_t &tu, TilePlan &p) {
    const int esize = dtype_bytes(dt);
    const int vmax = 16 / esize;
    const int64_t tc = int64_t(kWave) * vmax;  // columns per strip of the single pass
    if (tu.algo != SCAN_ALGO_REDUCE_THEN_SCAN && aligned && inner % vmax == 0 && 2 * inner >= tc &&
        find_columns_single(dt, op) != nullptr) {
        const int64_t strips = (inner + tc - 1) / tc, rblocks = (len + kColTileRows - 1) / kColTileRows;
        if (outer * strips * rblocks <= kColSingleMaxTiles && rblocks <= kColSingleMaxRowBlocks) {
            p.kernel = SCAN_KERNEL_COLUMNS_LOOKBACK;
            p.block = kColTileWaves * kWave;
            p.rows = kColTileRowsPerThread;
            p.vec = vmax;
            p.width = 1;
            p.col_strips = strips;
            p.col_chunks = rblocks;
            p.col_rows = kColTileRows;
            p.num_tiles = outer * strips * rblocks;
            p.tiles_per_seg = rblocks;
            p.tile = kColTileRows * tc;
            p.carry_words = desc_words(dt, op);  // per column
            p.rts_blocks = p.rts_chunk = 0;
            p.ws_bytes = kHeader + round_up(size_t(p.num_tiles * tc) * p.carry_words * 8, 256);
            p.launches = 1;
            return SCAN_OK;
        }
    }
    p.kernel = SCAN_KERNEL_COLUMNS;
    p.vec = (aligned && inner % vmax == 0) ? vmax : 1;
    if (!find_columns(dt, op, p.vec)) return SCAN_ERR_UNSUPPORTED;
    p.block = 256;
    p.rows = 1;
    p.width = 1;
    p.col_strips = (inner + 256 * p.vec - 1) / (256 * p.vec);
    // about 512 workgroups, chunks of at least 16 rows, at most 256 chunks
    // (the partials kernel's LDS block)
    int64_t chunks = (512 + p.col_strips * outer - 1) / (p.col_strips * outer);
    int64_t rows = (len + chunks - 1) / chunks;
    if (rows < 16) rows = 16;
    if (rows * 256 < len) rows = (len + 255) / 256;
    p.col_rows = rows;
    p.col_chunks = (len + rows - 1) / rows;
    const int64_t wgs = outer * p.col_chunks * p.col_strips;
    if (wgs > int64_t(INT32_MAX) || outer > int64_t(UINT32_MAX)) return SCAN_ERR_OVERFLOW;
    p.tile = rows * inner;
    p.tiles_per_seg = p.col_chunks;
    p.num_tiles = wgs;
    p.carry_words = carry_bytes(dt, op) / 4;
    p.rts_blocks = p.rts_chunk = 0;
    p.ws_bytes = kHeader + round_up(size_t(outer * p.col_chunks * inner) * carry_bytes(dt, op), 256);
    p.launches = 3;
    return SCAN_OK;
}

int plan_compact(scan_dtype_t dt, int64_t n, bool aligned, const scan_tuning_t &tu, TilePlan &p) {
    // Arrays that fit one register tile per compute unit: the resident pass
    // (the fewest rows that keep the tiles within kResMaxTiles), for the
    // default shape without a grid cap.  It was faster than the pipeline at
    // every size measured (back-to-back calls: 4096 keys 5.0 against 6.0 us,
    // 2^20 8.1 against 10.7, 1e7 15.7 against 23.1).
    const bool shape_free = tu.block_size <= 0 && tu.items_per_thread <= 0;
    if (shape_free && tu.grid_blocks <= 0 && aligned && n % 4 == 0 &&
        find_compact_resident(dt, SCAN_CMP_GT) != nullptr) {
        const int64_t re = int64_t(kResWaves - 1) * kWave * 4;
        for (int r = 1; r <= kResCompactMaxRows; r++) {
            const int64_t tiles = (n + r * re - 1) / (r * re);
            if (tiles <= kResMaxTiles) {
                p.kernel = SCAN_KERNEL_COMPACT_RESIDENT;
                p.block = kResWaves * kWave;
                p.rows = r;
                p.vec = 4;
                p.tile = r * re;
                p.tiles_per_seg = p.num_tiles = tiles;
                p.carry_words = 1;
                p.rts_blocks = p.rts_chunk = 0;
                p.ws_bytes = kHeader + round_up(size_t(p.num_tiles) * 8, 256);
                p.launches = 1;
                return SCAN_OK;
            }
        }
    }
    // 128-bit loads need 16-byte aligned x and whole vectors up to n
    const int rc = plan_shape(
        4, aligned && n % 4 == 0, tu, p,
        [&](int b, int r, int v) { return find_compact(dt, SCAN_CMP_GT, b, r, v) != nullptr; }, true, 5, 768);
    if (rc != SCAN_OK) return rc;
    p.kernel = SCAN_KERNEL_COMPACT;
    p.tiles_per_seg = p.num_tiles = (n + p.tile - 1) / p.tile;
    p.carry_words = 1;
    p.rts_blocks = p.rts_chunk = 0;
    p.ws_bytes = kHeader + round_up(size_t(p.num_tiles) * 8, 256);
    p.launches = 1;
    return SCAN_OK;
}

// A bit predicate takes an integer key and a bit index 0..31.
bool threshold_ok(scan_dtype_t dt, scan_cmp_t cmp, double t) {
    if (!bit_cmp(cmp)) return true;
    return dt != SCAN_F32 && t >= 0.0 && t <= 31.0 && t == double(int(t));
}

// The threshold converted once to x's type (its bit pattern): fp32 rounded,
// integers clamped to the type's range then truncated; the bit index for
// the bit predicates.
uint32_t threshold_bits(scan_dtype_t dt, scan_cmp_t cmp, double threshold) {
    uint32_t bits = 0;
    if (bit_cmp(cmp)) {
        bits = uint32_t(threshold);
    } else if (dt == SCAN_F32) {
        const float t = float(threshold);
        memcpy(&bits, &t, 4);
    } else if (dt == SCAN_I32) {
        const double c = threshold < double(INT32_MIN) ? double(INT32_MIN)
                         : threshold > double(INT32_MAX) ? double(INT32_MAX) : threshold;
        const int32_t t = int32_t(c);
        memcpy(&bits, &t, 4);
    } else {
        const double c = threshold < 0.0 ? 0.0 : threshold > double(UINT32_MAX) ? double(UINT32_MAX) : threshold;
        bits = uint32_t(c);
    }
    return bits;
}

// Ragged segmented scan.  Default: reduce-then-scan with small tiles (256
// threads x 2 rows of 128-bit vectors) in about kSegChunks chunks (at most
// 8192, the partials pass), whose per-tile chain of loads, head marking and
// barriers is hidden by many resident workgroups (1.9x faster than 512 x
// 8-row tiles in 1024 chunks).  Workspace: the tile map (one word per
// tile), the head planes (a quarter byte per element), then the chunk
// partials (16 bytes each).  algo = look-back: the single pass on the
// look-back pipeline (512 threads, 448 of them data, x 4 rows), after a map
// pass and a heads pass; the (flag, value) descriptors come first in the
// workspace, then the map and the planes.  Every map and plane word stays
// below 2^32, so a look-back reads it as unpublished.  The single pass
// measured slower on 3e7 elements (see segmented.hip).
constexpr int kSegBlock = 256, kSegRows = 2, kSegPipeRows = 4;
constexpr int64_t kSegChunks = 4096;

int plan_segmented(scan_dtype_t dt, scan_op_t op, int64_t n, bool aligned, const scan_tuning_t &tu, TilePlan &p) {
    const int esize = dtype_bytes(dt);
    const bool vec_ok = aligned;  // the last tile is accessed element-wise, so any n
    const bool rts = tu.algo != SCAN_ALGO_LOOKBACK;
    const int rc =
        rts ? plan_shape(
                  esize, vec_ok, tu, p, [&](int b, int r, int v) { return find_seg(dt, op, b, r, v) != nullptr; },
                  false, kSegRows, kSegBlock)
            : plan_shape(
                  esize, vec_ok, tu, p,
                  [&](int b, int r, int v) { return find_seg_pipe(dt, op, b, r, v) != nullptr; }, true,
                  kSegPipeRows, kDefaultBlock);
    if (rc != SCAN_OK) return rc;
    p.kernel = SCAN_KERNEL_SEGMENTED;
    p.tiles_per_seg = p.num_tiles = (n + p.tile - 1) / p.tile;
    if (p.num_tiles > int64_t(INT32_MAX)) return SCAN_ERR_OVERFLOW;
    int64_t chunks = tu.rts_blocks > 0 ? tu.rts_blocks : kSegChunks;
    if (chunks > 8192) chunks = 8192;
    if (chunks > p.num_tiles) chunks = p.num_tiles;
    p.rts_chunk = (p.num_tiles + chunks - 1) / chunks;
    p.rts_blocks = (p.num_tiles + p.rts_chunk - 1) / p.rts_chunk;
    const size_t maps = round_up(size_t(p.num_tiles) * 8, 16) + round_up(size_t(p.num_tiles) * (p.tile / 4), 16);
    if (rts) {
        p.carry_words = carry_bytes(dt, op) / 4;
        p.ws_bytes = kHeader + maps + round_up(size_t(p.rts_blocks) * 16, 256);
        p.launches = 4;
    } else {
        p.carry_words = carry_bytes(dt, op) / 4;  // (flag, value) descriptors: the value's chunks
        p.ws_bytes = kHeader + round_up(size_t(p.num_tiles) * p.carry_words * 8, 256) + round_up(maps, 256);
        p.launches = 3;
    }
    return SCAN_OK;
}

// Stable partition: the compaction's tiles, plus a count pass of at most
// 1024 workgroups whose counts follow the tile descriptors.
int plan_partition(scan_dtype_t dt, scan_cmp_t cmp, int64_t n, bool aligned, const scan_tuning_t &tu, TilePlan &p,
                   int64_t &count_wgs, int64_t &count_chunk) {
    // Arrays that fit one register tile per compute unit: the resident pass,
    // one launch, x read once (the tiles read every tile's count instead of
    // a count pass); the default shape without a grid cap.
    const bool shape_free = tu.block_size <= 0 && tu.items_per_thread <= 0;
    if (shape_free && tu.grid_blocks <= 0 && aligned && n % 4 == 0 && find_partition_resident(dt, cmp) != nullptr) {
        const int64_t re = int64_t(kResWaves - 1) * kWave * 4;
        for (int r = 1; r <= kResCompactMaxRows; r++) {
            const int64_t tiles = (n + r * re - 1) / (r * re);
            if (tiles <= kResMaxTiles) {
                p.kernel = SCAN_KERNEL_PARTITION_RESIDENT;
                p.block = kResWaves * kWave;
                p.rows = r;
                p.vec = 4;
                p.tile = r * re;
                p.tiles_per_seg = p.num_tiles = tiles;
                p.carry_words = 1;
                p.rts_blocks = p.rts_chunk = 0;
                p.ws_bytes = kHeader + round_up(size_t(p.num_tiles) * 8, 256);
                p.launches = 1;
                count_wgs = count_chunk = 0;
                return SCAN_OK;
            }
        }
    }
    const int rc = plan_shape(
        4, aligned && n % 4 == 0, tu, p,
        [&](int b, int r, int v) { return find_partition(dt, cmp, b, r, v) != nullptr; }, true, 3, 768);
    if (rc != SCAN_OK) return rc;
    p.kernel = SCAN_KERNEL_PARTITION;
    p.tiles_per_seg = p.num_tiles = (n + p.tile - 1) / p.tile;
    p.carry_words = 1;
    p.rts_blocks = p.rts_chunk = 0;
    // about 16 Ki elements per count workgroup, at most 1024 of them, chunks
    // on vector boundaries
    count_wgs = (n + 16383) / 16384;
    if (count_wgs > 1024) count_wgs = 1024;
    count_chunk = round_up(size_t((n + count_wgs - 1) / count_wgs), size_t(p.vec));
    count_wgs = (n + count_chunk - 1) / count_chunk;
    p.ws_bytes = kHeader + round_up(size_t(p.num_tiles + count_wgs) * 8, 256);
    p.launches = 2;
    return SCAN_OK;
}

bool aligned16(const void *a, const void *b) {
    return ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) & 15u) == 0;
}

int check_ws(const void *ws, size_t ws_bytes, size_t need) {
    if (ws == nullptr || ws_bytes < need) return SCAN_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(ws) & 255u) return SCAN_ERR_WORKSPACE;  // 256-byte aligned
    return SCAN_OK;
}

PipeArgs pipe_args(const TilePlan &p, void *ws, size_t ws_bytes, const scan_tuning_t &tu) {
    PipeArgs a;
    a.ws = ws;
    a.ws_words = (ws_bytes - kHeader) / 8;
    a.words_used = p.tiles_per_seg > 1 ? uint64_t(p.num_tiles) * p.carry_words : 0;
    a.num_tiles = uint32_t(p.num_tiles);
    a.tiles_per_seg = uint32_t(p.tiles_per_seg);
    a.spin_limit = tu.spin_limit > 0 ? uint32_t(tu.spin_limit) : kDefaultSpinLimit;
    a.mode_limit = tu.mode_limit > 0 ? uint32_t(tu.mode_limit) : kDefaultModeLimit;
    a.delay_stride = tu.delay_stride > 0 ? uint32_t(tu.delay_stride) : 0u;
    a.delay_sleeps = tu.delay_sleeps > 0 ? uint32_t(tu.delay_sleeps) : 0u;
    return a;
}

int scan_common(const void *in, void *out, int64_t outer, int64_t len, int64_t inner, scan_dtype_t dt,
                scan_op_t op, int exclusive, void *total_out, void *ws, size_t ws_bytes,
                const scan_tuning_t *tuning, hipStream_t stream) {
    if (!valid_dtype(dt) || !valid_op(op)) return SCAN_ERR_INVALID_ARG;
    if (outer < 0 || len < 0 || inner < 1) return SCAN_ERR_INVALID_ARG;
    if (outer == 0 || len == 0) return SCAN_OK;
    if (in == nullptr || out == nullptr) return SCAN_ERR_INVALID_ARG;
    const scan_tuning_t tu = tuning_or_default(tuning);
    if (tu.algo < SCAN_ALGO_AUTO || tu.algo > SCAN_ALGO_REDUCE_THEN_SCAN) return SCAN_ERR_INVALID_ARG;
    // without an identity: inclusive look-back scans of scalar elements only
    if (tu.no_identity && (exclusive || inner != 1 || total_out != nullptr)) return SCAN_ERR_UNSUPPORTED;
    if (inner != 1) {
        if (total_out != nullptr) return SCAN_ERR_UNSUPPORTED;
        TilePlan p;
        int rc = plan_element(dt, op, outer, len, inner, aligned16(in, out), tu, p);
        if (rc == SCAN_ERR_UNSUPPORTED) {
            rc = plan_columns(dt, op, outer, len, inner, aligned16(in, out), tu, p);
            if (rc != SCAN_OK) return rc;
            rc = check_ws(ws, ws_bytes, p.ws_bytes);
            if (rc != SCAN_OK) return rc;
            if (p.kernel == SCAN_KERNEL_COLUMNS_LOOKBACK) {
                ColSingleArgs c{};
                c.pipe = pipe_args(p, ws, ws_bytes, tu);
                c.pipe.words_used = uint64_t(p.num_tiles) * (int64_t(kWave) * p.vec) * p.carry_words;
                c.in = in;
                c.out = out;
                c.outer = uint32_t(outer);
                c.len = len;
                c.inner = inner;
                c.strips = uint32_t(p.col_strips);
                c.rblocks = uint32_t(p.col_chunks);
                c.exclusive = exclusive ? 1 : 0;
                return find_columns_single(dt, op)(c, stream);
            }
            ColArgs c{};
            c.in = in;
            c.out = out;
            c.outer = uint32_t(outer);
            c.len = len;
            c.inner = inner;
            c.rows = p.col_rows;
            c.chunks = uint32_t(p.col_chunks);
            c.strips = uint32_t(p.col_strips);
            c.exclusive = exclusive ? 1 : 0;
            c.partials = reinterpret_cast<char *>(ws) + kHeader;
            return find_columns(dt, op, p.vec)(c, stream);
        }
        if (rc != SCAN_OK) return rc;
        rc = check_ws(ws, ws_bytes, p.ws_bytes);
        if (rc != SCAN_OK) return rc;
        ElemArgs a{};
        a.in = in;
        a.out = out;
        a.outer = uint32_t(outer);
        a.len = len;
        a.chunks = uint32_t(p.rts_blocks);
        a.tiles_per_chunk = uint32_t(p.rts_chunk);
        a.exclusive = exclusive ? 1 : 0;
        a.partials = reinterpret_cast<char *>(ws) + kHeader;
        return find_element(dt, op, p.width, p.rows, p.vec > 1)(a, p.block, stream);
    }

    TilePlan p;
    int rc = plan_scan(dt, op, outer, len, aligned16(in, out), tu, p);
    if (rc != SCAN_OK) return rc;
    if (p.kernel == SCAN_KERNEL_ROWS) {  // no workspace
        if (total_out != nullptr) return SCAN_ERR_UNSUPPORTED;
        RowsArgs r{};
        r.in = in;
        r.out = out;
        r.len = len;
        r.rows = uint64_t(outer);
        r.exclusive = exclusive ? 1 : 0;
        return find_rows(dt, op, p.rows)(r, stream);
    }
    rc = check_ws(ws, ws_bytes, p.ws_bytes);
    if (rc != SCAN_OK) return rc;
    if (p.kernel == SCAN_KERNEL_RTS) {
        if (total_out != nullptr) return SCAN_ERR_UNSUPPORTED;
        RtsArgs r{};
        r.in = in;
        r.out = out;
        r.n = len;
        r.num_tiles = uint32_t(p.num_tiles);
        r.chunk_tiles = uint32_t(p.rts_chunk);
        r.blocks = uint32_t(p.rts_blocks);
        r.exclusive = exclusive ? 1 : 0;
        // larger than the 256 MB Infinity Cache can keep between the passes
        r.reverse = len * dtype_bytes(dt) > (int64_t(192) << 20) ? 1 : 0;
        r.partials = reinterpret_cast<char *>(ws) + kHeader;
        return find_rts(dt, op, p.block, p.rows, p.vec)(r, stream);
    }
    ScanArgs a{};
    a.pipe = pipe_args(p, ws, ws_bytes, tu);
    a.in = in;
    a.out = out;
    a.seg_len = len;
    a.exclusive = exclusive ? 1 : 0;
    a.total_out = total_out;
    if (p.kernel == SCAN_KERNEL_RESIDENT) {
        if (total_out != nullptr && dt == SCAN_I32 && op == SCAN_OP_SUM)  // count-scan-emit's offsets
            return find_pack_resident()(a, p.rows, p.sweeps, stream);
        return (tu.no_identity ? find_resident_noid(dt, op) : find_resident(dt, op))(a, p.rows, p.sweeps, stream);
    }
    const uint32_t grid_cap = tu.grid_blocks > 0 ? uint32_t(tu.grid_blocks) : 0u;
    if (total_out != nullptr && dt == SCAN_I32 && op == SCAN_OP_SUM)  // count-scan-emit's offsets
        return find_pack_lookback(p.block, p.rows, p.vec)(a, grid_cap, stream);
    if (tu.no_identity) return find_noid(dt, op, p.block, p.rows, p.vec)(a, grid_cap, stream);
    return find_lookback(dt, op, p.block, p.rows, p.vec)(a, grid_cap, stream);
}

// LDS of the element kernels (ElemTile::lds_bytes_rescan in element.hip):
// the tile in the owner layout, each thread's slots padded to an odd number
// of accesses, then one slot per wave (up to 8) and component, then the
// rescan's W running carries.
int64_t element_lds_bytes(scan_dtype_t dt, scan_op_t op, const TilePlan &p) {
    const int64_t s = dtype_bytes(dt), lv = p.vec;  // values per access
    const int64_t vpt = int64_t(p.rows) * p.width, upt = vpt / lv;
    const int64_t stride = vpt + (upt % 2 == 0 ? lv : 0);
    return int64_t(p.block) * stride * s + (8 + 1) * int64_t(p.width) * carry_bytes(dt, op);
}

void fill_plan(const TilePlan &p, scan_dtype_t dt, scan_op_t op, scan_plan_t *plan) {
    plan->kernel = p.kernel;
    plan->block_size = p.block;
    plan->items_per_thread = p.kernel == SCAN_KERNEL_ELEMENT ? p.rows : p.rows * p.vec;
    plan->vec = p.vec;
    plan->tile_elems = p.tile;  // elements (of `width` components for the element kernel)
    plan->num_tiles = p.kernel == SCAN_KERNEL_RTS ? p.rts_blocks : p.num_tiles;
    if (p.kernel == SCAN_KERNEL_ELEMENT) plan->num_tiles = p.num_tiles / p.tiles_per_seg * p.rts_blocks;
    if (p.kernel == SCAN_KERNEL_ELEMENT)
        plan->lds_bytes = element_lds_bytes(dt, op, p);
    else if (p.kernel == SCAN_KERNEL_COLUMNS_LOOKBACK)
        plan->lds_bytes = int64_t(kColTileWaves + 1) * kWave * p.vec * carry_bytes(dt, op) + 32;
    else if (p.kernel == SCAN_KERNEL_PARTITION_RESIDENT)
        plan->lds_bytes = int64_t(kResPartChunkRows) * (kResWaves - 1) * kWave * 4 * 6 +
                          int64_t(kResCompactMaxRows) * (kResWaves - 1) * 4 + 32;
    else if (p.kernel == SCAN_KERNEL_COMPACT_RESIDENT)
        plan->lds_bytes = int64_t(kResCompactMaxRows) * (kResWaves - 1) * kWave * 4 * 2 +
                          int64_t(kResCompactMaxRows) * (kResWaves - 1) * 4 + 32;
    else if (p.kernel == SCAN_KERNEL_RESIDENT) {
        const bool wide = dt == SCAN_I64 || dt == SCAN_F64;
        const int maxr = p.sweeps == 2 ? 2 * (wide ? kResMaxRows2x8 : kResMaxRows2x4) : (wide ? kResMaxRows8 : kResMaxRows4);
        plan->lds_bytes = int64_t(dtype_bytes(dt)) * (kResWaves - 1) * maxr + p.sweeps * carry_bytes(dt, op) + 32;
    }
    else
        plan->lds_bytes = int64_t(p.rows) * (p.block / 64) * dtype_bytes(dt) + carry_bytes(dt, op) + 32;
    plan->workspace_bytes = int64_t(p.ws_bytes);
    plan->launches = p.launches;
    plan->carry_words = p.carry_words;
    plan->tiles_per_block = p.kernel == SCAN_KERNEL_RESIDENT ? p.sweeps : 0;
}

}  // namespace
}  // namespace sw64

namespace sw64 {

// ------------------------------------------------- the no-allocation entry point
// The workspace of scan_inclusive_noalloc: a device array of the library's own,
// one copy per GPU (each device holds its own, at its own address, from the
// first call until the process ends).  Host code never passes `scratch`
// itself to a kernel or a copy -- on the host that name is only a stand-in --
// but the device address hipGetSymbolAddress returns for the current device.
constexpr size_t kStaticScratchBytes = SCAN_NOALLOC_SCRATCH_BYTES;
static_assert(kStaticScratchBytes % 256 == 0 && kStaticScratchBytes > kWsHeaderBytes, "scratch size");
static __device__ __align__(256) uint64_t scratch[kStaticScratchBytes / 8];

constexpr int kMaxDevices = 64;

// The current device's scratch address.  On a device's first call: look the
// address up (with that device current) and zero the array with a fill
// kernel on `stream`, recording its capacity in the workspace header the way
// scan_workspace_init does, so the call that follows on the same stream finds
// a fresh workspace.  A fill kernel, not a memset node: the first call may be
// under graph capture.
int noalloc_scratch(hipStream_t stream, void **out) {
    static std::mutex mu;
    static void *ptr[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SCAN_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return SCAN_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(mu);
    if (ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SCAN_ERR_HIP;
        if (reinterpret_cast<uintptr_t>(p) & 255u) return SCAN_ERR_HIP;
        const uint64_t cap = (kStaticScratchBytes - kWsHeaderBytes) / 8;
        const int rc = launch_fill_u64(p, kStaticScratchBytes / 8, 0, stream, offsetof(WsHeader, capacity) / 8, cap);
        if (rc != SCAN_OK) return rc;
        ptr[dev] = p;
    }
    *out = ptr[dev];
    return SCAN_OK;
}

}  // namespace sw64

using namespace sw64;

extern "C" {

int scan_plan(scan_call_t call, scan_dtype_t dtype, scan_op_t op, int64_t outer, int64_t len, int64_t inner,
              const scan_tuning_t *tuning, scan_plan_t *plan) {
    if (plan == nullptr) return SCAN_ERR_INVALID_ARG;
    memset(plan, 0, sizeof(*plan));
    if (!valid_dtype(dtype) || !valid_op(op)) return SCAN_ERR_INVALID_ARG;
    if (outer < 0 || len < 0 || inner < 1) return SCAN_ERR_INVALID_ARG;
    const scan_tuning_t tu = tuning_or_default(tuning);
    if (tu.no_identity && (call != SCAN_CALL_SCAN || inner != 1)) return SCAN_ERR_UNSUPPORTED;
    TilePlan p;
    int rc;
    switch (call) {
    case SCAN_CALL_SCAN:
        if (outer == 0 || len == 0) return SCAN_OK;
        if (inner == 1) {
            rc = plan_scan(dtype, op, outer, len, true, tu, p);
        } else {
            rc = plan_element(dtype, op, outer, len, inner, true, tu, p);
            if (rc == SCAN_ERR_UNSUPPORTED) rc = plan_columns(dtype, op, outer, len, inner, true, tu, p);
        }
        break;
    case SCAN_CALL_COMPACT:
        if (dtype != SCAN_F32 && dtype != SCAN_I32 && dtype != SCAN_U32) return SCAN_ERR_UNSUPPORTED;
        if (outer * len * inner > int64_t(INT32_MAX)) return SCAN_ERR_OVERFLOW;
        if (outer * len * inner == 0) return SCAN_OK;
        rc = plan_compact(dtype, outer * len * inner, true, tu, p);
        break;
    case SCAN_CALL_SEGMENTED:
        // outer = number of segments, len = elements
        if (inner != 1) return SCAN_ERR_INVALID_ARG;
        if (len > int64_t(INT32_MAX) || outer > int64_t(INT32_MAX)) return SCAN_ERR_OVERFLOW;
        if (len == 0) return SCAN_OK;
        rc = plan_segmented(dtype, op, len, true, tu, p);
        break;
    case SCAN_CALL_PARTITION: {
        // the predicate does not change the plan; GT stands for any
        if (dtype != SCAN_F32 && dtype != SCAN_I32 && dtype != SCAN_U32) return SCAN_ERR_UNSUPPORTED;
        if (outer * len * inner > int64_t(INT32_MAX)) return SCAN_ERR_OVERFLOW;
        if (outer * len * inner == 0) return SCAN_OK;
        int64_t cw = 0, cc = 0;
        rc = plan_partition(dtype, SCAN_CMP_GT, outer * len * inner, true, tu, p, cw, cc);
        break;
    }
    case SCAN_CALL_PACK: {
        if (dtype != SCAN_I32 || outer != 1 || inner != 1) return SCAN_ERR_INVALID_ARG;
        if (len > int64_t(INT32_MAX)) return SCAN_ERR_OVERFLOW;
        if (len == 0) return SCAN_OK;
        scan_tuning_t lb = tu;
        lb.algo = SCAN_ALGO_LOOKBACK;
        rc = plan_scan(SCAN_I32, SCAN_OP_SUM, 1, len, true, lb, p);
        if (rc == SCAN_OK) p.kernel = SCAN_KERNEL_PACK;
        break;
    }
    default:
        return SCAN_ERR_INVALID_ARG;
    }
    if (rc != SCAN_OK) return rc;
    fill_plan(p, dtype, op, plan);
    return SCAN_OK;
}

size_t scan_workspace_bytes(scan_dtype_t dtype, int64_t count) {
    (void)dtype;
    if (count < 0) count = 0;
    // <= 0.5 byte of descriptors or partials per value for any kernel and
    // tuning (smallest tiles: 16 values per 8-byte word), plus the header and
    // room for reduce-then-scan partials.
    return kHeader + round_up(size_t(count + 15) / 16 * 8, 256) + 65536;
}

int scan_workspace_init(void *ws, size_t ws_bytes, void *stream) {
    if (ws_bytes == 0) return SCAN_OK;
    if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & 7u)) return SCAN_ERR_INVALID_ARG;
    // zero everything; the header's capacity word records the descriptor
    // words of this buffer, so that a later call passing a smaller size still
    // clears what a larger one left tagged (end_call in device.hpp)
    const uint64_t cap = ws_bytes > kHeader ? uint64_t(ws_bytes - kHeader) / 8 : 0;
    return launch_fill_u64(ws, ws_bytes / 8, 0, reinterpret_cast<hipStream_t>(stream),
                           offsetof(WsHeader, capacity) / 8, cap);
}

int scan_workspace_error(const void *ws, int32_t *error, void *stream) {
    if (ws == nullptr || error == nullptr) return SCAN_ERR_INVALID_ARG;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // the error word follows the epoch
    const char *p = reinterpret_cast<const char *>(ws) + 4;
    if (hipMemcpyAsync(error, p, sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess) return SCAN_ERR_HIP;
    return hipStreamSynchronize(s) == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
}

int scan_inclusive(const void *in, void *out, int64_t n, scan_dtype_t dtype, scan_op_t op, int32_t width,
                   void *ws, size_t ws_bytes, const scan_tuning_t *tuning, void *stream) {
    if (width < 1 || n < 0) return SCAN_ERR_INVALID_ARG;
    return scan_common(in, out, 1, n, width, dtype, op, 0, nullptr, ws, ws_bytes, tuning,
                       reinterpret_cast<hipStream_t>(stream));
}

int scan_inclusive_noalloc(const void *in, void *out, int64_t n, scan_dtype_t dtype, scan_op_t op, int32_t width,
                           const scan_tuning_t *tuning, void *stream) {
    if (width < 1 || n < 0 || !valid_dtype(dtype) || !valid_op(op)) return SCAN_ERR_INVALID_ARG;
    if (n == 0) return SCAN_OK;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // the plan's workspace must fit the array; larger calls are rejected
    // before anything is enqueued
    scan_plan_t p;
    const int prc = scan_plan(SCAN_CALL_SCAN, dtype, op, 1, n, width, tuning, &p);
    if (prc != SCAN_OK) return prc;
    if (size_t(p.workspace_bytes) > kStaticScratchBytes) return SCAN_ERR_WORKSPACE;
    void *ws = nullptr;
    const int rc = noalloc_scratch(s, &ws);
    if (rc != SCAN_OK) return rc;
    return scan_common(in, out, 1, n, width, dtype, op, 0, nullptr, ws, kStaticScratchBytes, tuning, s);
}

int scan_exclusive(const void *in, void *out, int64_t n, scan_dtype_t dtype, scan_op_t op, int32_t width,
                   void *ws, size_t ws_bytes, const scan_tuning_t *tuning, void *stream) {
    if (width < 1 || n < 0) return SCAN_ERR_INVALID_ARG;
    return scan_common(in, out, 1, n, width, dtype, op, 1, nullptr, ws, ws_bytes, tuning,
                       reinterpret_cast<hipStream_t>(stream));
}

int scan_dim(const void *in, void *out, int64_t outer, int64_t len, int64_t inner, scan_dtype_t dtype,
             scan_op_t op, int exclusive, void *ws, size_t ws_bytes, const scan_tuning_t *tuning, void *stream) {
    return scan_common(in, out, outer, len, inner, dtype, op, exclusive, nullptr, ws, ws_bytes, tuning,
                       reinterpret_cast<hipStream_t>(stream));
}

int compact_if(const void *x, int64_t n, scan_dtype_t x_dtype, scan_cmp_t cmp, double threshold, int32_t *out_idx,
               int32_t *d_count, void *ws, size_t ws_bytes, const scan_tuning_t *tuning, void *stream) {
    if (n < 0 || !valid_cmp(cmp) || d_count == nullptr) return SCAN_ERR_INVALID_ARG;
    if (!valid_dtype(x_dtype)) return SCAN_ERR_INVALID_ARG;
    if (x_dtype != SCAN_F32 && x_dtype != SCAN_I32 && x_dtype != SCAN_U32) return SCAN_ERR_UNSUPPORTED;
    if (!threshold_ok(x_dtype, cmp, threshold)) return SCAN_ERR_INVALID_ARG;
    if (n > int64_t(INT32_MAX)) return SCAN_ERR_OVERFLOW;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (n == 0) return launch_fill_i32(d_count, 1, 0, s);
    if (x == nullptr || out_idx == nullptr) return SCAN_ERR_INVALID_ARG;
    const scan_tuning_t tu = tuning_or_default(tuning);
    if (tu.no_identity) return SCAN_ERR_UNSUPPORTED;  // inclusive scans only
    TilePlan p;
    int rc = plan_compact(x_dtype, n, aligned16(x, x), tu, p);
    if (rc != SCAN_OK) return rc;
    rc = check_ws(ws, ws_bytes, p.ws_bytes);
    if (rc != SCAN_OK) return rc;
    CompactArgs a{};
    a.pipe = pipe_args(p, ws, ws_bytes, tu);
    a.x = x;
    a.n = n;
    a.threshold = threshold_bits(x_dtype, cmp, threshold);
    a.out_idx = out_idx;
    a.count = d_count;
    if (p.kernel == SCAN_KERNEL_COMPACT_RESIDENT) return find_compact_resident(x_dtype, cmp)(a, p.rows, s);
    const uint32_t grid_cap = tu.grid_blocks > 0 ? uint32_t(tu.grid_blocks) : 0u;
    return find_compact(x_dtype, cmp, p.block, p.rows, p.vec)(a, grid_cap, s);
}

int partition_if(const void *x, int64_t n, scan_dtype_t x_dtype, scan_cmp_t cmp, double threshold, void *out_vals,
                 int32_t *out_idx, int32_t *d_count, void *ws, size_t ws_bytes, const scan_tuning_t *tuning,
                 void *stream) {
    if (n < 0 || !valid_cmp(cmp) || d_count == nullptr) return SCAN_ERR_INVALID_ARG;
    if (!valid_dtype(x_dtype)) return SCAN_ERR_INVALID_ARG;
    if (x_dtype != SCAN_F32 && x_dtype != SCAN_I32 && x_dtype != SCAN_U32) return SCAN_ERR_UNSUPPORTED;
    if (!threshold_ok(x_dtype, cmp, threshold)) return SCAN_ERR_INVALID_ARG;
    if (n > int64_t(INT32_MAX)) return SCAN_ERR_OVERFLOW;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (n == 0) return launch_fill_i32(d_count, 1, 0, s);
    if (x == nullptr || out_vals == nullptr) return SCAN_ERR_INVALID_ARG;
    const scan_tuning_t tu = tuning_or_default(tuning);
    if (tu.no_identity) return SCAN_ERR_UNSUPPORTED;  // inclusive scans only
    TilePlan p;
    int64_t count_wgs = 0, count_chunk = 0;
    int rc = plan_partition(x_dtype, cmp, n, aligned16(x, x), tu, p, count_wgs, count_chunk);
    if (rc != SCAN_OK) return rc;
    rc = check_ws(ws, ws_bytes, p.ws_bytes);
    if (rc != SCAN_OK) return rc;
    PartitionArgs a{};
    a.pipe = pipe_args(p, ws, ws_bytes, tu);
    if (p.kernel == SCAN_KERNEL_PARTITION)
        a.pipe.words_used = uint64_t(p.num_tiles + count_wgs);  // tile descriptors, then the counts
    a.x = x;
    a.n = n;
    a.threshold = threshold_bits(x_dtype, cmp, threshold);
    a.out_vals = out_vals;
    a.out_idx = out_idx;
    a.count = d_count;
    a.count_base = uint32_t(p.num_tiles);
    a.count_wgs = uint32_t(count_wgs);
    a.count_chunk = count_chunk;
    if (p.kernel == SCAN_KERNEL_PARTITION_RESIDENT) return find_partition_resident(x_dtype, cmp)(a, p.rows, s);
    const uint32_t grid_cap = tu.grid_blocks > 0 ? uint32_t(tu.grid_blocks) : 0u;
    return find_partition(x_dtype, cmp, p.block, p.rows, p.vec)(a, grid_cap, s);
}

int scan_segmented(const void *in, void *out, int64_t n, const int32_t *offsets, int64_t nseg,
                   scan_dtype_t dtype, scan_op_t op, int exclusive, void *ws, size_t ws_bytes,
                   const scan_tuning_t *tuning, void *stream) {
    if (n < 0 || nseg < 0 || !valid_dtype(dtype) || !valid_op(op)) return SCAN_ERR_INVALID_ARG;
    if (n > int64_t(INT32_MAX) || nseg > int64_t(INT32_MAX)) return SCAN_ERR_OVERFLOW;
    if (n == 0) return SCAN_OK;
    if (nseg == 0 || in == nullptr || out == nullptr || offsets == nullptr) return SCAN_ERR_INVALID_ARG;
    const scan_tuning_t tu = tuning_or_default(tuning);
    if (tu.no_identity) return SCAN_ERR_UNSUPPORTED;  // inclusive scans only
    TilePlan p;
    int rc = plan_segmented(dtype, op, n, aligned16(in, out), tu, p);
    if (rc != SCAN_OK) return rc;
    rc = check_ws(ws, ws_bytes, p.ws_bytes);
    if (rc != SCAN_OK) return rc;
    SegArgs a{};
    a.in = in;
    a.out = out;
    a.n = n;
    a.off = offsets;
    a.nseg = nseg;
    a.tile = p.tile;
    a.tile_log2 = -1;
    for (int l = 0; l < 31; l++)
        if ((int64_t(1) << l) == p.tile) a.tile_log2 = l;
    a.num_tiles = uint32_t(p.num_tiles);
    a.chunk_tiles = uint32_t(p.rts_chunk);
    a.blocks = uint32_t(p.rts_blocks);
    a.exclusive = exclusive ? 1 : 0;
    a.grid_cap = tu.grid_blocks > 0 ? uint32_t(tu.grid_blocks) : 0u;
    char *w = reinterpret_cast<char *>(ws) + kHeader;
    const bool rts = tu.algo != SCAN_ALGO_LOOKBACK;
    if (!rts) {
        a.pipe = pipe_args(p, ws, ws_bytes, tu);  // descriptors right after the header
        w += round_up(size_t(p.num_tiles) * p.carry_words * 8, 256);
    }
    a.map = reinterpret_cast<uint64_t *>(w);
    w += round_up(size_t(p.num_tiles) * 8, 16);
    a.heads = reinterpret_cast<uint64_t *>(w);
    w += round_up(size_t(p.num_tiles) * (p.tile / 4), 16);
    a.partials = w;
    if (rts) return find_seg(dtype, op, p.block, p.rows, p.vec)(a, reinterpret_cast<hipStream_t>(stream));
    return find_seg_pipe(dtype, op, p.block, p.rows, p.vec)(a, reinterpret_cast<hipStream_t>(stream));
}

int pack_offsets(const int32_t *counts, int64_t n, int32_t *offsets, void *ws, size_t ws_bytes,
                 const scan_tuning_t *tuning, void *stream) {
    if (n < 0 || offsets == nullptr) return SCAN_ERR_INVALID_ARG;
    if (n > INT32_MAX) return SCAN_ERR_OVERFLOW;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (n == 0) return launch_fill_i32(offsets, 1, 0, s);
    if (counts == nullptr) return SCAN_ERR_INVALID_ARG;
    scan_tuning_t tu = tuning_or_default(tuning);
    if (tu.no_identity) return SCAN_ERR_UNSUPPORTED;  // offsets are an exclusive scan
    tu.algo = SCAN_ALGO_LOOKBACK;  // the total comes from the look-back's last tile
    return scan_common(counts, offsets, 1, n, 1, SCAN_I32, SCAN_OP_SUM, 1, offsets + n, ws, ws_bytes, &tu, s);
}

int pack_emit_neighbors(const int32_t *offsets, int64_t n, int32_t *out, void *stream) {
    if (n < 0) return SCAN_ERR_INVALID_ARG;
    if (n == 0) return SCAN_OK;
    if (offsets == nullptr || out == nullptr) return SCAN_ERR_INVALID_ARG;
    if (n > INT32_MAX) return SCAN_ERR_OVERFLOW;
    return launch_emit_neighbors(offsets, n, out, reinterpret_cast<hipStream_t>(stream));
}

int scan_copy(const void *in, void *out, size_t bytes, void *stream) {
    if (bytes == 0) return SCAN_OK;
    if (in == nullptr || out == nullptr || bytes % 16 != 0 || !aligned16(in, out)) return SCAN_ERR_INVALID_ARG;
    return launch_copy(in, out, bytes, reinterpret_cast<hipStream_t>(stream));
}

const char *scan_status_string(int status) {
    switch (status) {
    case SCAN_OK: return "ok";
    case SCAN_ERR_INVALID_ARG: return "invalid argument";
    case SCAN_ERR_UNSUPPORTED: return "unsupported dtype/op/shape/tuning combination";
    case SCAN_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case SCAN_ERR_HIP: return "HIP runtime or launch error";
    case SCAN_ERR_OVERFLOW: return "size exceeds an index type";
    }
    return "unknown status";
}

const char *scan_version(void) { return "scan_wave64 0.2 (gfx950)"; }

}  // extern "C"
