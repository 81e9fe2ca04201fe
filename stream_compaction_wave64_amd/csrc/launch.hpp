// launch.hpp -- host-side interface between the C ABI (api.hip) and the kernel
// translation units.  Each kernel family exposes a lookup that returns a
// launcher for a (dtype, op, shape) combination, or nullptr when that
// combination is not instantiated.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "scan_wave64.h"

namespace sw64 {

// ---------------------------------------------------------------- look-back
// One launch of a persistent grid of at most resident-capacity workgroups of
// `block` threads; workgroup w scans tiles w, w+G, ... of block*rows*vec
// elements.  Segments (rows of a (outer, len, 1)
// array) are seg_len elements long and split into tiles_per_seg tiles; the
// look-back never crosses a segment start.
struct LbArgs {
    const void *in;
    void *out;
    int64_t seg_len;          // elements per segment
    uint32_t tiles_per_seg;   // tiles per segment (>= 1)
    uint32_t num_tiles;       // segments * tiles_per_seg (grid size)
    int32_t exclusive;        // 0 inclusive, 1 exclusive
    void *total_out;          // optional: per-segment total, written by its last tile
    void *ws;                 // workspace (header + descriptors)
    uint64_t ws_words;        // descriptor words the workspace holds
    uint64_t words_used;      // descriptor words this launch writes
    uint32_t spin_limit;      // polls of one look-back window before giving up
    uint32_t grid_blocks;     // cap on the persistent grid (0 = resident capacity)
    uint32_t mode_limit;      // polls before a call falls back to dynamic claiming
};
using LbLaunch = int (*)(const LbArgs &, hipStream_t);
LbLaunch find_lookback(scan_dtype_t dt, scan_op_t op, int block, int rows, int vec);

// ---------------------------------------------------------- reduce-then-scan
// Three launches over `blocks` workgroups, each owning `chunk_tiles`
// consecutive tiles of block*rows*vec elements: reduce each chunk into a
// partial, scan the partials in one workgroup, rescan each chunk from its
// base.  `partials` points at blocks carry values inside the workspace; the
// last launch zeroes them again so the workspace stays clean for the
// look-back descriptors.
struct RtsArgs {
    const void *in;
    void *out;
    int64_t n;
    uint32_t blocks;
    uint32_t chunk_tiles;
    int32_t exclusive;
    void *partials;
};
using RtsLaunch = int (*)(const RtsArgs &, hipStream_t);
RtsLaunch find_rts(scan_dtype_t dt, scan_op_t op, int block, int rows, int vec);

// -------------------------------------------------------------- utilities
int launch_fill_u64(void *p, uint64_t words, uint64_t value, hipStream_t s);
int launch_fill_i32(int32_t *p, int64_t count, int32_t value, hipStream_t s);
int launch_copy(const void *in, void *out, size_t bytes, hipStream_t s);

}  // namespace sw64
