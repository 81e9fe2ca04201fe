// pipeline.hpp -- the persistent, software-pipelined single-pass look-back
// driver shared by every look-back kernel (plain scans, compaction, element
// scans).  A tile policy P says how one tile is loaded, scanned and emitted;
// the driver owns tile ordering, descriptors, the look-back and the
// workspace protocol.
//
// Method: The CUDA Handbook ch. 13, decoupled look-back section (Figure
// 13-11): each tile publishes its aggregate (A), looks back over its
// predecessors for its exclusive prefix, then publishes its inclusive
// prefix (P).  MI355X design, differing from the page:
//  * Persistent grid of G resident workgroups; workgroup w scans tiles w,
//    w + G, ... in order.  When all G are resident the lowest unfinished
//    tile always belongs to a running workgroup whose predecessors are all
//    finished, so the look-back cannot deadlock -- the guarantee the page
//    gets from an atomic tile counter, whose same-address atomics serialize
//    at ~11.5 ns each on MI355X (12k of them exceed the HBM time of a
//    1e8-element scan).  Residency is verified at run time (decide_mode);
//    without it the call claims tiles in order from a counter instead.
//  * Software pipeline: three register tiles per workgroup.  While tile t
//    waits for its look-back, tile t + G is already scanned with its
//    aggregate published and the loads of t + 2G are in flight, so one slow
//    look-back does not hold back the next round's aggregates.
//
// Policy interface (all __device__):
//   using T, C (carry type), Op;   static constexpr int BLOCK, kDescWords
//   struct Args { PipeArgs pipe; ... }
//   struct Shared;                 LDS the tile scan needs
//   struct Tile {
//     void set_slot(int);          which of the three pipeline buffers it is
//     void load(const Args&, uint32_t tile);
//     void scan(Shared&);          one barrier; afterwards aggregate() valid
//     C aggregate() const;
//     void emit(const Args&, uint32_t tile, const C* prefix);  prefix in LDS
//   };
//   static void publish_aggregate(Tile&, uint64_t* desc, uint32_t tag);  thread 0
//   static void resolve(Tile&, ...);   wave 0: look back, publish P, write the
//                                      exclusive prefix to LDS
//   static void set_identity(C* prefix);   lane 0
#pragma once

#include "device.hpp"

namespace sw64 {

struct PipeArgs {
    void *ws;                 // workspace (header + descriptors)
    uint64_t ws_words;        // descriptor words the workspace holds
    uint64_t words_used;      // descriptor words this launch writes
    uint32_t num_tiles;       // segments * tiles_per_seg
    uint32_t tiles_per_seg;   // tiles per segment (>= 1)
    uint32_t spin_limit;      // polls of one look-back window before giving up
    uint32_t mode_limit;      // polls before a call falls back to dynamic claiming
};

template <class P>
struct Pipeline {
    using Tile = typename P::Tile;
    using C = typename P::C;
    using Args = typename P::Args;

    struct Smem {
        typename P::Shared ps;
        C prefix;
        uint32_t epoch, mode, ticket;
        uint64_t clear_end;
    };

    __device__ __forceinline__ static uint64_t *desc_of(uint64_t *desc, uint32_t tile) {
        return desc + uint64_t(tile) * P::kDescWords;
    }

    // Stage 1: scan a loaded tile and publish its aggregate (A), or its
    // inclusive prefix (P) if it opens its segment.  One barrier.
    __device__ __forceinline__ static void scan_publish(Tile &ts, const Args &a, uint32_t tile, Smem &sm,
                                                        uint64_t *desc, uint32_t epoch) {
        ts.scan(sm.ps);
        if (a.pipe.tiles_per_seg > 1 && threadIdx.x == 0) {
            const uint32_t state = (tile % a.pipe.tiles_per_seg == 0) ? kStateP : kStateA;
            P::publish_aggregate(ts, desc_of(desc, tile), (epoch << 2) | state);
        }
    }

    // Stage 2: look back for the tile's exclusive prefix (wave 0), publish
    // P, then every thread emits the tile with the prefix.  One barrier.
    __device__ __forceinline__ static void finish(Tile &ts, const Args &a, uint32_t tile, Smem &sm, WsHeader *hdr,
                                                  uint64_t *desc, uint32_t epoch) {
        const uint32_t j = tile % a.pipe.tiles_per_seg;
        if (threadIdx.x < kWave) {
            if (a.pipe.tiles_per_seg > 1 && j != 0)
                P::resolve(ts, desc, epoch, tile, int64_t(tile - j), hdr, a.pipe.spin_limit, &sm.prefix);
            else
                P::set_identity(&sm.prefix);
        }
        __syncthreads();
        ts.emit(a, tile, &sm.prefix);
    }

    // One pipeline step (see the header comment).  Returns false when tile
    // t + G is past the end.
    __device__ __forceinline__ static bool step(Tile &cur, Tile &nxt, Tile &fut, const Args &a, uint32_t t,
                                                Smem &sm, WsHeader *hdr, uint64_t *desc, uint32_t epoch) {
        const uint32_t n = a.pipe.num_tiles, G = gridDim.x;
        const uint32_t tn = t + G, tf = tn + G;
        if (tf < n) fut.load(a, tf);
        if (tn < n) scan_publish(nxt, a, tn, sm, desc, epoch);
        finish(cur, a, t, sm, hdr, desc, epoch);
        return tn < n;
    }

    // The kernel body.  The host launches at most as many workgroups as can
    // be resident and no more than there are tiles.
    __device__ __forceinline__ static void run(const Args &a) {
        __shared__ Smem sm;
        WsHeader *hdr = reinterpret_cast<WsHeader *>(a.pipe.ws);
        uint64_t *desc = reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(a.pipe.ws) + kWsHeaderBytes);
        const uint32_t n = a.pipe.num_tiles, G = gridDim.x;
        // Segments of a single tile need no look-back: their tiles are
        // independent and the header is not touched.
        const bool chained = a.pipe.tiles_per_seg > 1;
        if (chained && threadIdx.x == 0) sm.epoch = begin_call(hdr);

        // Three register tiles in rotation (scanned and waiting / loaded /
        // in flight).  The first two loads are issued before the mode is
        // known; dynamic mode drops them.
        Tile b0, b1, b2;
        b0.set_slot(0);
        b1.set_slot(1);
        b2.set_slot(2);
        uint32_t t = blockIdx.x;
        b0.load(a, t);
        if (t + G < n) b1.load(a, t + G);
        uint32_t epoch = 0, mode = kModeStatic;
        if (chained) {
            if (threadIdx.x == 0) sm.mode = decide_mode(hdr, G, a.pipe.mode_limit);
            __syncthreads();
            epoch = sm.epoch;
            mode = sm.mode;
        }

        if (mode == kModeStatic) {
            scan_publish(b0, a, t, sm, desc, epoch);
            for (;;) {
                if (!step(b0, b1, b2, a, t, sm, hdr, desc, epoch)) break;
                t += G;
                if (!step(b1, b2, b0, a, t, sm, hdr, desc, epoch)) break;
                t += G;
                if (!step(b2, b0, b1, a, t, sm, hdr, desc, epoch)) break;
                t += G;
            }
            if (chained && blockIdx.x == (n - 1) % G)
                end_call_static(hdr, G, epoch, a.pipe.words_used, a.pipe.ws_words, desc, a.pipe.spin_limit,
                                sm.clear_end);
            return;
        }

        // Dynamic mode: one tile at a time, claimed in order.  Every
        // workgroup makes exactly one claim past the last tile, so the holder
        // of ticket n + G - 1 knows all others are done with the header.
        for (;;) {
            if (threadIdx.x == 0)
                sm.ticket = __hip_atomic_fetch_add(&hdr->claim, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            const uint32_t tk = sm.ticket;
            if (tk >= n) {
                if (tk == n + G - 1) end_call(hdr, epoch, a.pipe.words_used, a.pipe.ws_words, desc, sm.clear_end);
                break;
            }
            b0.load(a, tk);
            scan_publish(b0, a, tk, sm, desc, epoch);
            finish(b0, a, tk, sm, hdr, desc, epoch);
        }
    }
};

// Descriptor I/O and look-back for a policy whose carry is one value of type
// C (scalar scans and compaction); its Tile provides aggregate().
template <class Op, class C>
struct ScalarCarry {
    static constexpr int kDescWords = Desc<C>::kWords;

    template <class Tile>
    __device__ __forceinline__ static void publish_aggregate(const Tile &ts, uint64_t *d, uint32_t tag) {
        Desc<C>::publish(d, tag, ts.aggregate());
    }

    template <class Tile>
    __device__ __forceinline__ static void resolve(const Tile &ts, const uint64_t *desc, uint32_t epoch,
                                                   uint32_t tile, int64_t first, WsHeader *hdr, uint32_t spin_limit,
                                                   C *prefix) {
        const C agg = ts.aggregate();
        const C pre = sw64::lookback<Op, C, 1>(desc, epoch, tile, first, hdr, spin_limit);
        if (lane_id() == 0) {
            Desc<C>::publish(const_cast<uint64_t *>(desc) + uint64_t(tile) * kDescWords, (epoch << 2) | kStateP,
                             Op::apply(pre, agg));
            *prefix = pre;
        }
    }

    __device__ __forceinline__ static void set_identity(C *prefix) {
        if (lane_id() == 0) *prefix = Op::template identity<C>();
    }
};

// Workgroups of a kernel that can be resident at once on the current device,
// cached per kernel.  The runtime's occupancy figure is trusted only up to 7
// waves per SIMD (28 per compute unit): at the full 8 the grid it implies was
// measured not to fit at once.  The kernel verifies residency itself
// (decide_mode), so this only keeps the fast path the common one.
int resident_blocks(const void *kernel, int waves_per_block);

// Grid of a persistent pipeline launch, or 0 on a runtime error.
inline int pipeline_grid(const void *kernel, int block, uint32_t num_tiles, uint32_t cap) {
    int g = resident_blocks(kernel, block / kWave);
    if (g <= 0) return 0;
    if (cap > 0 && uint32_t(g) > cap) g = int(cap);
    if (uint32_t(g) > num_tiles) g = int(num_tiles);
    return g;
}

}  // namespace sw64
