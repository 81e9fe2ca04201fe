// pipeline.hpp -- the persistent single-pass look-back drivers.  A tile
// policy P says how one tile is loaded, scanned and emitted; the driver owns
// tile ordering, descriptors, the look-back and the workspace protocol.
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
//  * A control wave owns the descriptors and the look-back, and scanned
//    tiles wait in LDS for their prefix (see CtrlPipeline's comment).
//  * In the static order a workgroup knows the inclusive prefix of its own
//    previous tile, so for grids of up to kGapGrid workgroups the look-back
//    reads only the aggregates published since (GapRead in device.hpp):
//    one round trip per tile and no chain of prefixes through a round.
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
    uint32_t delay_stride;    // test aid: tiles t with t % stride == stride - 1 publish late (0: off)
    uint32_t delay_sleeps;    // periods of s_sleep(64) those tiles wait before publishing
};

// The pipeline with a control wave and deferred emission, for policies whose
// carry is one value of type C.
//
// The workgroup is P::BLOCK data threads plus one extra wave that owns every
// descriptor access.  While HBM is saturated a descriptor round trip takes
// about 2 us (the request waits in the same queues as the tile traffic), so
// the look-back must not sit on the tile's critical path, and it must not
// need several round trips.  Hence:
//  * A scanned tile waits two steps in LDS before it is emitted (gfx950 has
//    160 KB of LDS per workgroup; each data thread stashes and later reads
//    back only its own slots, so no barrier guards the reuse).  By then the
//    aggregates of the whole round have long been published, and the
//    control wave's look-back for it completes in one round trip while the
//    data waves stream the next tiles.
//  * Descriptor reads are what the look-back costs: one round trip per
//    tile, issued a step before it is needed (GapRead); for larger grids and
//    in dynamic mode, windows of 64 predecessors per poll.  fp32 carries pack
//    into one word per tile (DescTrunc).
//  * On gfx950 a wave's vector memory counter retires loads and stores in
//    issue order: the control wave holds no tile traffic, so its polls are
//    never counted behind a tile.
//
// Tiles of workgroup w are T(k) = w + kG.  Step s (s = 0 .. K+1, K tiles):
//   data waves:    issue T(s+1)'s loads (the other register tile); scan T(s)
//                  (barrier 1); barrier 2; emit T(s-2) from its LDS stash
//                  with the prefix the control wave left; stash T(s).
//   control wave:  complete T(s-2)'s look-back and leave its exclusive
//                  prefix in LDS; barrier 1; combine T(s)'s per-wave totals
//                  into its aggregate and publish it (A, or P at a segment
//                  start); start T(s-1)'s look-back reads; barrier 2.  (With
//                  the windowed look-back, for large grids, T(s-2)'s whole
//                  look-back runs before barrier 1 and its inclusive prefix
//                  is published.)
// Every load a data wave issues is unconditional (a tile past the end loads
// the array's first vector and discards it), and so is every store of the
// scan policies (dropped past the end by the buffer resource), so the
// compiler counts the accesses in flight exactly and waits only for the
// tile it scans.
//
// Policy interface:
//   using T, C, Op, Args, Shared, Stash;  static constexpr int BLOCK, kDescWords
//   static C aggregate(const Shared&)     control wave, between the scan's
//                                         barrier and the next
//   static void emit(const Stash&, const Args&, uint32_t tile, C pre, bool valid, C total)
//                                         data threads; !valid: no effect;
//                                         total: what setup() returned
//   static constexpr bool kSetup          true: the control wave calls
//   static C setup(const Args&, const uint64_t *desc, uint32_t epoch, WsHeader*)
//                                         once, before the first barrier, and
//                                         the call always runs the workspace
//                                         protocol (epoch, end-of-call reset),
//                                         even with one tile, so setup() can
//                                         read words an earlier launch of the
//                                         same call tagged with the epoch
//   static void on_resolved(const Args&, uint32_t tile, C pre, C agg)
//                                         control lane 0, after the prefix
//   static constexpr bool kStagedEmit     optional; true: emit() reads stash
//                                         slots other threads wrote, so each
//                                         static-mode step has a third
//                                         barrier (both roles) between the
//                                         emit and the next stash
//   struct Tile {
//     void load(const Args&, uint32_t tile);   tile >= num_tiles: dummy loads
//     void scan(Shared&);                      exactly one __syncthreads()
//     void stash(Stash&, const Args&) const;   own slots only
//   };
template <class P>
struct CtrlPipeline {
    using Tile = typename P::Tile;
    using C = typename P::C;
    using Op = typename P::Op;
    using Args = typename P::Args;
    static constexpr int DATA = P::BLOCK;
    static constexpr int THREADS = DATA + kWave;
    static constexpr int kDepth = 1;  // look-back windows of 64 per round trip
    static constexpr int kGapReads = 8;  // GapRead slots per lane
    static constexpr uint32_t kGapGrid = kWave * kGapReads + 1;  // largest grid that uses GapRead
    static_assert(DATA % kWave == 0 && THREADS <= 1024, "whole waves");
    static constexpr bool kStaged = [] {
        if constexpr (requires { P::kStagedEmit; }) return bool(P::kStagedEmit);
        else return false;
    }();

    struct Smem {
        typename P::Stash stash[2];  // scanned tiles waiting for their prefix
        typename P::Shared ps;
        C prefix[2];  // exclusive prefix of the tile emitted in this step
        C total;      // setup()'s result
        uint32_t epoch, mode, ticket;
        uint64_t high_water, capacity;  // begin_call's, for end_call
    };

    // Whether a call runs the workspace protocol: every chained scan, and
    // every call of a policy with a setup step.
    __device__ __forceinline__ static bool protocol(const Args &a) { return a.pipe.tiles_per_seg > 1 || P::kSetup; }

    __device__ __forceinline__ static uint64_t *desc_of(uint64_t *desc, uint32_t tile) {
        return desc + uint64_t(tile) * P::kDescWords;
    }

    // Control wave, between the barrier of the data waves' scan of `tile`
    // and the next barrier: the tile's aggregate, published.
    __device__ __forceinline__ static C ctrl_publish(const Args &a, uint32_t tile, const Smem &sm, uint64_t *desc,
                                                     uint32_t epoch) {
        const C agg = P::aggregate(sm.ps);
        if (a.pipe.delay_stride > 0 && tile % a.pipe.delay_stride == a.pipe.delay_stride - 1) {
            // a late publisher, so tests reach the look-back's re-polls
            for (uint32_t i = 0; i < a.pipe.delay_sleeps; i++) __builtin_amdgcn_s_sleep(64);
        }
        if (a.pipe.tiles_per_seg > 1 && lane_id() == 0) {
            const uint32_t state = (tile % a.pipe.tiles_per_seg == 0) ? kStateP : kStateA;
            P::D::publish(desc_of(desc, tile), epoch, state, agg);
        }
        return agg;
    }

    // Control wave: the exclusive prefix of `tile` into `*prefix`.
    __device__ __forceinline__ static void ctrl_resolve(const Args &a, uint32_t tile, C agg, C *prefix, WsHeader *hdr,
                                                        uint64_t *desc, uint32_t epoch) {
        const uint32_t j = tile % a.pipe.tiles_per_seg;
        C pre = Op::template identity<C>();
        if (a.pipe.tiles_per_seg > 1 && j != 0) {
            pre = sw64::lookback<Op, C, kDepth, typename P::D>(desc, epoch, tile, int64_t(tile - j), hdr,
                                                               a.pipe.spin_limit);
            if (lane_id() == 0) P::D::publish(desc_of(desc, tile), epoch, kStateP, Op::apply(pre, agg));
        }
        if (lane_id() == 0) {
            *prefix = pre;
            P::on_resolved(a, tile, pre, agg);
        }
    }

    // Static-mode control wave with the aggregate-only look-back (GapRead):
    // for grids of at most kGapGrid workgroups.  Step s: combine the gap
    // reads issued one step earlier into T(s-2)'s exclusive prefix;
    // barrier 1; publish T(s)'s aggregate; issue T(s-1)'s gap reads, whose
    // aggregates were published a step or more before; barrier 2.  No
    // inclusive prefix is published, so every word read holds an aggregate
    // (a segment's first tile publishes its aggregate as P).
    __device__ __forceinline__ static void ctrl_static_gap(const Args &a, Smem &sm, WsHeader *hdr, uint64_t *desc,
                                                           uint32_t epoch, uint32_t K) {
        const uint32_t w = blockIdx.x, G = gridDim.x, tps = a.pipe.tiles_per_seg;
        const bool chained = tps > 1;
        const C id = Op::template identity<C>();
        C agg0 = id, agg1 = id;  // aggregates of T(s-2), T(s-1)
        C carry = id;            // inclusive prefix of this workgroup's last resolved tile
        bool use_carry = false;  // the gap being read continues from `carry`
        GapRead<C, typename P::D, kGapReads> gap;
        for (uint32_t s = 0; s < K + 2; s++) {
            if (s >= 2) {
                const uint32_t t = w + (s - 2) * G;
                C pre = id;
                if (chained) {
                    pre = gap.template finish<Op>(desc, epoch, hdr, a.pipe.spin_limit);
                    if (use_carry) pre = Op::apply(carry, pre);
                }
                carry = Op::apply(pre, agg0);
                if (lane_id() == 0) {
                    sm.prefix[s & 1] = pre;
                    P::on_resolved(a, t, pre, agg0);
                }
            }
            __syncthreads();
            agg0 = agg1;
            if (s < K) agg1 = ctrl_publish(a, w + s * G, sm, desc, epoch);
            if (chained && s >= 1 && s <= K) {
                const int64_t t = int64_t(w) + int64_t(s - 1) * G;
                const int64_t first = t - int64_t(uint32_t(t) % tps);  // segment start
                use_carry = t - int64_t(G) >= first;
                gap.issue(desc, use_carry ? t - G + 1 : first, t);
            }
            __syncthreads();
            if constexpr (kStaged) __syncthreads();
        }
    }

    // One static-mode step of the data waves: `cur` holds T(s), `other`
    // receives T(s+1).  Returns false after the last step.
    __device__ __forceinline__ static bool data_step(Tile &cur, Tile &other, const Args &a, uint32_t s, uint32_t K,
                                                     Smem &sm) {
        const uint32_t w = blockIdx.x, G = gridDim.x;
        other.load(a, s + 1 < K ? w + (s + 1) * G : a.pipe.num_tiles);
        if (s < K)
            cur.scan(sm.ps);
        else
            __syncthreads();
        __syncthreads();
        const bool emit = s >= 2;
        P::emit(sm.stash[s & 1], a, emit ? w + (s - 2) * G : a.pipe.num_tiles, sm.prefix[s & 1], emit, sm.total);
        if constexpr (kStaged) __syncthreads();
        if (s < K) cur.stash(sm.stash[s & 1], a);
        return s + 1 < K + 2;
    }

    // The kernel body.  The host launches THREADS threads per workgroup, at
    // most as many workgroups as can be resident and no more than there are
    // tiles.  The two roles run separate loops with the same sequence of
    // barriers (two per step), so the control wave keeps no tile registers
    // live.
    __device__ __forceinline__ static void run(const Args &a) {
        __shared__ Smem sm;
        WsHeader *hdr = reinterpret_cast<WsHeader *>(a.pipe.ws);
        uint64_t *desc = reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(a.pipe.ws) + kWsHeaderBytes);
        const uint32_t n = a.pipe.num_tiles, G = gridDim.x, w = blockIdx.x;
        const uint32_t K = (n - w + G - 1) / G;  // tiles of this workgroup (>= 1)
        const bool chained = protocol(a);
        // Wave-uniform role (a scalar branch: no wave ever runs both sides).
        const bool ctrl = uniform(uint32_t(threadIdx.x)) >= uint32_t(DATA);

        if (ctrl) {
            uint32_t e = 0;
            if (chained && lane_id() == 0) {
                uint64_t hw = 0, cap = 0;
                e = begin_call(hdr, hw, cap);
                sm.epoch = e;
                sm.high_water = hw;
                sm.capacity = cap;
                sm.mode = decide_mode(hdr, e, G, a.pipe.mode_limit);
            }
            if constexpr (P::kSetup) {
                const C t = P::setup(a, desc, uniform(e), hdr);  // uniform(): lane 0's epoch
                if (lane_id() == 0) sm.total = t;
            }
            __syncthreads();
            const uint32_t epoch = chained ? sm.epoch : 0u;
            const uint32_t mode = chained ? sm.mode : kModeStatic;
            if (mode == kModeStatic && G <= kGapGrid) {
                ctrl_static_gap(a, sm, hdr, desc, epoch, K);
                end_static(a, sm, hdr, desc, epoch);
            } else if (mode == kModeStatic) {
                C agg0 = Op::template identity<C>(), agg1 = agg0;  // aggregates of T(s-2), T(s-1)
                for (uint32_t s = 0; s < K + 2; s++) {
                    if (s >= 2) ctrl_resolve(a, w + (s - 2) * G, agg0, &sm.prefix[s & 1], hdr, desc, epoch);
                    __syncthreads();
                    agg0 = agg1;
                    if (s < K) agg1 = ctrl_publish(a, w + s * G, sm, desc, epoch);
                    __syncthreads();
                    if constexpr (kStaged) __syncthreads();
                }
                end_static(a, sm, hdr, desc, epoch);
            } else {
                ctrl_dynamic(a, sm, hdr, desc, epoch);
            }
            return;
        }

        Tile b0, b1;
        b0.load(a, w);
        __syncthreads();
        const uint32_t epoch = chained ? sm.epoch : 0u;
        const uint32_t mode = chained ? sm.mode : kModeStatic;
        if (mode == kModeStatic) {
            for (uint32_t s = 0;; s += 2) {
                if (!data_step(b0, b1, a, s, K, sm)) break;
                if (!data_step(b1, b0, a, s + 1, K, sm)) break;
            }
            end_static(a, sm, hdr, desc, epoch);
            return;
        }

        // Dynamic mode (data waves): one tile at a time, in claim order.
        for (;;) {
            __syncthreads();
            const uint32_t tk = sm.ticket;
            if (tk >= n) {
                if (tk == n + G - 1) end_call(hdr, epoch, sm.high_water, sm.capacity, a.pipe.words_used, a.pipe.ws_words, desc);
                break;
            }
            b0.load(a, tk);
            b0.scan(sm.ps);
            b0.stash(sm.stash[0], a);
            __syncthreads();
            __syncthreads();
            P::emit(sm.stash[0], a, tk, sm.prefix[0], true, sm.total);
        }
    }

    // End of a static call: the workgroup that owns the last tile resets the
    // workspace header (whole workgroup, both roles).
    __device__ __forceinline__ static void end_static(const Args &a, Smem &sm, WsHeader *hdr, uint64_t *desc,
                                                      uint32_t epoch) {
        const uint32_t n = a.pipe.num_tiles, G = gridDim.x;
        if (protocol(a) && blockIdx.x == (n - 1) % G)
            end_call(hdr, epoch, sm.high_water, sm.capacity, a.pipe.words_used, a.pipe.ws_words, desc);
    }

    // Dynamic mode (control wave): claim a tile, then resolve it.  Every
    // workgroup makes exactly one claim past the last tile, so the holder of
    // ticket n + G - 1 knows all others are done with the header.  Barriers
    // per tile match the data waves': claim; scan; aggregate; prefix.
    __device__ __forceinline__ static void ctrl_dynamic(const Args &a, Smem &sm, WsHeader *hdr, uint64_t *desc,
                                                        uint32_t epoch) {
        const uint32_t n = a.pipe.num_tiles, G = gridDim.x;
        for (;;) {
            if (lane_id() == 0)
                sm.ticket = __hip_atomic_fetch_add(&hdr->claim, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            const uint32_t tk = sm.ticket;
            if (tk >= n) {
                if (tk == n + G - 1) end_call(hdr, epoch, sm.high_water, sm.capacity, a.pipe.words_used, a.pipe.ws_words, desc);
                break;
            }
            __syncthreads();
            const C agg = ctrl_publish(a, tk, sm, desc, epoch);
            __syncthreads();
            ctrl_resolve(a, tk, agg, &sm.prefix[0], hdr, desc, epoch);
            __syncthreads();
        }
    }
};

// Workgroups of a kernel that can be resident at once on the current device,
// cached per kernel.  The runtime's occupancy figure is trusted only up to 6
// waves per SIMD (24 per compute unit): grids at the bound a kernel's
// resources set (8 waves, or 7 for the 64-bit kernels of 256 threads) were
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
