// lookback.hip -- single-pass decoupled look-back scan (The CUDA Handbook
// ch. 13, decoupled look-back section with Figure 13-11, and section 13.3.5's
// items-per-thread kernel), segmented so the same kernel scans a whole array
// (one segment) or every row of an (outer, len, 1) array.
//
// MI355X design (differs from the page's kernel, which gives each block one
// tile claimed from a global atomic counter):
//  * Persistent grid.  The host launches G workgroups, no more than can be
//    resident at once, and workgroup w scans tiles w, w + G, w + 2G, ... in
//    order.  When all G are resident, the lowest unfinished tile always
//    belongs to a running workgroup whose predecessors are all finished, so
//    the look-back cannot deadlock -- the guarantee the page gets from its
//    counter, without one same-address atomic per tile (on MI355X those
//    serialize at ~11.5 ns each; 12k of them exceed the whole HBM time of a
//    1e8-element scan).  Residency is checked at run time: if not all G
//    workgroups start promptly, the call falls back to claiming tiles in
//    order from a counter, as the page does (see decide_mode).
//  * Software pipeline.  Each workgroup keeps three register tiles: while it
//    looks back on tile t, tile t + G is already scanned with its aggregate
//    published, and the loads of t + 2G are in flight.  Look-back latency
//    overlaps HBM traffic, and a look-back only waits on aggregates that
//    were published a step earlier.
//  * Everything else per tile: 128-bit nontemporal loads, the register tile
//    scan (tile.hpp), wave 0 publishes A, looks back over the predecessors in
//    the same segment, publishes P; all waves add the prefix and store.
//
// This file is compiled once per element type (SW64_DT selects it) so the
// instantiations build in parallel.
#include <mutex>

#include "launch.hpp"
#include "tile.hpp"

namespace sw64 {

// Look-back window depth: DEPTH x 64 predecessors per round trip.
constexpr int kLookbackDepth = 1;

template <class T, class Op, int BLOCK, int ROWS, int VEC>
struct LookbackScan {
    using TS = TileScan<T, Op, BLOCK, ROWS, VEC>;
    using C = typename TS::C;

    struct Smem {
        typename TS::Shared sh;
        C prefix;
        uint32_t epoch, mode, ticket;
        uint64_t clear_end;
    };

    struct Geom {
        int64_t start, remaining;
        uint32_t seg, j;
    };

    __device__ __forceinline__ static Geom geom(const LbArgs &a, uint32_t tile) {
        Geom g;
        g.seg = tile / a.tiles_per_seg;
        g.j = tile - g.seg * a.tiles_per_seg;
        g.start = int64_t(g.seg) * a.seg_len + int64_t(g.j) * TS::TILE;
        g.remaining = a.seg_len - int64_t(g.j) * TS::TILE;
        return g;
    }

    __device__ __forceinline__ static uint64_t *desc_of(uint64_t *desc, uint32_t tile) {
        return desc + uint64_t(tile) * Desc<C>::kWords;
    }

    __device__ __forceinline__ static void load(TS &ts, const LbArgs &a, uint32_t tile) {
        const Geom g = geom(a, tile);
        ts.load(reinterpret_cast<const T *>(a.in) + g.start, g.remaining);
    }

    // Stage 1: scan a loaded tile and publish its aggregate (A), or its
    // inclusive prefix (P) if it opens its segment.  One barrier.
    __device__ __forceinline__ static void scan_publish(TS &ts, const LbArgs &a, uint32_t tile, Smem &sm,
                                                        uint64_t *desc, uint32_t epoch) {
        ts.scan(sm.sh);
        if (a.tiles_per_seg > 1 && threadIdx.x == 0) {
            const uint32_t state = (tile % a.tiles_per_seg == 0) ? kStateP : kStateA;
            Desc<C>::publish(desc_of(desc, tile), (epoch << 2) | state, C(ts.agg));
        }
    }

    // Stage 2: look back for the tile's exclusive prefix, publish P, add the
    // prefix and store.  One barrier.
    __device__ __forceinline__ static void finish(TS &ts, const LbArgs &a, uint32_t tile, Smem &sm,
                                                  WsHeader *hdr, uint64_t *desc, uint32_t epoch) {
        const Geom g = geom(a, tile);
        if (threadIdx.x < kWave) {
            const int lane = lane_id();
            const C agg = C(ts.agg);
            C pre = Op::template identity<C>();
            if (a.tiles_per_seg > 1 && g.j != 0) {
                pre = lookback<Op, C, kLookbackDepth>(desc, epoch, tile, int64_t(g.seg) * a.tiles_per_seg, hdr,
                                                       a.spin_limit);
                if (lane == 0) Desc<C>::publish(desc_of(desc, tile), (epoch << 2) | kStateP, Op::apply(pre, agg));
            }
            if (lane == 0) {
                sm.prefix = pre;
                if (a.total_out != nullptr && g.j == a.tiles_per_seg - 1)
                    reinterpret_cast<T *>(a.total_out)[g.seg] = T(Op::apply(pre, agg));
            }
        }
        __syncthreads();
        ts.store(reinterpret_cast<T *>(a.out) + g.start, g.remaining, sm.prefix, a.exclusive != 0);
    }

    // One pipeline step with tile t in `cur` (scanned, A published), t + G in
    // `nxt` (loaded) and t + 2G to be loaded into `fut`: the loads of t + 2G
    // are issued first, then t + G is scanned and its A published, and only
    // then does tile t wait for its look-back.  A look-back therefore waits
    // on aggregates that were published one step earlier, so one slow
    // look-back does not hold back the next round's aggregates.
    // Returns false when t + G is past the end.
    __device__ __forceinline__ static bool step(TS &cur, TS &nxt, TS &fut, const LbArgs &a, uint32_t t, Smem &sm,
                                                WsHeader *hdr, uint64_t *desc, uint32_t epoch) {
        const uint32_t n = a.num_tiles, G = gridDim.x;
        const uint32_t tn = t + G, tf = tn + G;
        if (tf < n) load(fut, a, tf);
        if (tn < n) scan_publish(nxt, a, tn, sm, desc, epoch);
        finish(cur, a, t, sm, hdr, desc, epoch);
        return tn < n;
    }
};

template <class T, class Op, int BLOCK, int ROWS, int VEC>
__global__ __launch_bounds__(BLOCK) void k_lookback(LbArgs a) {
    using K = LookbackScan<T, Op, BLOCK, ROWS, VEC>;
    __shared__ typename K::Smem sm;
    WsHeader *hdr = reinterpret_cast<WsHeader *>(a.ws);
    uint64_t *desc = reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(a.ws) + kWsHeaderBytes);
    const uint32_t n = a.num_tiles, G = gridDim.x;
    // Segments of a single tile need no look-back: their tiles are
    // independent and the header is not touched.
    const bool chained = a.tiles_per_seg > 1;
    if (chained && threadIdx.x == 0) sm.epoch = begin_call(hdr);

    // Three register tiles in rotation (scanned and waiting / loaded / in
    // flight).  The first two loads are issued before the mode is known;
    // dynamic mode drops them.  The host guarantees blockIdx.x < n.
    typename K::TS b0, b1, b2;
    uint32_t t = blockIdx.x;
    K::load(b0, a, t);
    if (t + G < n) K::load(b1, a, t + G);
    uint32_t epoch = 0, mode = kModeStatic;
    if (chained) {
        if (threadIdx.x == 0) sm.mode = decide_mode(hdr, G, a.mode_limit);
        __syncthreads();
        epoch = sm.epoch;
        mode = sm.mode;
    }

    if (mode == kModeStatic) {
        K::scan_publish(b0, a, t, sm, desc, epoch);
        for (;;) {
            if (!K::step(b0, b1, b2, a, t, sm, hdr, desc, epoch)) break;
            t += G;
            if (!K::step(b1, b2, b0, a, t, sm, hdr, desc, epoch)) break;
            t += G;
            if (!K::step(b2, b0, b1, a, t, sm, hdr, desc, epoch)) break;
            t += G;
        }
        if (chained && blockIdx.x == (n - 1) % G)
            end_call_static(hdr, G, epoch, a.words_used, a.ws_words, desc, a.spin_limit, sm.clear_end);
        return;
    }

    // Dynamic mode: one tile at a time, claimed in order.  Every workgroup
    // makes exactly one claim past the last tile, so the holder of ticket
    // n + G - 1 knows all others are done with the header and ends the call.
    for (;;) {
        if (threadIdx.x == 0)
            sm.ticket = __hip_atomic_fetch_add(&hdr->claim, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const uint32_t tk = sm.ticket;
        if (tk >= n) {
            if (tk == n + G - 1) end_call(hdr, epoch, a.words_used, a.ws_words, desc, sm.clear_end);
            break;
        }
        K::load(b0, a, tk);
        K::scan_publish(b0, a, tk, sm, desc, epoch);
        K::finish(b0, a, tk, sm, hdr, desc, epoch);
    }
}

// Workgroups of a kernel that can be resident at once on the current device,
// cached per kernel.  The runtime's occupancy figure is trusted only up to 7
// waves per SIMD (28 per compute unit): at the full 8 the grid it implies was
// measured not to fit at once.  The kernel verifies residency itself (static
// or dynamic mode), so this only keeps the fast path the common one.
static int resident_blocks(const void *kernel, int waves_per_block) {
    const int block = waves_per_block * kWave;
    static std::mutex mu;
    static const void *keys[256];
    static int devs[256], vals[256], count = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < count; i++)
        if (keys[i] == kernel && devs[i] == dev) return vals[i];
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (per_cu * waves_per_block > 28) per_cu = 28 / waves_per_block > 0 ? 28 / waves_per_block : 1;
    const int v = per_cu * cus;
    if (count < 256) {
        keys[count] = kernel;
        devs[count] = dev;
        vals[count] = v;
        count++;
    }
    return v;
}

template <class T, class Op, int B, int R, int V>
static int launch_lookback_impl(const LbArgs &a, hipStream_t s) {
    const void *kern = reinterpret_cast<const void *>(&k_lookback<T, Op, B, R, V>);
    int g = resident_blocks(kern, B / kWave);
    if (g <= 0) return SCAN_ERR_HIP;
    if (a.grid_blocks > 0 && uint32_t(g) > a.grid_blocks) g = int(a.grid_blocks);
    if (uint32_t(g) > a.num_tiles) g = int(a.num_tiles);
    hipLaunchKernelGGL((k_lookback<T, Op, B, R, V>), dim3(g), dim3(B), 0, s, a);
    return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
}

// Instantiated (block, rows) shapes.  Every type gets the default shape
// (512 threads x 8 rows of 128-bit vectors, 64 KiB per tile, the best
// measured on MI355X; 4 rows for 8-byte elements) and a one-row shape (small tiles, used to force many
// tiles at small n); fp32 sum also gets the shapes the tuning sweep visits.
template <class T, class Op, int V>
static LbLaunch pick_shape(int block, int rows) {
#define SW64_SHAPE(B, R) \
    if (block == B && rows == R) return &launch_lookback_impl<T, Op, B, R, V>;
    SW64_SHAPE(256, 1)
    if constexpr (sizeof(T) == 4) {
        SW64_SHAPE(512, 8)
    } else {
        SW64_SHAPE(512, 4)  // 8-byte elements: 8 rows would spill past 256 VGPRs
    }
    if constexpr (std::is_same_v<T, float> && std::is_same_v<Op, OpSum>) {
        SW64_SHAPE(256, 2)
        SW64_SHAPE(256, 4)
        SW64_SHAPE(256, 8)
        SW64_SHAPE(512, 2)
        SW64_SHAPE(512, 4)
        SW64_SHAPE(1024, 2)
    }
#undef SW64_SHAPE
    return nullptr;
}

template <class T, class Op>
static LbLaunch pick_vec(int block, int rows, int vec) {
    constexpr int VMAX = 16 / int(sizeof(T));
    if (vec == VMAX) return pick_shape<T, Op, VMAX>(block, rows);
    if (vec == 1) return pick_shape<T, Op, 1>(block, rows);
    return nullptr;
}

template <class T>
static LbLaunch pick_op(scan_op_t op, int block, int rows, int vec) {
    switch (op) {
    case SCAN_OP_SUM: return pick_vec<T, OpSum>(block, rows, vec);
    case SCAN_OP_PROD: return pick_vec<T, OpProd>(block, rows, vec);
    case SCAN_OP_MAX: return pick_vec<T, OpMax>(block, rows, vec);
    case SCAN_OP_MIN: return pick_vec<T, OpMin>(block, rows, vec);
    }
    return nullptr;
}

#if SW64_DT == 0
LbLaunch find_lookback_i32(scan_op_t op, int b, int r, int v) { return pick_op<int32_t>(op, b, r, v); }
#elif SW64_DT == 1
LbLaunch find_lookback_u32(scan_op_t op, int b, int r, int v) { return pick_op<uint32_t>(op, b, r, v); }
#elif SW64_DT == 2
LbLaunch find_lookback_i64(scan_op_t op, int b, int r, int v) { return pick_op<int64_t>(op, b, r, v); }
#elif SW64_DT == 3
LbLaunch find_lookback_f32(scan_op_t op, int b, int r, int v) { return pick_op<float>(op, b, r, v); }
#elif SW64_DT == 4
LbLaunch find_lookback_f64(scan_op_t op, int b, int r, int v) { return pick_op<double>(op, b, r, v); }
#else
#error "SW64_DT must select an element type (0..4)"
#endif

}  // namespace sw64
