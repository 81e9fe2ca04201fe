// lookback.hip -- single-pass decoupled look-back scan (The CUDA Handbook
// ch. 13, decoupled look-back section with Figure 13-11, and section 13.3.5's
// items-per-thread kernel), segmented so the same kernel scans a whole array
// (one segment) or every row of an (outer, len, 1) array.
//
// MI355X design (differs from the page's kernel, which gives each block one
// tile claimed from a global atomic counter):
//  * Persistent grid.  The host launches G workgroups, no more than can be
//    resident at once (occupancy x compute units), and workgroup w scans
//    tiles w, w + G, w + 2G, ... in order.  Because all G are resident, the
//    lowest unfinished tile always belongs to a running workgroup whose
//    predecessors are all finished, so the look-back cannot deadlock -- the
//    guarantee the page gets from its counter, without one same-address
//    atomic per tile (on MI355X those serialize at ~11 ns each, more than the
//    whole HBM time of a 1e8-element scan's tiles).
//  * Prefetch.  While a workgroup scans and looks back on tile t, the loads
//    of its next tile t + G are already in flight in a second register set,
//    so look-back latency overlaps HBM traffic.
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

template <class T, class Op, int BLOCK, int ROWS, int VEC>
struct LookbackScan {
    using TS = TileScan<T, Op, BLOCK, ROWS, VEC>;
    using C = typename TS::C;

    struct Smem {
        typename TS::Shared sh;
        C prefix;
        uint32_t epoch;
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

    __device__ __forceinline__ static void load(TS &ts, const LbArgs &a, uint32_t tile) {
        const Geom g = geom(a, tile);
        ts.load(reinterpret_cast<const T *>(a.in) + g.start, g.remaining);
    }

    // Scan, look back and store one loaded tile.  Two barriers.
    __device__ __forceinline__ static void process(TS &ts, const LbArgs &a, uint32_t tile, Smem &sm,
                                                   WsHeader *hdr, uint64_t *desc, uint32_t epoch) {
        const Geom g = geom(a, tile);
        ts.scan(sm.sh);
        if (threadIdx.x < kWave) {
            const int lane = lane_id();
            const C agg = C(ts.agg);
            C pre = Op::template identity<C>();
            if (a.tiles_per_seg > 1) {
                uint64_t *d = desc + uint64_t(tile) * Desc<C>::kWords;
                const uint32_t tag = epoch << 2;
                if (g.j == 0) {
                    if (lane == 0) Desc<C>::publish(d, tag | kStateP, agg);
                } else {
                    if (lane == 0) Desc<C>::publish(d, tag | kStateA, agg);
                    pre = lookback<Op, C>(desc, epoch, tile, int64_t(g.seg) * a.tiles_per_seg, hdr, a.spin_limit);
                    if (lane == 0) Desc<C>::publish(d, tag | kStateP, Op::apply(pre, agg));
                }
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
};

template <class T, class Op, int BLOCK, int ROWS, int VEC>
__global__ __launch_bounds__(BLOCK) void k_lookback(LbArgs a) {
    using K = LookbackScan<T, Op, BLOCK, ROWS, VEC>;
    __shared__ typename K::Smem sm;
    WsHeader *hdr = reinterpret_cast<WsHeader *>(a.ws);
    uint64_t *desc = reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(a.ws) + kWsHeaderBytes);
    const bool chained = a.tiles_per_seg > 1;
    const uint32_t epoch = chained ? begin_call(hdr, sm.epoch) : 0u;
    const uint32_t n = a.num_tiles, G = gridDim.x;

    // Two register tiles, alternating: the next tile's loads are issued before
    // the current one is scanned.  The host guarantees blockIdx.x < n.
    typename K::TS b0, b1;
    uint32_t t = blockIdx.x;
    K::load(b0, a, t);
    for (;;) {
        const uint32_t t1 = t + G;
        if (t1 < n) K::load(b1, a, t1);
        K::process(b0, a, t, sm, hdr, desc, epoch);
        if (t1 >= n) break;
        const uint32_t t2 = t1 + G;
        if (t2 < n) K::load(b0, a, t2);
        K::process(b1, a, t1, sm, hdr, desc, epoch);
        if (t2 >= n) break;
        t = t2;
    }
    if (chained && blockIdx.x == (n - 1) % G)
        end_call(hdr, G, epoch, a.words_used, a.ws_words, desc, a.spin_limit, sm.clear_end);
}

// Resident workgroups of a kernel on the current device, cached per kernel.
static int resident_blocks(const void *kernel, int block) {
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
    int g = resident_blocks(kern, B);
    if (g <= 0) return SCAN_ERR_HIP;
    if (a.grid_blocks > 0 && uint32_t(g) > a.grid_blocks) g = int(a.grid_blocks);
    if (uint32_t(g) > a.num_tiles) g = int(a.num_tiles);
    hipLaunchKernelGGL((k_lookback<T, Op, B, R, V>), dim3(g), dim3(B), 0, s, a);
    return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
}

// Instantiated (block, rows) shapes.  Every type gets the default shape and a
// one-row shape (small tiles, used to force many tiles at small n); fp32 sum
// also gets the shapes the tuning sweep visits.
template <class T, class Op, int V>
static LbLaunch pick_shape(int block, int rows) {
#define SW64_SHAPE(B, R) \
    if (block == B && rows == R) return &launch_lookback_impl<T, Op, B, R, V>;
    SW64_SHAPE(256, 1)
    SW64_SHAPE(256, 8)
    if constexpr (std::is_same_v<T, float> && std::is_same_v<Op, OpSum>) {
        SW64_SHAPE(256, 2)
        SW64_SHAPE(256, 4)
        SW64_SHAPE(256, 16)
        SW64_SHAPE(512, 2)
        SW64_SHAPE(512, 4)
        SW64_SHAPE(512, 8)
        SW64_SHAPE(1024, 2)
        SW64_SHAPE(1024, 4)
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
