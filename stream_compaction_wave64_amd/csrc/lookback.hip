// lookback.hip -- single-pass decoupled look-back scan of scalar elements
// (The CUDA Handbook ch. 13, decoupled look-back section with Figure 13-11,
// and section 13.3.5's items-per-thread kernel), segmented so the same
// kernel scans a whole array (one segment), every row of an (outer, len, 1)
// array, or the counts of count-scan-emit (with the total written after).
//
// The tile policy: 128-bit nontemporal loads, the register tile scan of
// tile.hpp, the prefix added in the carry type, 128-bit stores.  Ordering,
// descriptors and the look-back are the persistent pipeline's
// (pipeline.hpp).
//
// This file is compiled once per element type (SW64_DT selects it) so the
// instantiations build in parallel.
#include "launch.hpp"
#include "tile.hpp"

namespace sw64 {

// OUT_AUX: the output stores' cache policy: nontemporal (2) for scans;
// the default (0) for count-scan-emit's offsets, which the emit kernel reads
// next and may then find in the caches.
template <class T_, class Op_, int BLOCK_, int ROWS, int VEC, int OUT_AUX = 2>
struct ScanPolicy {
    using T = T_;
    using Op = Op_;
    using C = typename Carry<T, Op>::type;
    using D = DescFor<T, C>;
    static constexpr int kDescWords = D::kWords;
    static constexpr int BLOCK = BLOCK_;
    using TS = TileScan<T, Op, BLOCK, ROWS, VEC>;
    using Args = ScanArgs;
    using Shared = typename TS::Shared;

    __device__ __forceinline__ static C aggregate(const Shared &sh) { return TS::template aggregate_from<C>(sh); }

    // A scanned tile waiting for its prefix: every thread's fold()ed rows.
    struct Stash {
        Vec<T, VEC> v[ROWS][BLOCK];
    };

    __device__ __forceinline__ static void geom(const Args &a, uint32_t tile, int64_t &start, int64_t &remaining,
                                                uint32_t &seg, uint32_t &j) {
        seg = tile / a.pipe.tiles_per_seg;
        j = tile - seg * a.pipe.tiles_per_seg;
        start = uniform(int64_t(seg) * a.seg_len + int64_t(j) * TS::TILE);
        remaining = uniform(a.seg_len - int64_t(j) * TS::TILE);
    }

    // Store the stashed tile with its prefix.  An invalid call stores
    // nothing (its buffer resource has no range) but issues the same
    // instructions.
    static constexpr bool kSetup = false;
    __device__ __forceinline__ static C setup(const Args &, const uint64_t *, uint32_t, WsHeader *) { return C{}; }

    __device__ __forceinline__ static void emit(const Stash &st, const Args &a, uint32_t tile, C pre, bool valid,
                                                C) {
        int64_t start, remaining;
        uint32_t seg, j;
        geom(a, tile, start, remaining, seg, j);
        Vec<T, VEC> w[ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; r++) w[r] = st.v[r][threadIdx.x];
        TS::template store_folded<OUT_AUX>(w, reinterpret_cast<T *>(a.out) + (valid ? start : 0),
                                           valid ? remaining : 0, pre);
    }

    // The segment total after its last tile (count-scan-emit's offsets[n]).
    __device__ __forceinline__ static void on_resolved(const Args &a, uint32_t tile, C pre, C agg) {
        int64_t start, remaining;
        uint32_t seg, j;
        geom(a, tile, start, remaining, seg, j);
        if (a.total_out != nullptr && j == a.pipe.tiles_per_seg - 1)
            reinterpret_cast<T *>(a.total_out)[seg] = T(Op::apply(pre, agg));
    }

    struct Tile {
        TS ts;

        // A tile past the end (the pipeline's prefetch beyond the last tile)
        // loads the array's first vector in every row and is never scanned.
        __device__ __forceinline__ void load(const Args &a, uint32_t tile) {
            int64_t start, remaining;
            uint32_t seg, j;
            geom(a, tile, start, remaining, seg, j);
            const bool valid = tile < a.pipe.num_tiles;
            ts.load(reinterpret_cast<const T *>(a.in) + (valid ? start : 0), valid ? remaining : 0);
        }

        __device__ __forceinline__ void scan(Shared &sh) { ts.scan(sh); }

        __device__ __forceinline__ void stash(Stash &st, const Args &a) {
            ts.fold(a.exclusive != 0);
#pragma unroll
            for (int r = 0; r < ROWS; r++) st.v[r][threadIdx.x] = ts.v[r];
        }
    };
};

template <class P>
__global__ __launch_bounds__(CtrlPipeline<P>::THREADS) void k_lookback(typename P::Args a) {
    CtrlPipeline<P>::run(a);
}

// B threads per workgroup: B - 64 data threads and the control wave.
template <class T, class Op, int B, int R, int V, int OUT_AUX = 2>
static int launch_lookback_impl(const ScanArgs &a, uint32_t grid_cap, hipStream_t s) {
    using P = ScanPolicy<T, Op, B - kWave, R, V, OUT_AUX>;
    static_assert(CtrlPipeline<P>::THREADS == B, "launch size");
    const int g = pipeline_grid(reinterpret_cast<const void *>(&k_lookback<P>), B, a.pipe.num_tiles, grid_cap);
    if (g <= 0) return SCAN_ERR_HIP;
    hipLaunchKernelGGL((k_lookback<P>), dim3(g), dim3(B), 0, s, a);
    return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
}

// Instantiated (block, rows) shapes, block counting the control wave.
// Every type gets a default shape -- 768 threads (704 data threads) x 7 rows
// of 128-bit vectors for 4-byte elements (77 KiB per tile), 512 threads (448)
// x 8 rows for 8-byte elements (56 KiB): tiles whose two LDS stashes fit the
// 160 KiB of LDS, measured fastest on MI355X -- and a one-row shape (small
// tiles, used to force many tiles at small n), and 512-thread shapes of 1,
// 2, 3 and 5 rows, which the planner picks so that one tile holds a whole
// short segment.  fp32 sum also gets the shapes the tuning sweep visits.
template <class T, class Op, int V>
static LbLaunch pick_shape(int block, int rows) {
#define SW64_SHAPE(B, R) \
    if (block == B && rows == R) return &launch_lookback_impl<T, Op, B, R, V>;
    SW64_SHAPE(256, 1)
    SW64_SHAPE(512, 1)
    SW64_SHAPE(512, 2)
    SW64_SHAPE(512, 3)
    SW64_SHAPE(512, 5)
    if constexpr (sizeof(T) == 4) {
        SW64_SHAPE(768, 7)
    } else {
        SW64_SHAPE(512, 8)
    }
    if constexpr (std::is_same_v<T, float> && std::is_same_v<Op, OpSum>) {
        SW64_SHAPE(256, 2)
        SW64_SHAPE(256, 4)
        SW64_SHAPE(256, 8)
        SW64_SHAPE(512, 4)
        SW64_SHAPE(512, 8)
        SW64_SHAPE(512, 10)
        SW64_SHAPE(1024, 2)
        SW64_SHAPE(768, 6)
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
// count-scan-emit's offsets (int32 sums) in the default and small-array
// shapes, stored with the default cache policy so that the emit kernel finds
// them in the caches; other shapes use the scan's launchers
LbLaunch find_pack_lookback(int b, int r, int v) {
    if (b == 768 && r == 7 && v == 4) return &launch_lookback_impl<int32_t, OpSum, 768, 7, 4, 0>;
    if (b == 512 && r == 5 && v == 4) return &launch_lookback_impl<int32_t, OpSum, 512, 5, 4, 0>;
    return pick_op<int32_t>(SCAN_OP_SUM, b, r, v);
}
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
