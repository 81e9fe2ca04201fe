// noid.hip -- inclusive scans that never use the operator's identity
// (AcceleratedKernels.jl PR #208, description, first bullet: for operators
// with no neutral element the partial results are "Optional"; its timing
// table has a "no neutral" cumsum row).  The single-pass look-back pipeline
// of lookback.hip, with
//  * the element operator wrapped in NoId, which has apply() and no
//    identity(): a use of the identity anywhere in the tile code does not
//    compile;
//  * the wave scan on DPP row shifts and broadcasts with per-lane
//    predicates: a lane whose source is outside the row keeps its value
//    instead of receiving an identity;
//  * tile offsets with a presence bit (thread 0's first row has nothing
//    before it in the tile);
//  * carries between tiles as Opt<C>, a value and a presence flag, whose
//    only identity is "empty": the first tile of a segment gets an empty
//    prefix, and look-back slots before the segment are empty.  Published
//    aggregates and prefixes always hold a value, so the descriptor words
//    are those of the plain scan.
// Elements past the end of a segment are loaded (as copies of its first
// vector) and scanned but never masked: an inclusive result combines only
// its own and earlier elements, so they reach only results past the end,
// which the bounded stores drop, and the last tile's aggregate, which no
// tile reads.  Exclusive scans are not defined without an identity.
//
// This file is compiled once per element type (SW64_DT selects it).
#include "launch.hpp"
#include "noid.hpp"
#include "tile.hpp"

namespace sw64 {

// The tile of tile.hpp (ROWS rows of BLOCK x VEC elements, thread t holding
// vector r * BLOCK + t of each row), scanned without an identity.
template <class T, class Op0, int BLOCK, int ROWS, int VEC>
struct TileScanNoId {
    using Op = NoId<Op0>;
    static_assert(BLOCK % kWave == 0 && BLOCK <= 1024 && ROWS <= 32, "tile shape");
    static constexpr int W = BLOCK / kWave;
    static constexpr int64_t TILE = int64_t(BLOCK) * ROWS * VEC;

    struct Shared {
        T tot[ROWS][W];
    };

    Vec<T, VEC> v[ROWS];
    T off[ROWS];       // combination of everything before this thread's vector in row r
    uint32_t has_off;  // bit r: off[r] holds a value (not so only for thread 0's first row)

    __device__ __forceinline__ static int64_t elem(int r) {
        return (int64_t(r) * BLOCK + threadIdx.x) * VEC;
    }

    // As TileScan::load: every load unconditional, rows past the end re-read
    // the tile's first vector.
    __device__ __forceinline__ void load(const T *src, int64_t remaining) {
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            const int64_t e = elem(r);
            v[r] = load_vec<T, VEC>(src + (e < remaining ? e : 0));
        }
    }

    // Thread-serial scan of each vector, wave scan of the thread totals, one
    // LDS slot per wave and row; then each thread's row offsets from the
    // slots.  Contains one __syncthreads().
    __device__ __forceinline__ void scan(Shared &sh) {
        const int lane = lane_id();
        const int wave = threadIdx.x / kWave;
        T winc[ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            T acc = v[r].v[0];
#pragma unroll
            for (int c = 1; c < VEC; c++) {
                acc = Op::apply(acc, v[r].v[c]);
                v[r].v[c] = acc;
            }
            winc[r] = wave_scan_incl_noid<Op>(acc);
        }
        if (lane == kWave - 1) {
#pragma unroll
            for (int r = 0; r < ROWS; r++) sh.tot[r][wave] = winc[r];
        }
        __syncthreads();
        T run = sh.tot[0][0];  // rows before r (present from r = 1 on)
        has_off = 0;
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            T wb = sh.tot[r][0];  // waves before this one in row r (present when wave > 0)
#pragma unroll
            for (int w = 1; w < W; w++) {
                if (w < wave) wb = Op::apply(wb, sh.tot[r][w]);
            }
            // lanes before this one: lane - 1's inclusive value (lane 0: none)
            T o = dpp_mov<kWaveShr1>(winc[r], winc[r]);
            bool present = lane > 0;
            if (wave > 0) {
                o = present ? Op::apply(wb, o) : wb;
                present = true;
            }
            if (r > 0) {
                o = present ? Op::apply(run, o) : run;
                present = true;
            }
            off[r] = o;
            has_off |= uint32_t(present) << r;
            T row = sh.tot[r][0];
#pragma unroll
            for (int w = 1; w < W; w++) row = Op::apply(row, sh.tot[r][w]);
            run = r > 0 ? Op::apply(run, row) : row;
        }
    }

    // The tile aggregate (present) in the carry type, from the slots scan()
    // left in LDS, by any one whole wave after scan()'s barrier.
    template <class C0>
    __device__ __forceinline__ static Opt<C0> aggregate(const Shared &sh) {
        using X = Opt<C0>;
        X acc = OptOp<Op0>::template identity<X>();
        for (int i = lane_id(); i < ROWS * W; i += kWave)
            acc = OptOp<Op0>::apply(acc, X{C0(sh.tot[i / W][i % W]), 1});
        return wave_reduce<OptOp<Op0>>(acc);
    }

    // After scan(): every value replaced by its tile-local inclusive result.
    __device__ __forceinline__ void fold() {
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            if (has_off & (1u << r)) {
#pragma unroll
                for (int c = 0; c < VEC; c++) v[r].v[c] = Op::apply(off[r], v[r].v[c]);
            }
        }
    }

    // Store fold()ed values with the tile's prefix applied when present (in
    // the carry type, rounded once).  Rows at or past `remaining` are dropped.
    template <class C0>
    __device__ __forceinline__ static void store_folded(const Vec<T, VEC> (&w)[ROWS], T *dst, int64_t remaining,
                                                        Opt<C0> pre) {
        const BufRsrc rs = make_rsrc(dst, remaining < TILE ? (remaining > 0 ? remaining : 0) : TILE);
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            Vec<T, VEC> o;
#pragma unroll
            for (int c = 0; c < VEC; c++) o.v[c] = pre.has ? T(Op::apply(pre.v, C0(w[r].v[c]))) : w[r].v[c];
            store_vec_bounded<T, VEC>(rs, uint32_t(elem(r) * int64_t(sizeof(T))), o);
        }
    }
};

template <class T_, class Op0, int BLOCK_, int ROWS, int VEC>
struct NoIdScanPolicy {
    using T = T_;
    using C0 = typename Carry<T, Op0>::type;
    using C = Opt<C0>;
    using Op = OptOp<Op0>;
    using D = OptDesc<DescFor<T, C0>>;
    static constexpr int kDescWords = D::kWords;
    static constexpr int BLOCK = BLOCK_;
    using TS = TileScanNoId<T, Op0, BLOCK, ROWS, VEC>;
    using Args = ScanArgs;
    using Shared = typename TS::Shared;

    __device__ __forceinline__ static C aggregate(const Shared &sh) { return TS::template aggregate<C0>(sh); }

    struct Stash {
        Vec<T, VEC> v[ROWS][BLOCK];
    };

    static constexpr bool kSetup = false;
    __device__ __forceinline__ static C setup(const Args &, const uint64_t *, uint32_t, WsHeader *) {
        return Op::template identity<C>();
    }

    __device__ __forceinline__ static void geom(const Args &a, uint32_t tile, int64_t &start, int64_t &remaining) {
        const uint32_t seg = tile / a.pipe.tiles_per_seg;
        const uint32_t j = tile - seg * a.pipe.tiles_per_seg;
        start = uniform(int64_t(seg) * a.seg_len + int64_t(j) * TS::TILE);
        remaining = uniform(a.seg_len - int64_t(j) * TS::TILE);
    }

    __device__ __forceinline__ static void emit(const Stash &st, const Args &a, uint32_t tile, C pre, bool valid,
                                                C) {
        int64_t start, remaining;
        geom(a, tile, start, remaining);
        Vec<T, VEC> w[ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; r++) w[r] = st.v[r][threadIdx.x];
        TS::template store_folded<C0>(w, reinterpret_cast<T *>(a.out) + (valid ? start : 0), valid ? remaining : 0,
                                      pre);
    }

    __device__ __forceinline__ static void on_resolved(const Args &, uint32_t, C, C) {}

    struct Tile {
        TS ts;
        __device__ __forceinline__ void load(const Args &a, uint32_t tile) {
            int64_t start, remaining;
            geom(a, tile, start, remaining);
            const bool valid = tile < a.pipe.num_tiles;
            ts.load(reinterpret_cast<const T *>(a.in) + (valid ? start : 0), valid ? remaining : 0);
        }
        __device__ __forceinline__ void scan(Shared &sh) { ts.scan(sh); }
        __device__ __forceinline__ void stash(Stash &st, const Args &) {
            ts.fold();
#pragma unroll
            for (int r = 0; r < ROWS; r++) st.v[r][threadIdx.x] = ts.v[r];
        }
    };
};

template <class P>
__global__ __launch_bounds__(CtrlPipeline<P>::THREADS) void k_lookback_noid(typename P::Args a) {
    CtrlPipeline<P>::run(a);
}

// B threads per workgroup: B - 64 data threads and the control wave.
template <class T, class Op0, int B, int R, int V>
static int launch_noid_impl(const ScanArgs &a, uint32_t grid_cap, hipStream_t s) {
    using P = NoIdScanPolicy<T, Op0, B - kWave, R, V>;
    static_assert(CtrlPipeline<P>::THREADS == B, "launch size");
    const int g = pipeline_grid(reinterpret_cast<const void *>(&k_lookback_noid<P>), B, a.pipe.num_tiles, grid_cap);
    if (g <= 0) return SCAN_ERR_HIP;
    hipLaunchKernelGGL((k_lookback_noid<P>), dim3(g), dim3(B), 0, s, a);
    return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
}

// The look-back scan's shapes that its planner picks without a tuned shape:
// the default (768 x 7 rows for 4-byte elements, 512 x 8 for 8-byte ones),
// 512 x 5 for small whole arrays, 512 x 1, 2, 3 for short segments, and the
// one-row 256-thread shape (many small tiles).
template <class T, class Op0, int V>
static LbLaunch pick_noid_shape(int block, int rows) {
#define SW64_SHAPE(B, R) \
    if (block == B && rows == R) return &launch_noid_impl<T, Op0, B, R, V>;
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
#undef SW64_SHAPE
    return nullptr;
}

template <class T, class Op0>
static LbLaunch pick_noid_vec(int block, int rows, int vec) {
    constexpr int VMAX = 16 / int(sizeof(T));
    if (vec == VMAX) return pick_noid_shape<T, Op0, VMAX>(block, rows);
    if (vec == 1) return pick_noid_shape<T, Op0, 1>(block, rows);
    return nullptr;
}

template <class T>
static LbLaunch pick_noid(scan_op_t op, int block, int rows, int vec) {
    switch (op) {
    case SCAN_OP_SUM: return pick_noid_vec<T, OpSum>(block, rows, vec);
    case SCAN_OP_PROD: return pick_noid_vec<T, OpProd>(block, rows, vec);
    case SCAN_OP_MAX: return pick_noid_vec<T, OpMax>(block, rows, vec);
    case SCAN_OP_MIN: return pick_noid_vec<T, OpMin>(block, rows, vec);
    }
    return nullptr;
}

#if SW64_DT == 0
LbLaunch find_noid_i32(scan_op_t op, int b, int r, int v) { return pick_noid<int32_t>(op, b, r, v); }
#elif SW64_DT == 1
LbLaunch find_noid_u32(scan_op_t op, int b, int r, int v) { return pick_noid<uint32_t>(op, b, r, v); }
#elif SW64_DT == 2
LbLaunch find_noid_i64(scan_op_t op, int b, int r, int v) { return pick_noid<int64_t>(op, b, r, v); }
#elif SW64_DT == 3
LbLaunch find_noid_f32(scan_op_t op, int b, int r, int v) { return pick_noid<float>(op, b, r, v); }
#elif SW64_DT == 4
LbLaunch find_noid_f64(scan_op_t op, int b, int r, int v) { return pick_noid<double>(op, b, r, v); }
#else
#error "SW64_DT must select an element type (0..4)"
#endif

}  // namespace sw64
