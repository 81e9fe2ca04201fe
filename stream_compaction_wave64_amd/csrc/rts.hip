// rts.hip -- reduce-then-scan, the measured comparison path (The CUDA
// Handbook ch. 13 section 13.3.3 with Merrill's fixed number of partials;
// Merry, "Prefix sums on GPUs", slides "Reduce-then-Scan strategy", "Fixed
// Block Count" and "Prefix-Summing a Block").
//
// Three launches: (1) C workgroups each reduce a chunk of consecutive tiles
// into one partial; (2) one workgroup scans the C partials into exclusive
// bases; (3) the same C workgroups rescan their chunks tile by tile,
// carrying the base from tile to tile.  HBM traffic is 3n (two reads, one
// write) against the look-back's 2n; on MI355X the second read of a chunk
// can hit the 256 MB Infinity Cache when the array is small.
//
// Compiled once per element type (SW64_DT), like lookback.hip.
#include "launch.hpp"
#include "tile.hpp"

namespace sw64 {

template <class T, class Op, int B, int R, int V>
__global__ __launch_bounds__(B) void k_rts_reduce(RtsArgs a) {
    using TS = TileScan<T, Op, B, R, V>;
    using C = typename TS::C;
    __shared__ typename TS::Shared sh;
    const uint64_t t0 = uint64_t(blockIdx.x) * a.chunk_tiles;
    const uint64_t t1 = t0 + a.chunk_tiles < a.num_tiles ? t0 + a.chunk_tiles : a.num_tiles;
    C acc = Op::template identity<C>();
    TS ts;
    for (uint64_t t = t0; t < t1; t++) {
        const int64_t start = int64_t(t) * TS::TILE;
        // plain (temporal) loads, unlike TileScan::load: the rescan reads the
        // chunk again and may find part of it in the caches
        const T *src = reinterpret_cast<const T *>(a.in) + start;
        ts.rem = a.n - start;
#pragma unroll
        for (int r = 0; r < R; r++) {
            const int64_t e = TS::elem(r);
            ts.v[r] = *reinterpret_cast<const Vec<T, V> *>(src + (e < ts.rem ? e : 0));
        }
        ts.reduce(sh);
        acc = Op::apply(acc, C(ts.agg));
        __syncthreads();
    }
    if (threadIdx.x == 0) reinterpret_cast<C *>(a.partials)[blockIdx.x] = acc;
}

// One workgroup of 256 threads: thread k owns a run of consecutive partials,
// reduces it, the 256 run totals are scanned (wave scan + one LDS slot per
// wave), and each thread rewrites its run as exclusive bases.
template <class C, class Op>
__global__ __launch_bounds__(256) void k_rts_partials(C *partials, uint32_t count) {
    __shared__ C wt[4];
    const C id = Op::template identity<C>();
    const uint32_t per = (count + 255) / 256;
    const uint32_t b = threadIdx.x * per, e = b + per < count ? b + per : count;
    C local = id;
    for (uint32_t i = b; i < e; i++) local = Op::apply(local, partials[i]);
    const C inc = wave_scan_incl<Op>(local);
    const int wave = threadIdx.x / kWave;
    if (lane_id() == kWave - 1) wt[wave] = inc;
    __syncthreads();
    C base = id;
    for (int w = 0; w < wave; w++) base = Op::apply(base, wt[w]);
    C run = Op::apply(base, wave_shr1(id, inc));
    for (uint32_t i = b; i < e; i++) {
        const C v = partials[i];
        partials[i] = run;
        run = Op::apply(run, v);
    }
}

template <class T, class Op, int B, int R, int V>
__global__ __launch_bounds__(B) void k_rts_rescan(RtsArgs a) {
    using TS = TileScan<T, Op, B, R, V>;
    using C = typename TS::C;
    __shared__ typename TS::Shared sh;
    __shared__ C s_base;
    C *partials = reinterpret_cast<C *>(a.partials);
    // For arrays larger than the caches, chunks in reverse: workgroups start
    // in index order, so the first ones take the chunks the reduce pass read
    // last, the likeliest still cached.  Workgroup b runs on XCD b mod 8
    // (round-robin dispatch), so the reversal keeps b mod 8: each chunk is
    // rescanned on the XCD whose L2 read it.  The last G mod 8 workgroups
    // keep their own chunks.  (Arrays that fit measured fastest in the
    // reduce pass's own order.)
    const uint32_t b = blockIdx.x, full = a.blocks & ~7u;
    const uint32_t chunk = a.reverse && b < full ? full - 8u - (b & ~7u) + (b & 7u) : b;
    if (threadIdx.x == 0) s_base = partials[chunk];
    __syncthreads();
    C base = s_base;
    if (threadIdx.x == 0) partials[chunk] = C{};  // leave the workspace zeroed
    const uint64_t t0 = uint64_t(chunk) * a.chunk_tiles;
    const uint64_t t1 = t0 + a.chunk_tiles < a.num_tiles ? t0 + a.chunk_tiles : a.num_tiles;
    TS ts;
    for (uint64_t t = t0; t < t1; t++) {
        const int64_t start = int64_t(t) * TS::TILE;
        ts.load(reinterpret_cast<const T *>(a.in) + start, a.n - start);
        ts.scan(sh);
        ts.store(reinterpret_cast<T *>(a.out) + start, a.n - start, base, a.exclusive != 0);
        base = Op::apply(base, C(ts.agg));
        __syncthreads();
    }
}

template <class T, class Op, int B, int R, int V>
static int launch_rts_impl(const RtsArgs &a, hipStream_t s) {
    using C = typename Carry<T, Op>::type;
    hipLaunchKernelGGL((k_rts_reduce<T, Op, B, R, V>), dim3(a.blocks), dim3(B), 0, s, a);
    if (hipGetLastError() != hipSuccess) return SCAN_ERR_HIP;
    hipLaunchKernelGGL((k_rts_partials<C, Op>), dim3(1), dim3(256), 0, s, reinterpret_cast<C *>(a.partials),
                       a.blocks);
    if (hipGetLastError() != hipSuccess) return SCAN_ERR_HIP;
    hipLaunchKernelGGL((k_rts_rescan<T, Op, B, R, V>), dim3(a.blocks), dim3(B), 0, s, a);
    return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
}

template <class T, class Op, int V>
static RtsLaunch pick_rts_shape(int block, int rows) {
    if (block == 256 && rows == 1) return &launch_rts_impl<T, Op, 256, 1, V>;
    if constexpr (sizeof(T) == 4) {
        if (block == 512 && rows == 8) return &launch_rts_impl<T, Op, 512, 8, V>;
    } else {
        if (block == 512 && rows == 4) return &launch_rts_impl<T, Op, 512, 4, V>;
    }
    return nullptr;
}

template <class T, class Op>
static RtsLaunch pick_rts_vec(int block, int rows, int vec) {
    constexpr int VMAX = 16 / int(sizeof(T));
    if (vec == VMAX) return pick_rts_shape<T, Op, VMAX>(block, rows);
    if (vec == 1) return pick_rts_shape<T, Op, 1>(block, rows);
    return nullptr;
}

template <class T>
static RtsLaunch pick_rts_op(scan_op_t op, int block, int rows, int vec) {
    switch (op) {
    case SCAN_OP_SUM: return pick_rts_vec<T, OpSum>(block, rows, vec);
    case SCAN_OP_PROD: return pick_rts_vec<T, OpProd>(block, rows, vec);
    case SCAN_OP_MAX: return pick_rts_vec<T, OpMax>(block, rows, vec);
    case SCAN_OP_MIN: return pick_rts_vec<T, OpMin>(block, rows, vec);
    }
    return nullptr;
}

#if SW64_DT == 0
RtsLaunch find_rts_i32(scan_op_t op, int b, int r, int v) { return pick_rts_op<int32_t>(op, b, r, v); }
#elif SW64_DT == 1
RtsLaunch find_rts_u32(scan_op_t op, int b, int r, int v) { return pick_rts_op<uint32_t>(op, b, r, v); }
#elif SW64_DT == 2
RtsLaunch find_rts_i64(scan_op_t op, int b, int r, int v) { return pick_rts_op<int64_t>(op, b, r, v); }
#elif SW64_DT == 3
RtsLaunch find_rts_f32(scan_op_t op, int b, int r, int v) { return pick_rts_op<float>(op, b, r, v); }
#elif SW64_DT == 4
RtsLaunch find_rts_f64(scan_op_t op, int b, int r, int v) { return pick_rts_op<double>(op, b, r, v); }
#else
#error "SW64_DT must select an element type (0..4)"
#endif

}  // namespace sw64
