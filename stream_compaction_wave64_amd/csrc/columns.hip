// columns.hip -- scan along the middle axis of an (outer, len, inner) array
// whose inner extent is too wide for one element per thread: every column
// (o, :, k) is an independent scan of stride `inner` (AcceleratedKernels.jl
// PR #208: SliceScan along dims; a 4096 x 4096 row-major matrix scanned down
// its columns is (1, 4096, 4096)).
//
// Reduce-then-scan over row chunks, with threads across columns (The CUDA
// Handbook ch. 13 section 13.3.3; Merry, "Prefix sums on GPUs", slides
// "Reduce-then-Scan strategy" and "Prefix-Summing a Block": each workgroup
// scans its block serially).  A workgroup owns a strip of 256 x VEC columns
// and a chunk of R rows; every thread owns VEC adjacent columns, so each row
// of a strip is one coalesced 128-bit access per thread.
//   1. reduce: each thread folds its columns over the chunk's R rows into one
//      partial per column (carry type);
//   2. partials: for every column, an exclusive scan over the chunks
//      (columns in groups of 16, transposed through LDS);
//   3. rescan: each thread runs down its columns again from the chunk's base
//      and writes the outputs, then zeroes its partials (the workspace's
//      descriptor area must be left zeroed).
// Traffic is two reads and one write of the array; the second read of a
// chunk often hits the 256 MB Infinity Cache when the array is small.
//
// Compiled once per element type (SW64_DT).
#include "launch.hpp"
#include "tile.hpp"

namespace sw64 {

constexpr int kColThreads = 256, kColBatch = 16;

// Workgroup index -> (outer slice, row chunk, column strip).
__device__ __forceinline__ static void col_decode(const ColArgs &a, uint32_t wg, uint32_t &o, uint32_t &c,
                                                  uint32_t &s) {
    s = wg % a.strips;
    const uint32_t rest = wg / a.strips;
    c = rest % a.chunks;
    o = rest / a.chunks;
}

template <class T, class Op, int V>
__global__ __launch_bounds__(kColThreads) void k_col_reduce(ColArgs a) {
    using C = typename Carry<T, Op>::type;
    uint32_t o, c, s;
    col_decode(a, blockIdx.x, o, c, s);
    const int64_t col = (int64_t(s) * kColThreads + threadIdx.x) * V;
    if (col >= a.inner) return;
    const int64_t r0 = int64_t(c) * a.rows, r1 = r0 + a.rows < a.len ? r0 + a.rows : a.len;
    const T *src = reinterpret_cast<const T *>(a.in) + (int64_t(o) * a.len) * a.inner + col;
    C acc[V];
#pragma unroll
    for (int v = 0; v < V; v++) acc[v] = Op::template identity<C>();
    // V > 1 only when inner is a multiple of V with 16-byte aligned rows, so
    // a thread's V columns are one aligned 128-bit access per row.  Rows go
    // in batches of kColBatch whose loads are all issued before the first is
    // folded: the grid is about one workgroup wave, so nothing else hides
    // the round trips.
    int64_t r = r0;
    for (; r + kColBatch <= r1; r += kColBatch) {
        Vec<T, V> x[kColBatch];
#pragma unroll
        for (int i = 0; i < kColBatch; i++) x[i] = *reinterpret_cast<const Vec<T, V> *>(src + (r + i) * a.inner);
#pragma unroll
        for (int i = 0; i < kColBatch; i++)
#pragma unroll
            for (int v = 0; v < V; v++) acc[v] = Op::apply(acc[v], C(x[i].v[v]));
    }
    for (; r < r1; r++) {
        const Vec<T, V> x = *reinterpret_cast<const Vec<T, V> *>(src + r * a.inner);
#pragma unroll
        for (int v = 0; v < V; v++) acc[v] = Op::apply(acc[v], C(x.v[v]));
    }
    C *part = reinterpret_cast<C *>(a.partials) + (int64_t(o) * a.chunks + c) * a.inner + col;
#pragma unroll
    for (int v = 0; v < V; v++) part[v] = acc[v];
}

// Partials: per (outer, column), an exclusive scan over the chunks.  A
// workgroup takes kColGroup adjacent columns of one outer slice: it reads the
// [chunks][kColGroup] block of partials with consecutive lanes on consecutive
// columns (rows of the block are contiguous), scans each column in LDS with
// kColSegs threads per column (each serial over a run of chunks, then the
// run totals combined), and writes the exclusive prefixes back the same way.
// The host keeps chunks <= kColMaxChunks.  Groups of 16 columns (256
// workgroups for 4096 columns) measured 5.1 us against 6.6 us for 32.
constexpr int kColGroup = 16, kColSegs = kColThreads / kColGroup, kColMaxChunks = 256;

template <class T, class Op>
__global__ __launch_bounds__(kColThreads) void k_col_partials(ColArgs a) {
    using C = typename Carry<T, Op>::type;
    __shared__ C blk[kColMaxChunks][kColGroup + 1];  // +1: column-wise walks hit distinct banks
    __shared__ C seg[kColSegs][kColGroup];
    const int64_t groups = (a.inner + kColGroup - 1) / kColGroup;
    const uint32_t o = uint32_t(blockIdx.x / groups);
    const int64_t col0 = int64_t(blockIdx.x % groups) * kColGroup;
    const int ncol = int(a.inner - col0 < kColGroup ? a.inner - col0 : kColGroup);
    const int nch = int(a.chunks);
    const C id = Op::template identity<C>();
    C *part = reinterpret_cast<C *>(a.partials) + int64_t(o) * a.chunks * a.inner + col0;
    // every load of the block issued before any is used (one round trip)
    constexpr int kPer = kColMaxChunks * kColGroup / kColThreads;
    C x[kPer];
#pragma unroll
    for (int it = 0; it < kPer; it++) {
        const int i = it * kColThreads + threadIdx.x, c = i / kColGroup, k = i % kColGroup;
        x[it] = (c < nch && k < ncol) ? part[int64_t(c) * a.inner + k] : id;
    }
#pragma unroll
    for (int it = 0; it < kPer; it++) {
        const int i = it * kColThreads + threadIdx.x;
        if (i < nch * kColGroup) blk[i / kColGroup][i % kColGroup] = x[it];
    }
    __syncthreads();
    const int k = threadIdx.x % kColGroup, sgi = threadIdx.x / kColGroup;
    const int per = (nch + kColSegs - 1) / kColSegs;
    const int c0 = sgi * per, c1 = c0 + per < nch ? c0 + per : nch;
    C run = id;
    for (int c = c0; c < c1; c++) run = Op::apply(run, blk[c][k]);
    seg[sgi][k] = run;
    __syncthreads();
    C ex = id;
    for (int g = 0; g < sgi; g++) ex = Op::apply(ex, seg[g][k]);
    for (int c = c0; c < c1; c++) {
        const C x = blk[c][k];
        blk[c][k] = ex;
        ex = Op::apply(ex, x);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nch * kColGroup; i += kColThreads) {
        const int c = i / kColGroup, kk = i % kColGroup;
        if (kk < ncol) part[int64_t(c) * a.inner + kk] = blk[c][kk];
    }
}

template <class T, class Op, int V>
__global__ __launch_bounds__(kColThreads) void k_col_rescan(ColArgs a) {
    using C = typename Carry<T, Op>::type;
    uint32_t o, c, s;
    col_decode(a, blockIdx.x, o, c, s);
    const int64_t col = (int64_t(s) * kColThreads + threadIdx.x) * V;
    if (col >= a.inner) return;
    const int64_t r0 = int64_t(c) * a.rows, r1 = r0 + a.rows < a.len ? r0 + a.rows : a.len;
    const int64_t base_off = (int64_t(o) * a.len) * a.inner + col;
    const T *src = reinterpret_cast<const T *>(a.in) + base_off;
    T *dst = reinterpret_cast<T *>(a.out) + base_off;
    C *part = reinterpret_cast<C *>(a.partials) + (int64_t(o) * a.chunks + c) * a.inner + col;
    C run[V];
#pragma unroll
    for (int v = 0; v < V; v++) {
        run[v] = part[v];
        part[v] = C{};  // leave the workspace zeroed
    }
#pragma unroll 8
    for (int64_t r = r0; r < r1; r++) {
        const T *p = src + r * a.inner;
        T *q = dst + r * a.inner;
        if constexpr (V > 1) {
            const Vec<T, V> x = *reinterpret_cast<const Vec<T, V> *>(p);
            Vec<T, V> y;
#pragma unroll
            for (int v = 0; v < V; v++) {
                const C next = Op::apply(run[v], C(x.v[v]));
                y.v[v] = T(a.exclusive ? run[v] : next);
                run[v] = next;
            }
            store_vec<T, V>(q, y);
        } else {
            const C next = Op::apply(run[0], C(p[0]));
            store_vec<T, 1>(q, Vec<T, 1>{{T(a.exclusive ? run[0] : next)}});
            run[0] = next;
        }
    }
}

template <class T, class Op, int V>
static int launch_columns_impl(const ColArgs &a, hipStream_t s) {
    const uint32_t wgs = a.outer * a.chunks * a.strips;
    hipLaunchKernelGGL((k_col_reduce<T, Op, V>), dim3(wgs), dim3(kColThreads), 0, s, a);
    if (hipGetLastError() != hipSuccess) return SCAN_ERR_HIP;
    if (a.chunks > uint32_t(kColMaxChunks)) return SCAN_ERR_UNSUPPORTED;
    const int64_t groups = (a.inner + kColGroup - 1) / kColGroup;
    hipLaunchKernelGGL((k_col_partials<T, Op>), dim3(uint32_t(a.outer * groups)), dim3(kColThreads), 0, s, a);
    if (hipGetLastError() != hipSuccess) return SCAN_ERR_HIP;
    hipLaunchKernelGGL((k_col_rescan<T, Op, V>), dim3(wgs), dim3(kColThreads), 0, s, a);
    return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
}

template <class T, class Op>
static ColLaunch pick_col_vec(int vec) {
    constexpr int VMAX = 16 / int(sizeof(T));
    if (vec == VMAX) return &launch_columns_impl<T, Op, VMAX>;
    if (vec == 1) return &launch_columns_impl<T, Op, 1>;
    return nullptr;
}

template <class T>
static ColLaunch pick_col_op(scan_op_t op, int vec) {
    switch (op) {
    case SCAN_OP_SUM: return pick_col_vec<T, OpSum>(vec);
    case SCAN_OP_PROD: return pick_col_vec<T, OpProd>(vec);
    case SCAN_OP_MAX: return pick_col_vec<T, OpMax>(vec);
    case SCAN_OP_MIN: return pick_col_vec<T, OpMin>(vec);
    }
    return nullptr;
}

#if SW64_DT == 0
ColLaunch find_columns_i32(scan_op_t op, int v) { return pick_col_op<int32_t>(op, v); }
#elif SW64_DT == 1
ColLaunch find_columns_u32(scan_op_t op, int v) { return pick_col_op<uint32_t>(op, v); }
#elif SW64_DT == 2
ColLaunch find_columns_i64(scan_op_t op, int v) { return pick_col_op<int64_t>(op, v); }
#elif SW64_DT == 3
ColLaunch find_columns_f32(scan_op_t op, int v) { return pick_col_op<float>(op, v); }
#elif SW64_DT == 4
ColLaunch find_columns_f64(scan_op_t op, int v) { return pick_col_op<double>(op, v); }
#else
#error "SW64_DT must select an element type (0..4)"
#endif

}  // namespace sw64
