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

// ------------------------------------------------------------ single pass
// Wide inner extents in one pass, reading and writing the array once.  A
// 1024-thread workgroup holds a tile of kColTileRows rows x (64 x V) columns
// in registers: wave w owns rows w * 16 .. w * 16 + 15 of the tile, lane l
// owns V adjacent columns, so each row is one coalesced 128-bit access per
// lane.  The tile is scanned down its columns (each thread over its 16 rows,
// then one thread per column over the 16 waves' totals in LDS), publishes
// its column aggregates (state A, one descriptor word per column and carry
// word) and adds the aggregates of every tile above it in its strip, read by
// the same thread per column, so no tile waits for another's prefix (The
// CUDA Handbook ch. 13, decoupled look-back section: tiles publish
// aggregates, successors combine them; here every predecessor's aggregate
// is read, there being at most kColSingleMaxRowBlocks - 1).  A tile's
// outputs are then written with one rounding per element.
//
// Tile t is (outer slice, row block, strip) in row-block-major order, so the
// tiles above a tile have smaller indices.  The grid is one workgroup per
// tile (the planner keeps the tiles within one per compute unit).  Tile t
// belongs to workgroup t when the residency check confirms the whole grid
// is resident (static mode, as in pipeline.hpp); otherwise tiles are
// claimed in order from the workspace's counter, so a tile only waits for
// tiles already claimed by running workgroups.  The static tile's loads are
// issued before the decision.  Measured on MI355X, 4096 x 4096 fp32, one
// call after the caches were cleared by a read: 30 us, against 43.5 us for
// the three-launch reduce-then-scan and 24.8 us for a plain 64 MiB copy.
template <class T, class Op, int V>
__global__ __launch_bounds__(kColTileWaves *kWave) void k_col_single(ColSingleArgs a) {
    using C = typename Carry<T, Op>::type;
    using D = DescFor<T, C>;
    constexpr int TC = kWave * V;                // columns per strip
    constexpr int RPT = kColTileRowsPerThread;   // rows per thread
    __shared__ C tot[kColTileWaves][TC];         // per wave: column totals of its rows
    __shared__ C above[TC];                      // per column: the tiles above combined
    __shared__ uint32_t s_epoch, s_mode, s_tile;
    __shared__ uint64_t s_hw, s_cap;
    WsHeader *hdr = reinterpret_cast<WsHeader *>(a.pipe.ws);
    uint64_t *desc = reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(a.pipe.ws) + kWsHeaderBytes);
    const int lane = lane_id();
    const uint32_t wr = uniform(uint32_t(threadIdx.x / kWave));
    const uint32_t n = a.pipe.num_tiles;
    const C id = Op::template identity<C>();
    const T *in = reinterpret_cast<const T *>(a.in);

    auto geom = [&](uint32_t t, uint32_t &o, uint32_t &rb, uint32_t &cs) {
        cs = t % a.strips;
        const uint32_t rest = t / a.strips;
        rb = rest % a.rblocks;
        o = rest / a.rblocks;
    };
    // Buffer accesses from the tile's first element: lane offset in a vector
    // register, row step in a scalar one.  The range ends with the outer
    // slice, so rows past len read 0 and drop their stores; lanes past inner
    // get an offset beyond any range (no wrap: the planner keeps a tile's
    // rows under 2^31 bytes).
    static_assert(V * sizeof(T) == 16, "128-bit rows");
    Vec<T, V> x[RPT];
    uint32_t voff = 0, row_bytes = uniform(uint32_t(a.inner * int64_t(sizeof(T))));
    BufRsrc rs_in, rs_out;
    auto place = [&](uint32_t t) {
        uint32_t o, rb, cs;
        geom(t, o, rb, cs);
        const int64_t start = int64_t(o) * a.len * a.inner + int64_t(rb) * kColTileRows * a.inner + int64_t(cs) * TC;
        const int64_t count = (a.len - int64_t(rb) * kColTileRows) * a.inner - int64_t(cs) * TC;
        rs_in = make_rsrc(in + start, count);
        rs_out = make_rsrc(reinterpret_cast<T *>(a.out) + start, count);
        const bool col_ok = int64_t(cs) * TC + lane * V < a.inner;
        voff = col_ok ? uint32_t((int64_t(wr) * RPT * a.inner + lane * V) * int64_t(sizeof(T))) : 0x80000000u;
    };
    auto load = [&](uint32_t t) {
        place(t);
#pragma unroll
        for (int i = 0; i < RPT; i++)
            x[i] = __builtin_bit_cast(Vec<T, V>, __builtin_amdgcn_raw_buffer_load_b128(rs_in, voff, i * row_bytes, 2));
    };
    // Wave 0 runs the workspace protocol before it issues any tile load: a
    // wave's memory counter retires in issue order, so the protocol's reads
    // behind 16 tile rows waited for them (the mode was known only after
    // 15-20 us for 4096 x 4096).  It then loads the tile it was given; the
    // other waves load the static order's tile at once and load again after
    // the barrier if a dynamic-mode claim gave the workgroup another one
    // (one load site, so the tile's registers are allocated once).
    uint32_t tile = blockIdx.x;
    if (wr == 0) {
        uint32_t tk = 0;
        if (lane == 0) {
            uint64_t hw = 0, cap = 0;
            const uint32_t e = begin_call(hdr, hw, cap);
            s_epoch = e;
            s_hw = hw;
            s_cap = cap;
            const uint32_t m = decide_mode(hdr, e, gridDim.x, a.pipe.mode_limit);
            s_mode = m;
            tk = m == kModeStatic
                     ? uint32_t(blockIdx.x)
                     : __hip_atomic_fetch_add(&hdr->claim, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_tile = tk;
        }
        tile = uint32_t(__builtin_amdgcn_readlane(int(tk), 0));
    }
    for (uint32_t pass = 0;; pass++) {
        load(tile);
        if (pass > 0) break;
        __syncthreads();
        if (s_tile == tile) break;
        tile = s_tile;
    }
    const uint32_t epoch = s_epoch;

    uint32_t o, rb, cs;
    geom(tile, o, rb, cs);
    const int64_t row0 = int64_t(rb) * kColTileRows + int64_t(wr) * RPT;
    // this thread's column totals over its rows (rows past the end excluded)
    C t[V];
#pragma unroll
    for (int v = 0; v < V; v++) t[v] = id;
#pragma unroll
    for (int i = 0; i < RPT; i++) {
        if (row0 + i < a.len) {
#pragma unroll
            for (int v = 0; v < V; v++) t[v] = Op::apply(t[v], C(x[i].v[v]));
        }
    }
#pragma unroll
    for (int v = 0; v < V; v++) tot[wr][lane * V + v] = t[v];
    // The outputs convert the tile's values to the carry type again: an
    // empty register barrier keeps the compiler from holding all RPT x V
    // converted values (twice the registers for fp32 in fp64) across the
    // look-back, which spilled.
#pragma unroll
    for (int i = 0; i < RPT; i++) {
#pragma unroll
        for (int v = 0; v < V; v++) asm volatile("" : "+v"(x[i].v[v]));
    }
    __syncthreads();
    // Column pass, one thread per column (the first TC threads; lanes hold
    // adjacent columns, so every descriptor access is coalesced): the 16
    // waves' totals scanned in place (tot[w][c] becomes the combination of
    // waves 0 .. w - 1), the tile's column aggregate published, then the
    // aggregates of the tiles above combined in row-block order.  (One wave
    // reducing all TC columns from LDS, and every thread combining 16
    // per-wave look-back pieces, cost about 1.7 us of LDS latency per tile.)
    if (threadIdx.x < uint32_t(TC)) {
        const uint32_t c = threadIdx.x;
        C acc = id;
#pragma unroll 4
        for (int w = 0; w < kColTileWaves; w++) {
            const C v = tot[w][c];
            tot[w][c] = acc;
            acc = Op::apply(acc, v);
        }
        D::publish(desc + (uint64_t(tile) * TC + c) * D::kWords, epoch, kStateA, acc);
        // First wait on one word per tile above (lane l: row block l; the
        // planner keeps rb below 64): the last column's last word.  Reading
        // every column of every unfinished tile on each poll loaded the
        // memory system so much that a publish took 5-7 us to be seen
        // instead of about 0.6.  The word is only a hint: every word is still
        // checked below.
        const uint32_t base = o * a.rblocks;
        bool seen = uint32_t(lane) >= rb;
        const uint64_t *hint = desc + (uint64_t((base + uint32_t(lane)) * a.strips + cs) * TC + TC - 1) * D::kWords +
                               (D::kWords - 1);
        for (uint32_t polls = 0; __ballot(!seen) != 0ull && polls < a.pipe.spin_limit; polls++) {
            if (!seen) seen = desc_state(__hip_atomic_load(hint, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), epoch) != 0u;
            if (__ballot(!seen) != 0ull) __builtin_amdgcn_s_sleep(1);
        }
        // then this column's word of every tile above, kBatch reads in
        // flight; a word not yet visible is re-read (bounded: after
        // spin_limit polls the error word is flagged and it counts as the
        // identity)
        constexpr uint32_t kBatch = D::kWords >= 4 ? 1u : 4u / D::kWords;  // more spilled registers
        acc = id;
        for (uint32_t p0 = 0; p0 < rb; p0 += kBatch) {
            uint64_t w[kBatch][D::kWords];
#pragma unroll
            for (uint32_t k = 0; k < kBatch; k++) {
                if (p0 + k < rb) D::fetch(desc + (uint64_t((base + p0 + k) * a.strips + cs) * TC + c) * D::kWords, w[k]);
            }
#pragma unroll
            for (uint32_t k = 0; k < kBatch; k++) {
                if (p0 + k < rb) {
                    const uint64_t *pd = desc + (uint64_t((base + p0 + k) * a.strips + cs) * TC + c) * D::kWords;
                    C v;
                    for (uint32_t polls = 0; D::decode(w[k], epoch, v) == 0u; polls++) {
                        if (polls >= a.pipe.spin_limit) {
                            flag_error(hdr, kErrSpin);
                            v = id;
                            break;
                        }
                        __builtin_amdgcn_s_sleep(1);
                        D::fetch(pd, w[k]);
                    }
                    acc = Op::apply(acc, v);
                }
            }
        }
        above[c] = acc;
    }
    __syncthreads();
    // prefix of this thread's first row: the tiles above, then the waves
    // above in the tile; then one output per row
    C run[V];
#pragma unroll
    for (int v = 0; v < V; v++) run[v] = Op::apply(above[lane * V + v], tot[wr][lane * V + v]);
#pragma unroll
    for (int i = 0; i < RPT; i++) {
        Vec<T, V> y;
#pragma unroll
        for (int v = 0; v < V; v++) {
            const C next = Op::apply(run[v], C(x[i].v[v]));
            y.v[v] = T(a.exclusive ? run[v] : next);
            run[v] = next;
        }
        // The row step goes into the vector offset, the scalar offset stays a
        // constant 0: 128-bit buffer stores with a scalar-register offset
        // had their data registers overwritten by the next instruction before
        // the store read them (measured: lanes 12-15 of every 16, rows 1-15;
        // the compiler inserted no wait state on gfx950).  The empty asm keeps
        // the sum out of the scalar operand.
        uint32_t vo = voff + uint32_t(i) * row_bytes;
        asm volatile("" : "+v"(vo));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, y), rs_out, vo, 0, 2);
    }
    // end of the call: in static mode every workgroup was counted before the
    // decision; in dynamic mode the holder of the last ticket claimed last
    if (tile == n - 1) end_call(hdr, epoch, s_hw, s_cap, a.pipe.words_used, a.pipe.ws_words, desc);
}

template <class T, class Op>
static int launch_col_single_impl(const ColSingleArgs &a, hipStream_t s) {
    constexpr int V = 16 / int(sizeof(T));
    hipLaunchKernelGGL((k_col_single<T, Op, V>), dim3(a.pipe.num_tiles), dim3(kColTileWaves * kWave), 0, s, a);
    return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
}

template <class T>
static ColSingleLaunch pick_col_single(scan_op_t op) {
    switch (op) {
    case SCAN_OP_SUM: return &launch_col_single_impl<T, OpSum>;
    case SCAN_OP_PROD: return &launch_col_single_impl<T, OpProd>;
    case SCAN_OP_MAX: return &launch_col_single_impl<T, OpMax>;
    case SCAN_OP_MIN: return &launch_col_single_impl<T, OpMin>;
    }
    return nullptr;
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
ColSingleLaunch find_columns_single_i32(scan_op_t op) { return pick_col_single<int32_t>(op); }
#elif SW64_DT == 1
ColLaunch find_columns_u32(scan_op_t op, int v) { return pick_col_op<uint32_t>(op, v); }
ColSingleLaunch find_columns_single_u32(scan_op_t op) { return pick_col_single<uint32_t>(op); }
#elif SW64_DT == 2
ColLaunch find_columns_i64(scan_op_t op, int v) { return pick_col_op<int64_t>(op, v); }
ColSingleLaunch find_columns_single_i64(scan_op_t op) { return pick_col_single<int64_t>(op); }
#elif SW64_DT == 3
ColLaunch find_columns_f32(scan_op_t op, int v) { return pick_col_op<float>(op, v); }
ColSingleLaunch find_columns_single_f32(scan_op_t op) { return pick_col_single<float>(op); }
#elif SW64_DT == 4
ColLaunch find_columns_f64(scan_op_t op, int v) { return pick_col_op<double>(op, v); }
ColSingleLaunch find_columns_single_f64(scan_op_t op) { return pick_col_single<double>(op); }
#else
#error "SW64_DT must select an element type (0..4)"
#endif

}  // namespace sw64
