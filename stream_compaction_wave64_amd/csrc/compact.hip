// compact.hip -- stream compaction and the emit step of count-scan-emit.
//
// compact_if (Merry, "Prefix sums on GPUs", slide "Other Applications":
// compaction selects the objects that satisfy a predicate; AcceleratedKernels
// PR #208: findall's block scans run on Int32 counts) as one fused pass on
// the persistent look-back pipeline: each tile loads x with 128-bit
// accesses, evaluates the predicate into 0/1 counts held in registers, scans
// the counts (int32, exact), looks back for the number of selected elements
// before the tile, and writes the index of every selected element at its
// position.  No flag or offset array ever reaches HBM: traffic is one read
// of x plus one write per selected index.  The last tile writes the count.
//
// pack_emit_neighbors (same slides, "Solution" step 3): each object writes
// its records from its start offset; record j of object i is (i + 1 + j)
// mod n, a reading of the deliberately open record content.
//
// This file is compiled once per key type (SW64_DT: 0 int32, 1 uint32, 3
// fp32) and per entry point (SW64_PART: 0 compaction and the emit kernel,
// 1 partition), so the instantiations build in parallel.
#include "launch.hpp"
#include "tile.hpp"

namespace sw64 {

// The predicate.  For integer keys the bit predicates test bit t (0..31) of
// the key's 32-bit pattern: a one-bit radix digit.
template <class X, int CMP>
__device__ __forceinline__ bool keep(X v, X t) {
    if constexpr (CMP == SCAN_CMP_GT) return v > t;
    else if constexpr (CMP == SCAN_CMP_GE) return v >= t;
    else if constexpr (CMP == SCAN_CMP_LT) return v < t;
    else if constexpr (CMP == SCAN_CMP_LE) return v <= t;
    else if constexpr (CMP == SCAN_CMP_EQ) return v == t;
    else if constexpr (CMP == SCAN_CMP_NE) return v != t;
    else {
        static_assert(!std::is_floating_point_v<X>, "bit predicates take integer keys");
        const uint32_t bit = (uint32_t(v) >> (uint32_t(t) & 31u)) & 1u;
        return CMP == SCAN_CMP_BIT_SET ? bit != 0u : bit == 0u;
    }
}

// Writes dst[g0 + i] = f(i) for i in [0, len), skipping positions outside
// [0, lim).  The range is cut at dst's 16-byte boundaries: whole quads go
// out as one nontemporal 16-byte store, the partial quads at its two ends
// element by element.  The BLOCK data threads take quads in turn.
template <int BLOCK, class F>
__device__ __forceinline__ void write_range(int32_t *dst, int64_t g0, int32_t len, int64_t lim, F f) {
    typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
    if (len <= 0) return;
    const int32_t lead = int32_t(((reinterpret_cast<uintptr_t>(dst) >> 2) + uint64_t(g0)) & 3u);
    const int64_t a0 = g0 - lead;  // dst + a0 is 16-byte aligned
    const int32_t nq = (lead + len + 3) >> 2;
    const bool inside = g0 >= 0 && g0 + len <= lim;
    for (int32_t q = threadIdx.x; q < nq; q += BLOCK) {
        const int32_t i0 = 4 * q - lead;  // range index of the quad's first element
        int32_t *d = dst + a0 + 4 * q;
        if (inside && i0 >= 0 && i0 + 4 <= len) {
            const i32x4 x = {f(i0), f(i0 + 1), f(i0 + 2), f(i0 + 3)};
            __builtin_nontemporal_store(x, reinterpret_cast<i32x4 *>(d));
        } else {
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const int32_t i = i0 + c;
                const int64_t g = a0 + 4 * q + c;
                if (i >= 0 && i < len && g >= 0 && g < lim) d[c] = f(i);
            }
        }
    }
}

template <class X, int CMP, int BLOCK_, int ROWS, int VEC>
struct CompactPolicy {
    using T = int32_t;
    using Op = OpSum;
    using C = int32_t;
    using D = Desc<C>;
    static constexpr int kDescWords = D::kWords;
    static constexpr int BLOCK = BLOCK_;
    using TS = TileScan<int32_t, OpSum, BLOCK, ROWS, VEC>;
    using Args = CompactArgs;
    using Shared = typename TS::Shared;
    static_assert(ROWS * VEC <= 32, "selection bits fit one word");

    __device__ __forceinline__ static C aggregate(const Shared &sh) { return TS::template aggregate_from<C>(sh); }

    // A scanned tile waiting for its prefix: the tile-local indices of its
    // selected elements in output order, and how many there are.  The emit
    // then writes one contiguous range with whole 16-byte stores instead of
    // 4-byte stores scattered by the selection.
    static_assert(TS::TILE <= 65536, "tile-local indices fit 16 bits");
    struct Stash {
        uint16_t lidx[TS::TILE];
        int32_t nsel;
    };
    static constexpr bool kStagedEmit = true;  // emit reads other threads' slots

    // Each selected element's index at its position.
    static constexpr bool kSetup = false;
    __device__ __forceinline__ static C setup(const Args &, const uint64_t *, uint32_t, WsHeader *) { return C{}; }

    __device__ __forceinline__ static void emit(const Stash &st, const Args &a, uint32_t tile, C pre, bool valid,
                                                C) {
        if (!valid) return;
        const int32_t start = int32_t(int64_t(tile) * TS::TILE);  // n <= INT32_MAX
        write_range<BLOCK>(a.out_idx, int64_t(pre), st.nsel, a.n,
                           [&](int32_t i) { return start + int32_t(st.lidx[i]); });
    }

    // The count after the last tile.
    __device__ __forceinline__ static void on_resolved(const Args &a, uint32_t tile, C pre, C agg) {
        if (tile == a.pipe.num_tiles - 1) *a.count = pre + agg;
    }

    struct Tile {
        TS ts;          // raw element bits after load, 0/1 counts after scan
        uint32_t bits;  // bit r*VEC + c: element c of this thread's vector in row r is selected
        uint32_t thr;   // threshold bits
        int64_t rem;    // elements of the tile in range

        // Issue the loads only (see TileScan::load): the predicate is
        // evaluated in scan(), so pipelined loads stay in flight.  Every
        // load is unconditional: rows past the end re-read the tile's first
        // vector (n is a multiple of VEC), and a tile past the end (the
        // pipeline's prefetch beyond the last tile) reads x's first vector.
        __device__ __forceinline__ void load(const Args &a, uint32_t tile) {
            const bool valid = tile < a.pipe.num_tiles;
            const int64_t start = valid ? int64_t(tile) * TS::TILE : 0;
            rem = valid ? uniform(a.n - start) : 0;
            thr = a.threshold;
            const int32_t *x = reinterpret_cast<const int32_t *>(a.x) + uniform(start);
#pragma unroll
            for (int r = 0; r < ROWS; r++) {
                const int64_t e = TS::elem(r);
                ts.v[r] = load_vec<int32_t, VEC>(x + (e < rem ? e : 0));
            }
        }

        __device__ __forceinline__ void scan(Shared &sh) {
            const X t = __builtin_bit_cast(X, thr);
            bits = 0;
#pragma unroll
            for (int r = 0; r < ROWS; r++) {
                const int64_t e = TS::elem(r);
#pragma unroll
                for (int c = 0; c < VEC; c++) {
                    const bool k = (e + c < rem) && keep<X, CMP>(__builtin_bit_cast(X, ts.v[r].v[c]), t);
                    ts.v[r].v[c] = k ? 1 : 0;
                    bits |= uint32_t(k) << (r * VEC + c);
                }
            }
            ts.rem = TS::TILE;  // counts past the end are already 0
            ts.scan(sh);
        }

        __device__ __forceinline__ void stash(Stash &st, const Args &) const {
#pragma unroll
            for (int r = 0; r < ROWS; r++) {
                int32_t pos = ts.off[r];
#pragma unroll
                for (int c = 0; c < VEC; c++) {
                    if (bits & (1u << (r * VEC + c))) {
                        st.lidx[pos] = uint16_t(TS::elem(r) + c);
                        pos++;
                    }
                }
            }
            if (threadIdx.x == 0) st.nsel = ts.agg;
        }
    };
};

template <class P>
__global__ __launch_bounds__(CtrlPipeline<P>::THREADS) void k_compact(typename P::Args a) {
    CtrlPipeline<P>::run(a);
}

// B threads per workgroup: B - 64 data threads and the control wave.
template <class X, int CMP, int B, int R, int V>
static int launch_compact_impl(const CompactArgs &a, uint32_t grid_cap, hipStream_t s) {
    using P = CompactPolicy<X, CMP, B - kWave, R, V>;
    const int g = pipeline_grid(reinterpret_cast<const void *>(&k_compact<P>), B, a.pipe.num_tiles, grid_cap);
    if (g <= 0) return SCAN_ERR_HIP;
    hipLaunchKernelGGL((k_compact<P>), dim3(g), dim3(B), 0, s, a);
    return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
}

// Shapes: the default 768 threads (704 data) x 5 rows of 4 (tile 14080;
// 161 VGPRs, three waves per SIMD: 25.8 us against 26.6 us for 448 x 8 on
// 1e7), 512 x 8, and 256 x 1 (small tiles for tests); element-wide variants
// for misaligned x.
template <class X, int CMP>
static CompactLaunch pick_compact_shape(int block, int rows, int vec) {
    if (vec == 4) {
        if (block == 512 && rows == 8) return &launch_compact_impl<X, CMP, 512, 8, 4>;
        if (block == 768 && rows == 5) return &launch_compact_impl<X, CMP, 768, 5, 4>;
        if (block == 256 && rows == 1) return &launch_compact_impl<X, CMP, 256, 1, 4>;
    } else if (vec == 1) {
        if (block == 512 && rows == 8) return &launch_compact_impl<X, CMP, 512, 8, 1>;
        if (block == 768 && rows == 5) return &launch_compact_impl<X, CMP, 768, 5, 1>;
        if (block == 256 && rows == 1) return &launch_compact_impl<X, CMP, 256, 1, 1>;
    }
    return nullptr;
}

template <class X>
static CompactLaunch pick_compact_cmp(scan_cmp_t cmp, int block, int rows, int vec) {
    switch (cmp) {
    case SCAN_CMP_GT: return pick_compact_shape<X, SCAN_CMP_GT>(block, rows, vec);
    case SCAN_CMP_GE: return pick_compact_shape<X, SCAN_CMP_GE>(block, rows, vec);
    case SCAN_CMP_LT: return pick_compact_shape<X, SCAN_CMP_LT>(block, rows, vec);
    case SCAN_CMP_LE: return pick_compact_shape<X, SCAN_CMP_LE>(block, rows, vec);
    case SCAN_CMP_EQ: return pick_compact_shape<X, SCAN_CMP_EQ>(block, rows, vec);
    case SCAN_CMP_NE: return pick_compact_shape<X, SCAN_CMP_NE>(block, rows, vec);
    case SCAN_CMP_BIT_CLEAR:
    case SCAN_CMP_BIT_SET:
        if constexpr (!std::is_floating_point_v<X>) {
            if (cmp == SCAN_CMP_BIT_CLEAR) return pick_compact_shape<X, SCAN_CMP_BIT_CLEAR>(block, rows, vec);
            return pick_compact_shape<X, SCAN_CMP_BIT_SET>(block, rows, vec);
        }
        return nullptr;
    }
    return nullptr;
}

// ------------------------------------------------- resident compaction
// Arrays that fit one tile per compute unit, in one step (the resident scan
// pass of resident.hip, applied to the selection counts): a control wave
// (wave 0) runs the call protocol while 15 data waves load their rows of x
// and, row by row as the data arrives, evaluate the predicate and count the
// selected elements before each lane in the row with four ballots (no wave
// scan).  After a barrier the control wave scans the (row, wave) counts in
// tile order and publishes the tile's count; after a second, each data
// thread places the tile-local index of each of its selected elements at its
// slot of an LDS stash while the control wave reads the counts of every
// earlier tile (one gap read); after a third, all 16 waves write the tile's
// contiguous output range with whole 16-byte stores.  Traffic: x read once,
// the selected indices written once.
//
// The stable partition (PartitionArgs) in the same shape: the control wave
// reads the counts of all tiles in one gap read -- the selected elements
// before its tile and the total k -- so no count pass is needed; then every
// data thread writes each of its elements (value, and index) to its final
// slot: selected element with s selected before it to s, the others to
// k + (rejected before it).  The tile's output goes out in chunks of
// kResPartChunkRows rows staged in LDS (values and tile-local indices): a
// chunk's selected elements are one contiguous run of the output and its
// rejected ones another, so each is written with whole 16-byte stores.
// (4-byte stores straight from the registers, two runs per (row, wave),
// took 43.9 us for 1e7 against 47.1 for the two-pass pipeline.)  Traffic:
// x read once, values and indices written once.
template <class X, int CMP, int MAXR, class A>
__global__ __launch_bounds__(kResWaves *kWave) void k_compact_resident(A a, uint32_t rows) {
    constexpr bool PART = std::is_same_v<A, PartitionArgs>;
    using D = Desc<int32_t>;
    constexpr int V = 4;
    constexpr int NDW = kResWaves - 1;                    // data waves
    constexpr int RE = NDW * kWave * V;                   // elements per tile row
    constexpr int KE = (MAXR * NDW + kWave - 1) / kWave;  // (row, wave) counts per lane of the control wave
    static_assert(MAXR * RE <= 65536, "tile-local indices fit 16 bits");
    constexpr int CH = kResPartChunkRows;
    constexpr int LIDX = PART ? CH * RE : MAXR * RE;
    __shared__ uint16_t lidx[LIDX];     // tile-local indices in output order (partition: of the chunk's rows)
    __shared__ int32_t sval[PART ? CH * RE : 1];  // partition: the chunk's values in output order
    __shared__ int32_t ent[MAXR * NDW];   // (row, wave) counts, then their exclusive prefixes in the tile
    __shared__ int32_t s_pre, s_nsel, s_total;
    __shared__ uint32_t s_epoch, s_dyn, s_claim;  // s_dyn: nonzero in dynamic mode
    __shared__ uint64_t s_hw, s_cap;
    WsHeader *hdr = reinterpret_cast<WsHeader *>(a.pipe.ws);
    uint64_t *desc = reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(a.pipe.ws) + kWsHeaderBytes);
    const int lane = lane_id();
    const uint32_t wr = uniform(uint32_t(threadIdx.x / kWave));
    const bool ctrl = wr == 0;
    const uint32_t dw = wr - 1;                         // data wave index (data waves only)
    const uint32_t dt = uint32_t(threadIdx.x) - kWave;  // data thread index
    const uint32_t nt = a.pipe.num_tiles;
    rows = uniform(rows);
    const int64_t tile_elems = int64_t(rows) * RE;
    const X thr = __builtin_bit_cast(X, a.threshold);
    const int32_t *xs = reinterpret_cast<const int32_t *>(a.x);

    Vec<int32_t, V> x[MAXR];
    uint32_t pk[MAXR];  // per row: selection bits (4) | selected elements in lower lanes << 4
    const uint32_t voff = dt * V * 4u;
    constexpr uint32_t kRowBytes = uint32_t(RE) * 4u;
    auto load = [&](uint32_t t) {
        const int64_t start = int64_t(t) * tile_elems, rem = a.n - start;
        const BufRsrc rs = make_rsrc(xs + start, rem < tile_elems ? rem : tile_elems);
#pragma unroll
        for (int r = 0; r < MAXR; r++) {
            if (r < int(rows))
                x[r] = __builtin_bit_cast(Vec<int32_t, V>, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, r * kRowBytes, 2));
        }
    };
    auto select_rows = [&](uint32_t t) {
        const int64_t rem = uniform(a.n - int64_t(t) * tile_elems);
#pragma unroll
        for (int r = 0; r < MAXR; r++) {
            if (r < int(rows)) {
                const int64_t e0 = int64_t(r) * RE + int64_t(dt) * V;
                uint32_t b = 0;
#pragma unroll
                for (int c = 0; c < V; c++)
                    b |= uint32_t(e0 + c < rem && keep<X, CMP>(__builtin_bit_cast(X, x[r].v[c]), thr)) << c;
                uint32_t below = 0, total = 0;
#pragma unroll
                for (int c = 0; c < V; c++) {
                    const uint64_t m = __ballot((b >> c) & 1u);
                    below += __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
                    total += uint32_t(__builtin_popcountll(m));
                }
                pk[r] = b | (below << 4);
                if (lane == 0) ent[r * NDW + dw] = int32_t(total);
            }
        }
    };
    // The control wave: the tile's (row, wave) counts into their exclusive
    // offsets in LDS, the tile's count published.
    auto scan_counts = [&](uint32_t t) {
        const uint32_t ne = rows * NDW;
        int32_t e[KE];
        int32_t acc = 0;
#pragma unroll
        for (int k = 0; k < KE; k++) {
            const uint32_t i = uint32_t(lane) * KE + k;
            e[k] = i < ne ? ent[i] : 0;
            acc += e[k];
        }
        const int32_t linc = wave_scan_incl<OpSum>(acc);
        int32_t run = linc - acc;
#pragma unroll
        for (int k = 0; k < KE; k++) {
            const uint32_t i = uint32_t(lane) * KE + k;
            if (i < ne) ent[i] = run;
            run += e[k];
        }
        const int32_t nsel = wave_read(linc, kWave - 1);
        if (lane == 0) {
            s_nsel = nsel;
            if (nt > 1) {
                if (a.pipe.delay_stride > 0 && t % a.pipe.delay_stride == a.pipe.delay_stride - 1) {
                    // a late publisher, so tests reach the look-back's re-polls
                    for (uint32_t i = 0; i < a.pipe.delay_sleeps; i++) __builtin_amdgcn_s_sleep(64);
                }
                D::publish(desc + uint64_t(t) * D::kWords, s_epoch, kStateA, nsel);
            }
        }
    };
    // As in the resident scan (resident.hip): the control wave starts the
    // call and, for tiles of at most kResLateDecisionRows rows, publishes its
    // static tile's count before the residency decision (the tile's claimer
    // in dynamic mode publishes the same word); longer tiles decide while
    // they load.  The two kinds of waves run separate programs that meet at
    // the same barriers: B1 (the static tile's rows selected), Bm (the mode
    // decided; in static mode the offsets ready), and in dynamic mode Bd
    // (the claimed tile selected) and Bp (its offsets ready).
    uint32_t tile = blockIdx.x;
    if (ctrl) {
        // short tiles decide after publishing, long ones while loading
        const bool late = rows <= uint32_t(kResLateDecisionRows);
        uint32_t dm = 0, ck = 0;
        auto decide = [&]() {
            const uint32_t m = decide_mode(hdr, s_epoch, gridDim.x, a.pipe.mode_limit);
            dm = m == kModeStatic ? 0u : 1u;
            ck = m == kModeStatic ? uint32_t(blockIdx.x)
                                  : __hip_atomic_fetch_add(&hdr->claim, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        };
        if (lane == 0) {
            uint64_t hw = 0, cap = 0;
            s_epoch = begin_call(hdr, hw, cap);
            s_hw = hw;
            s_cap = cap;
            if (!late) decide();
        }
        __syncthreads();  // B1
        scan_counts(tile);
        if (lane == 0) {
            if (late) decide();
            s_dyn = dm;
            s_claim = ck;
        }
        dm = uint32_t(__builtin_amdgcn_readlane(int(dm), 0));
        ck = uint32_t(__builtin_amdgcn_readlane(int(ck), 0));
        __syncthreads();  // Bm
        if (dm != 0u) {
            tile = ck;
            __syncthreads();  // Bd
            scan_counts(tile);
            __syncthreads();  // Bp
        }
    } else {
        load(tile);
        select_rows(tile);
        __syncthreads();  // B1
        __syncthreads();  // Bm
        if (s_dyn != 0u) {
            tile = s_claim;
            load(tile);
            select_rows(tile);
            __syncthreads();  // Bd
            __syncthreads();  // Bp
        }
    }
    const uint32_t epoch = s_epoch;
    const int64_t start = int64_t(tile) * tile_elems;
    if constexpr (PART) {
        const int64_t rem = a.n - start;
        const int32_t nsel = s_nsel;
        // chunk [c0, c1) of the tile's rows: selected before it (in the tile),
        // selected and rejected in it, rejected before it
        auto chunk = [&](int c0, int &c1, int32_t &sel0, int32_t &nsc, int32_t &nrc, int32_t &rej_b) {
            c1 = c0 + CH < int(rows) ? c0 + CH : int(rows);
            sel0 = ent[c0 * NDW];
            const int32_t sel1 = c1 < int(rows) ? ent[c1 * NDW] : nsel;
            const int64_t end = int64_t(c1) * RE < rem ? int64_t(c1) * RE : rem;
            nsc = sel1 - sel0;
            nrc = int32_t(end - int64_t(c0) * RE) - nsc;
            rej_b = c0 * RE - sel0;
        };
        // the chunk's values and tile-local indices into LDS in output order
        // (tile-local: no prefix needed)
        auto stage = [&](int c0, int c1, int32_t sel0, int32_t nsc, int32_t rej_b) {
#pragma unroll
            for (int r = 0; r < MAXR; r++) {
                if (r >= c0 && r < c1) {
                    int32_t sb = ent[r * NDW + dw] + int32_t(pk[r] >> 4);  // selected before, in the tile
#pragma unroll
                    for (int c = 0; c < V; c++) {
                        const int32_t li = r * RE + int32_t(dt) * V + c;
                        if (li < rem) {
                            const bool sel = (pk[r] >> c) & 1u;
                            const int32_t slot = sel ? sb - sel0 : nsc + (li - sb) - rej_b;
                            sval[slot] = x[r].v[c];
                            lidx[slot] = uint16_t(li);
                            sb += int32_t(sel);
                        }
                    }
                }
            }
        };
        if (ctrl) {
            // every tile's count: the total, and the sum over the earlier ones
            int32_t total = s_nsel, pre = 0;
            if (nt > 1) {
                GapRead<int32_t, D, kResMaxTiles / kWave> g;
                g.issue(desc, 0, int64_t(nt));
                total = g.template finish<OpSum>(desc, epoch, hdr, a.pipe.spin_limit);
                int32_t part = 0;
#pragma unroll
                for (int k = 0; k < kResMaxTiles / kWave; k++) {
                    const uint32_t t = uint32_t(lane) + uint32_t(kWave) * k;
                    int32_t v = 0;
                    if (t < tile && D::decode(g.w[k], epoch, v) != 0u) part += v;
                }
                pre = wave_reduce<OpSum>(part);
            }
            if (lane == 0) {
                s_pre = pre;
                s_total = total;
                if (tile == nt - 1) *a.count = total;
            }
        } else {
            // the first chunk is staged while the control wave reads the counts
            int c1;
            int32_t sel0, nsc, nrc, rej_b;
            chunk(0, c1, sel0, nsc, nrc, rej_b);
            stage(0, c1, sel0, nsc, rej_b);
        }
        __syncthreads();
        const int64_t pre = s_pre, rej0 = int64_t(s_total) + (start - pre);  // first rejected slot of the tile
        const int32_t s0 = int32_t(start);  // n <= INT32_MAX
        int32_t *vals = reinterpret_cast<int32_t *>(a.out_vals);
#pragma unroll
        for (int c0 = 0; c0 < MAXR; c0 += CH) {
            if (c0 >= int(rows)) break;
            int c1;
            int32_t sel0, nsc, nrc, rej_b;
            chunk(c0, c1, sel0, nsc, nrc, rej_b);
            if (c0 > 0) {
                if (!ctrl) stage(c0, c1, sel0, nsc, rej_b);
                __syncthreads();
            }
            write_range<kResWaves * kWave>(vals, pre + sel0, nsc, a.n, [&](int32_t i) { return sval[i]; });
            write_range<kResWaves * kWave>(vals, rej0 + rej_b, nrc, a.n, [&](int32_t i) { return sval[nsc + i]; });
            if (a.out_idx != nullptr) {
                write_range<kResWaves * kWave>(a.out_idx, pre + sel0, nsc, a.n,
                                               [&](int32_t i) { return s0 + int32_t(lidx[i]); });
                write_range<kResWaves * kWave>(a.out_idx, rej0 + rej_b, nrc, a.n,
                                               [&](int32_t i) { return s0 + int32_t(lidx[nsc + i]); });
            }
            __syncthreads();
        }
        if (tile == nt - 1) end_call(hdr, epoch, s_hw, s_cap, a.pipe.words_used, a.pipe.ws_words, desc);
        return;
    }
    if (ctrl) {
        int32_t pre = 0;
        if (tile > 0) {
            GapRead<int32_t, D, kResMaxTiles / kWave> g;
            g.issue(desc, 0, int64_t(tile));
            pre = g.template finish<OpSum>(desc, epoch, hdr, a.pipe.spin_limit);
        }
        if (lane == 0) {
            s_pre = pre;
            if (tile == nt - 1) *a.count = pre + s_nsel;
        }
    } else {
#pragma unroll
        for (int r = 0; r < MAXR; r++) {
            if (r < int(rows)) {
                int32_t pos = ent[r * NDW + dw] + int32_t(pk[r] >> 4);
#pragma unroll
                for (int c = 0; c < V; c++) {
                    if ((pk[r] >> c) & 1u) lidx[pos++] = uint16_t(r * RE + int32_t(dt) * V + c);
                }
            }
        }
    }
    __syncthreads();
    const int32_t s0 = int32_t(start);  // n <= INT32_MAX
    write_range<kResWaves * kWave>(a.out_idx, int64_t(s_pre), s_nsel, a.n,
                                   [&](int32_t i) { return s0 + int32_t(lidx[i]); });
    // end of the call: in static mode every workgroup was counted before the
    // decision; in dynamic mode the holder of the last ticket claimed last
    if (tile == nt - 1) end_call(hdr, epoch, s_hw, s_cap, a.pipe.words_used, a.pipe.ws_words, desc);
}

template <class X, int CMP, class A>
static int launch_compact_resident_impl(const A &a, int rows, hipStream_t s) {
    if (rows < 1 || rows > kResCompactMaxRows || a.pipe.num_tiles > uint32_t(kResMaxTiles)) return SCAN_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((k_compact_resident<X, CMP, kResCompactMaxRows, A>), dim3(a.pipe.num_tiles),
                       dim3(kResWaves * kWave), 0, s, a, uint32_t(rows));
    return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
}

// The launcher for (X, cmp) with arguments A (CompactArgs or PartitionArgs).
template <class X, class A>
static auto pick_compact_resident(scan_cmp_t cmp) -> int (*)(const A &, int, hipStream_t) {
    switch (cmp) {
    case SCAN_CMP_GT: return &launch_compact_resident_impl<X, SCAN_CMP_GT, A>;
    case SCAN_CMP_GE: return &launch_compact_resident_impl<X, SCAN_CMP_GE, A>;
    case SCAN_CMP_LT: return &launch_compact_resident_impl<X, SCAN_CMP_LT, A>;
    case SCAN_CMP_LE: return &launch_compact_resident_impl<X, SCAN_CMP_LE, A>;
    case SCAN_CMP_EQ: return &launch_compact_resident_impl<X, SCAN_CMP_EQ, A>;
    case SCAN_CMP_NE: return &launch_compact_resident_impl<X, SCAN_CMP_NE, A>;
    case SCAN_CMP_BIT_CLEAR:
    case SCAN_CMP_BIT_SET:
        if constexpr (!std::is_floating_point_v<X>) {
            if (cmp == SCAN_CMP_BIT_CLEAR) return &launch_compact_resident_impl<X, SCAN_CMP_BIT_CLEAR, A>;
            return &launch_compact_resident_impl<X, SCAN_CMP_BIT_SET, A>;
        }
        return nullptr;
    }
    return nullptr;
}

#if SW64_PART == 0
#if SW64_DT == 0
ResCompactLaunch find_compact_resident_i32(scan_cmp_t cmp) { return pick_compact_resident<int32_t, CompactArgs>(cmp); }
#elif SW64_DT == 1
ResCompactLaunch find_compact_resident_u32(scan_cmp_t cmp) { return pick_compact_resident<uint32_t, CompactArgs>(cmp); }
#elif SW64_DT == 3
ResCompactLaunch find_compact_resident_f32(scan_cmp_t cmp) { return pick_compact_resident<float, CompactArgs>(cmp); }
#endif
#else
#if SW64_DT == 0
ResPartitionLaunch find_partition_resident_i32(scan_cmp_t cmp) { return pick_compact_resident<int32_t, PartitionArgs>(cmp); }
#elif SW64_DT == 1
ResPartitionLaunch find_partition_resident_u32(scan_cmp_t cmp) { return pick_compact_resident<uint32_t, PartitionArgs>(cmp); }
#elif SW64_DT == 3
ResPartitionLaunch find_partition_resident_f32(scan_cmp_t cmp) { return pick_compact_resident<float, PartitionArgs>(cmp); }
#endif
#endif

#if SW64_PART == 0
#if SW64_DT == 0
CompactLaunch find_compact_i32(scan_cmp_t cmp, int b, int r, int v) { return pick_compact_cmp<int32_t>(cmp, b, r, v); }
#elif SW64_DT == 1
CompactLaunch find_compact_u32(scan_cmp_t cmp, int b, int r, int v) { return pick_compact_cmp<uint32_t>(cmp, b, r, v); }
#elif SW64_DT == 3
CompactLaunch find_compact_f32(scan_cmp_t cmp, int b, int r, int v) { return pick_compact_cmp<float>(cmp, b, r, v); }
#endif
#endif

// -------------------------------------------------------------- partition
// Stable partition (Merry, "Prefix sums on GPUs", slide "Other
// Applications": partitioning places the objects that satisfy a predicate
// before the others; radix sort is repeated partitioning, so each part keeps
// the input order).  Element i with s_i selected elements before it goes to
// s_i when selected, else to k + (i - s_i), k being the total selected.
// s_i comes from the compaction's fused scan on the look-back pipeline; k
// must be known before the first rejected element is written, so a count
// pass runs first and publishes one count per workgroup as descriptor
// words of this call (state A, the call's epoch) just above the scan's own
// tile descriptors; the scan's control wave adds them up in its setup step.
// Traffic: x read twice, the values (and indices) written once.

// Count pass: workgroup w counts the selected elements of its contiguous
// chunk of x and publishes the count.
constexpr int kPartCountThreads = 256, kPartCountMax = 1024;  // at most this many count words

template <class X, int CMP, int VEC>
__global__ __launch_bounds__(kPartCountThreads) void k_part_count(PartitionArgs a) {
    __shared__ int32_t wsum[kPartCountThreads / kWave];
    const WsHeader *hdr = reinterpret_cast<const WsHeader *>(a.pipe.ws);
    uint64_t *desc = reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(a.pipe.ws) + kWsHeaderBytes);
    const int64_t b = int64_t(blockIdx.x) * a.count_chunk;
    const int64_t e = b + a.count_chunk < a.n ? b + a.count_chunk : a.n;
    const X t = __builtin_bit_cast(X, a.threshold);
    const X *x = reinterpret_cast<const X *>(a.x);
    int32_t cnt = 0;
    constexpr int64_t kStep = int64_t(kPartCountThreads) * VEC;
#pragma unroll 4
    for (int64_t i = b + int64_t(threadIdx.x) * VEC; i < e; i += kStep) {
        // chunks start on VEC boundaries and n is a multiple of VEC here.
        // Plain (temporal) loads: the partition pass reads x again right
        // after, and may then find it in the caches.
        const Vec<X, VEC> v = *reinterpret_cast<const Vec<X, VEC> *>(x + i);
#pragma unroll
        for (int c = 0; c < VEC; c++) cnt += keep<X, CMP>(v.v[c], t) ? 1 : 0;
    }
    cnt = wave_reduce<OpSum>(cnt);
    if (lane_id() == 0) wsum[threadIdx.x / kWave] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t tot = 0;
        for (int w = 0; w < kPartCountThreads / kWave; w++) tot += wsum[w];
        Desc<int32_t>::publish(desc + a.count_base + blockIdx.x, ld(&hdr->epoch), kStateA, tot);
    }
}

template <class X, int CMP, int BLOCK_, int ROWS, int VEC>
struct PartitionPolicy {
    using T = int32_t;
    using Op = OpSum;
    using C = int32_t;
    using D = Desc<C>;
    static constexpr int kDescWords = D::kWords;
    static constexpr int BLOCK = BLOCK_;
    using TS = TileScan<int32_t, OpSum, BLOCK, ROWS, VEC>;
    using Args = PartitionArgs;
    using Shared = typename TS::Shared;
    using V = Vec<uint32_t, VEC>;
    static_assert(ROWS * VEC <= 32, "selection bits fit one word");

    __device__ __forceinline__ static C aggregate(const Shared &sh) { return TS::template aggregate_from<C>(sh); }

    // The total selected: the count pass's words, one round trip.
    static constexpr bool kSetup = true;
    __device__ __forceinline__ static C setup(const Args &a, const uint64_t *desc, uint32_t epoch, WsHeader *hdr) {
        GapRead<C, D, kPartCountMax / kWave> counts;
        counts.issue(desc, int64_t(a.count_base), int64_t(a.count_base) + a.count_wgs);
        return counts.template finish<Op>(desc, epoch, hdr, a.pipe.spin_limit);
    }

    // A scanned tile waiting for its prefix, already in output order: the
    // selected elements (values and tile-local indices), then the rejected
    // ones, and the selected count.  Each part then goes out as one
    // contiguous range of whole 16-byte stores.
    static_assert(TS::TILE <= 65536, "tile-local indices fit 16 bits");
    struct Stash {
        uint32_t val[TS::TILE];
        uint16_t lidx[TS::TILE];
        int32_t nsel;
    };
    static constexpr bool kStagedEmit = true;  // emit reads other threads' slots

    __device__ __forceinline__ static void emit(const Stash &st, const Args &a, uint32_t tile, C pre, bool valid,
                                                C total) {
        if (!valid) return;
        const int64_t start = int64_t(tile) * TS::TILE;
        const int32_t cnt = int32_t(a.n - start < TS::TILE ? a.n - start : TS::TILE);
        const int32_t nsel = st.nsel, s32 = int32_t(start);  // n <= INT32_MAX
        int32_t *vals = reinterpret_cast<int32_t *>(a.out_vals);
        // selected: from position pre; rejected: after all k selected, from
        // k + (elements before the tile) - pre.  A failed wait (flagged in
        // the workspace) must not write outside [0, n).
        const int64_t g_sel = int64_t(pre), g_rej = int64_t(total) + (start - int64_t(pre));
        write_range<BLOCK>(vals, g_sel, nsel, a.n, [&](int32_t i) { return int32_t(st.val[i]); });
        write_range<BLOCK>(vals, g_rej, cnt - nsel, a.n, [&](int32_t i) { return int32_t(st.val[nsel + i]); });
        if (a.out_idx != nullptr) {
            write_range<BLOCK>(a.out_idx, g_sel, nsel, a.n, [&](int32_t i) { return s32 + int32_t(st.lidx[i]); });
            write_range<BLOCK>(a.out_idx, g_rej, cnt - nsel, a.n,
                               [&](int32_t i) { return s32 + int32_t(st.lidx[nsel + i]); });
        }
    }

    __device__ __forceinline__ static void on_resolved(const Args &a, uint32_t tile, C pre, C agg) {
        if (tile == a.pipe.num_tiles - 1) *a.count = pre + agg;
    }

    struct Tile {
        TS ts;          // raw element bits after load, 0/1 counts after scan
        V raw[ROWS];    // the loaded values, kept for emission
        uint32_t bits;  // bit r*VEC + c: element c of this thread's vector in row r is selected
        uint32_t thr;
        int64_t rem;

        __device__ __forceinline__ void load(const Args &a, uint32_t tile) {
            const bool valid = tile < a.pipe.num_tiles;
            const int64_t start = valid ? int64_t(tile) * TS::TILE : 0;
            rem = valid ? uniform(a.n - start) : 0;
            thr = a.threshold;
            const int32_t *x = reinterpret_cast<const int32_t *>(a.x) + uniform(start);
#pragma unroll
            for (int r = 0; r < ROWS; r++) {
                const int64_t e = TS::elem(r);
                ts.v[r] = load_vec<int32_t, VEC>(x + (e < rem ? e : 0));
            }
        }

        __device__ __forceinline__ void scan(Shared &sh) {
            const X t = __builtin_bit_cast(X, thr);
            bits = 0;
#pragma unroll
            for (int r = 0; r < ROWS; r++) {
                const int64_t e = TS::elem(r);
                raw[r] = __builtin_bit_cast(V, ts.v[r]);
#pragma unroll
                for (int c = 0; c < VEC; c++) {
                    const bool k = (e + c < rem) && keep<X, CMP>(__builtin_bit_cast(X, ts.v[r].v[c]), t);
                    ts.v[r].v[c] = k ? 1 : 0;
                    bits |= uint32_t(k) << (r * VEC + c);
                }
            }
            ts.rem = TS::TILE;
            ts.scan(sh);
        }

        // Element i of the tile with s selected before it goes to s when
        // selected, else to nsel + (i - s).
        __device__ __forceinline__ void stash(Stash &st, const Args &) const {
            const int32_t nsel = ts.agg;
#pragma unroll
            for (int r = 0; r < ROWS; r++) {
                const int32_t e = int32_t(TS::elem(r));
                int32_t sel = ts.off[r];
#pragma unroll
                for (int c = 0; c < VEC; c++) {
                    const bool k = (bits >> (r * VEC + c)) & 1u;
                    const int32_t p = k ? sel : nsel + (e + c - sel);
                    if (e + c < rem) {
                        st.val[p] = raw[r].v[c];
                        st.lidx[p] = uint16_t(e + c);
                    }
                    sel += k ? 1 : 0;
                }
            }
            if (threadIdx.x == 0) st.nsel = nsel;
        }
    };
};

template <class P>
__global__ __launch_bounds__(CtrlPipeline<P>::THREADS) void k_partition(typename P::Args a) {
    CtrlPipeline<P>::run(a);
}

template <class X, int CMP, int B, int R, int V>
static int launch_partition_impl(const PartitionArgs &a, uint32_t grid_cap, hipStream_t s) {
    using P = PartitionPolicy<X, CMP, B - kWave, R, V>;
    if (a.count_wgs < 1 || a.count_wgs > uint32_t(kPartCountMax)) return SCAN_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((k_part_count<X, CMP, V>), dim3(a.count_wgs), dim3(kPartCountThreads), 0, s, a);
    if (hipGetLastError() != hipSuccess) return SCAN_ERR_HIP;
    const int g = pipeline_grid(reinterpret_cast<const void *>(&k_partition<P>), B, a.pipe.num_tiles, grid_cap);
    if (g <= 0) return SCAN_ERR_HIP;
    hipLaunchKernelGGL((k_partition<P>), dim3(g), dim3(B), 0, s, a);
    return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
}

// Shapes: the default 768 threads (704 data) x 3 rows of 4 (tile 8448:
// 48.4 us against 49.6 us for 448 x 6 on 1e7 fp32, including the count
// pass), 512 x 6, and 256 x 1 (small tiles for tests); element-wide
// variants for misaligned x.
template <class X, int CMP>
static PartitionLaunch pick_partition_shape(int block, int rows, int vec) {
    if (vec == 4) {
        if (block == 512 && rows == 6) return &launch_partition_impl<X, CMP, 512, 6, 4>;
        if (block == 768 && rows == 3) return &launch_partition_impl<X, CMP, 768, 3, 4>;
        if (block == 256 && rows == 1) return &launch_partition_impl<X, CMP, 256, 1, 4>;
    } else if (vec == 1) {
        if (block == 512 && rows == 6) return &launch_partition_impl<X, CMP, 512, 6, 1>;
        if (block == 768 && rows == 3) return &launch_partition_impl<X, CMP, 768, 3, 1>;
        if (block == 256 && rows == 1) return &launch_partition_impl<X, CMP, 256, 1, 1>;
    }
    return nullptr;
}

template <class X>
static PartitionLaunch pick_partition_cmp(scan_cmp_t cmp, int block, int rows, int vec) {
    switch (cmp) {
    case SCAN_CMP_GT: return pick_partition_shape<X, SCAN_CMP_GT>(block, rows, vec);
    case SCAN_CMP_GE: return pick_partition_shape<X, SCAN_CMP_GE>(block, rows, vec);
    case SCAN_CMP_LT: return pick_partition_shape<X, SCAN_CMP_LT>(block, rows, vec);
    case SCAN_CMP_LE: return pick_partition_shape<X, SCAN_CMP_LE>(block, rows, vec);
    case SCAN_CMP_EQ: return pick_partition_shape<X, SCAN_CMP_EQ>(block, rows, vec);
    case SCAN_CMP_NE: return pick_partition_shape<X, SCAN_CMP_NE>(block, rows, vec);
    case SCAN_CMP_BIT_CLEAR:
    case SCAN_CMP_BIT_SET:
        if constexpr (!std::is_floating_point_v<X>) {
            if (cmp == SCAN_CMP_BIT_CLEAR) return pick_partition_shape<X, SCAN_CMP_BIT_CLEAR>(block, rows, vec);
            return pick_partition_shape<X, SCAN_CMP_BIT_SET>(block, rows, vec);
        }
        return nullptr;
    }
    return nullptr;
}

#if SW64_PART == 1
#if SW64_DT == 0
PartitionLaunch find_partition_i32(scan_cmp_t cmp, int b, int r, int v) { return pick_partition_cmp<int32_t>(cmp, b, r, v); }
#elif SW64_DT == 1
PartitionLaunch find_partition_u32(scan_cmp_t cmp, int b, int r, int v) { return pick_partition_cmp<uint32_t>(cmp, b, r, v); }
#elif SW64_DT == 3
PartitionLaunch find_partition_f32(scan_cmp_t cmp, int b, int r, int v) { return pick_partition_cmp<float>(cmp, b, r, v); }
#endif
#endif

#if SW64_PART == 0 && SW64_DT == 0
// ------------------------------------------------------------------- emit
// One thread per object; the record value starts at (i + 1) mod n and wraps
// at n without a division per record.
// Emit in windows of LDS.  A workgroup takes kEmitObjects consecutive
// objects, whose records form one contiguous output range.  Each thread
// writes its objects' records into an LDS window (4-byte LDS stores, cheap
// even where counts vary within a wave), then the workgroup copies the
// window out with 16-byte stores that are whole and aligned except at the
// range's two ends.  Writing the records straight from each object's thread
// gives 4-byte stores scattered by the counts, which measured 2.4x slower.
// A range longer than the window is done in several windows, so any counts
// work; Poisson(3) counts fill one window per workgroup.
constexpr int kEmitThreads = 256, kEmitObjects = 1024, kEmitWindow = 3968;

__global__ __launch_bounds__(kEmitThreads) void k_emit_neighbors(const int32_t *offsets, int64_t n, int32_t *out) {
    typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
    static_assert(kEmitObjects == 4 * kEmitThreads, "one 16-byte offsets load per thread");
    __shared__ __attribute__((aligned(16))) int32_t off[kEmitObjects + 4];
    __shared__ __attribute__((aligned(16))) int32_t win[kEmitWindow + 4];
    const int64_t i0 = int64_t(blockIdx.x) * kEmitObjects;
    const int cnt = int(n - i0 < kEmitObjects ? n - i0 : kEmitObjects);
    const int32_t *src = offsets + i0;
    if (cnt == kEmitObjects && (reinterpret_cast<uintptr_t>(src) & 15u) == 0) {
        // all of the workgroup's offset loads in flight at once
        const i32x4 v = *reinterpret_cast<const i32x4 *>(src + 4 * threadIdx.x);
        const int32_t last = threadIdx.x == 0 ? src[kEmitObjects] : 0;
        *reinterpret_cast<i32x4 *>(off + 4 * threadIdx.x) = v;
        if (threadIdx.x == 0) off[kEmitObjects] = last;
    } else {
        for (int t = threadIdx.x; t <= cnt; t += kEmitThreads) off[t] = src[t];
    }
    __syncthreads();
    const int64_t ob = off[0], oe = off[cnt];
    // windows start where out + k is 16-byte aligned
    const int64_t phase = int64_t((reinterpret_cast<uintptr_t>(out) >> 2) & 3u);
    for (int64_t w0 = ob - ((phase + ob) & 3); w0 < oe; w0 += kEmitWindow) {
        const int64_t w1 = oe - w0 < kEmitWindow ? oe : w0 + kEmitWindow;
        for (int j = threadIdx.x; j < cnt; j += kEmitThreads) {
            const int64_t b = off[j], e = off[j + 1];
            const int64_t lo = b > w0 ? b : w0, hi = e < w1 ? e : w1;
            int64_t r0 = i0 + j + 1 + (lo - b);  // first record value, (i + 1 + j) mod n
            if (r0 >= n) r0 -= n;
            if (r0 >= n) r0 %= n;
            // within the window everything fits 32 bits (n <= INT32_MAX)
            const int32_t n32 = int32_t(n), k1 = int32_t(hi - w0);
            int32_t r = int32_t(r0);
            for (int32_t k = int32_t(lo - w0); k < k1; k++) {
                win[k] = r;
                r = r + 1 == n32 ? 0 : r + 1;
            }
        }
        __syncthreads();
        for (int q = threadIdx.x; int64_t(4) * q < w1 - w0; q += kEmitThreads) {
            const int64_t k = w0 + 4 * q;
            const i32x4 x = *reinterpret_cast<const i32x4 *>(win + 4 * q);
            if (k >= ob && k + 4 <= w1) {
                __builtin_nontemporal_store(x, reinterpret_cast<i32x4 *>(out + k));
            } else {
#pragma unroll
                for (int c = 0; c < 4; c++)
                    if (k + c >= ob && k + c < w1) out[k + c] = x[c];
            }
        }
        __syncthreads();
    }
}

int launch_emit_neighbors(const int32_t *offsets, int64_t n, int32_t *out, hipStream_t s) {
    if (n <= 0) return SCAN_OK;
    const int64_t blocks = (n + kEmitObjects - 1) / kEmitObjects;
    hipLaunchKernelGGL(k_emit_neighbors, dim3(unsigned(blocks)), dim3(kEmitThreads), 0, s, offsets, n, out);
    return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
}

#endif

}  // namespace sw64

#if !defined(SW64_PART) || !defined(SW64_DT) || (SW64_DT != 0 && SW64_DT != 1 && SW64_DT != 3)
#error "SW64_PART (0, 1) and SW64_DT (0, 1, 3) select the unit"
#endif
