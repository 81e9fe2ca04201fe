// resident.hip -- single-pass scan of arrays that fit the chip's registers:
// one tile per compute unit, loaded once, scanned, written once.
//
// The look-back pipeline (pipeline.hpp) runs K + 2 steps per workgroup for
// K tiles, and a step is no shorter than a memory round trip under load, so
// at 1e7 elements (K of 2 to 5) its latency, not HBM, sets the time.  When
// the whole array fits in at most 256 register tiles, each workgroup instead
// loads one tile, publishes its aggregate, reads the aggregates of every
// tile before it in one round trip (the aggregate-only look-back of
// device.hpp, GapRead: the page's decoupled look-back with no inclusive
// prefixes, every predecessor read -- The CUDA Handbook ch. 13, decoupled
// look-back section) and stores: one step, no chain from tile to tile.
//
// A workgroup is a control wave (wave 0) and 15 data waves.  A tile is
// `rows` rows (chosen per call, at most MAXR) of 960 x V consecutive
// elements; row r is one coalesced 128-bit access per data thread (data
// thread t: elements (r * 960 + t) * V .. + V - 1).  Scan levels: each thread's V elements
// serially, each row across its wave with the DPP scan (the wave's
// exclusive prefix folded in at once, so nothing per row stays live but the
// values), then the control wave scans the rows x 15 (row, wave) totals from
// LDS in tile order.  Values stay in the element type inside the tile; the
// tile's prefix is added in the carry type, one rounding per output, as the
// look-back kernels do.
//
// The control wave holds no data: it runs the call protocol (the residency
// check, as in the pipeline: the tile index is the workgroup index when the
// whole grid is resident, else tiles are claimed in order) while the data
// waves load the static tile and scan each row as it arrives, then
// publishes and looks back.  Measured at 1e7 fp64: with a data wave running
// the protocol its rows arrived about 3 us late; with the control wave last
// in the workgroup its requests queued behind every data wave's loads (the
// mode was known after 16 us instead of 11); with the row scans after the
// barrier that waits for the protocol, 21 rows of wave scans (about 3.5 us)
// started only once the protocol was done instead of overlapping it.
//
// This file is compiled once per element type (SW64_DT selects it).
#include "launch.hpp"
#include "noid.hpp"

namespace sw64 {

// NOID: an inclusive scan that never uses the operator's identity (Op is
// then wrapped in NoId, which has none): elements past the segment's end
// are scanned as loaded (they reach only results past the end, which the
// bounded stores drop, and the last tile's aggregate, which no tile
// reads); a lane, a (row, wave) entry or a tile with nothing before it
// skips the combination instead of taking an identity; the look-back
// combines optional carries (Opt, "absent" being their only identity).
//
// SW = 2 (whole arrays only): each workgroup holds two tiles of `rows`
// rows, w and w + G in the static order (G workgroups), both loaded at
// once.  The first tile is scanned, published and looked back while the
// second one's loads land; the second is published and looked back while
// the first one's results are stored.  Its look-back is the pipeline's
// aggregate-only form: the workgroup's own first tile's inclusive prefix
// and the G - 1 aggregates between the two.  With one tile per workgroup
// the whole look-back sits between the loads and the stores, with HBM idle.
// Dynamic mode (tiles claimed in order) gives claim k the tiles 2k and
// 2k + 1, so every tile a look-back reads belongs to an earlier claim.
template <class T, class Op0, int V, int MAXR, int OUT_AUX, bool NOID = false, int SW = 1>
__global__ __launch_bounds__(kResWaves *kWave) void k_resident(ScanArgs a, uint32_t rows) {
    static_assert(SW == 1 || SW == 2, "one or two tiles per workgroup");
    using Op = std::conditional_t<NOID, NoId<Op0>, Op0>;
    using C = typename Carry<T, Op0>::type;
    using D = DescFor<T, C>;
    constexpr int NDW = kResWaves - 1;                          // data waves
    constexpr int RE = NDW * kWave * V;                         // elements per tile row
    constexpr int KE = ((MAXR / SW) * NDW + kWave - 1) / kWave;  // (row, wave) totals per lane of the control wave
    constexpr int NRW = int(kResMaxTiles / kWave);              // look-back windows of 64 tiles
    constexpr int MS = MAXR / SW;                               // register rows (slots) per tile
    static_assert(V * sizeof(T) == 16, "128-bit rows");
    __shared__ T ent[MAXR * NDW];        // (row, wave) totals, then their exclusive prefixes in the tile
    __shared__ C s_pre[SW];              // each tile's exclusive prefix (NOID: none for a segment's first tile)
    __shared__ uint32_t s_epoch, s_claim, s_dyn;
    __shared__ uint64_t s_hw, s_cap;
    WsHeader *hdr = reinterpret_cast<WsHeader *>(a.pipe.ws);
    uint64_t *desc = reinterpret_cast<uint64_t *>(reinterpret_cast<char *>(a.pipe.ws) + kWsHeaderBytes);
    const int lane = lane_id();
    const uint32_t wr = uniform(uint32_t(threadIdx.x / kWave));
    const bool ctrl = wr == 0;
    const uint32_t dw = wr - 1;                                  // data wave index (data waves only)
    const uint32_t dt = uint32_t(threadIdx.x) - kWave;           // data thread index
    const uint32_t n = a.pipe.num_tiles, tps = a.pipe.tiles_per_seg;
    rows = uniform(rows);
    const int64_t tile_elems = int64_t(rows) * RE;
    const T *in = reinterpret_cast<const T *>(a.in);
    T *out = reinterpret_cast<T *>(a.out);

    auto geom = [&](uint32_t t, int64_t &start, int64_t &rem, uint32_t &seg, uint32_t &j) {
        seg = t / tps;
        j = t - seg * tps;
        start = uniform(int64_t(seg) * a.seg_len + int64_t(j) * tile_elems);
        rem = uniform(a.seg_len - int64_t(j) * tile_elems);
    };
    // Buffer accesses from the tile's first element, bounded by the segment:
    // rows and vectors past its end read 0 (replaced by the identity below)
    // and drop their stores.  Tile s of the workgroup holds its rows in the
    // register slots x[s * MS ..], its (row, wave) totals in LDS from entry
    // row s * rows.
    Vec<T, V> x[MAXR];
    const uint32_t voff = dt * V * uint32_t(sizeof(T));
    constexpr uint32_t kRowBytes = uint32_t(RE) * sizeof(T);
    BufRsrc rs_in[SW], rs_out[SW];
    auto load = [&](uint32_t t, int s) {
        int64_t start, rem;
        uint32_t seg, j;
        geom(t, start, rem, seg, j);
        int64_t cnt = rem < tile_elems ? rem : tile_elems;
        if (t >= n) cnt = 0;  // no such tile (an odd tile count's last workgroup): nothing in range
        rs_in[s] = make_rsrc(in + start, cnt);
        rs_out[s] = make_rsrc(out + start, cnt);
        // The first tile loads its rows only.  The second loads every slot,
        // rows past `rows` from beyond the buffer's range (they read 0 and
        // touch no memory): a fixed number of loads after the first tile's,
        // so the first tile's scan waits for its own loads only.  (With the
        // second tile's loads also counted at run time, the first tile's
        // scan waited for every load; with every slot loaded in one-tile
        // plans of few rows, the unused loads cost int32 2^22 10.9 -> 12.4 us.)
#pragma unroll
        for (int rr = 0; rr < MS; rr++) {
            if (s == 1 || uint32_t(rr) < rows)
                x[s * MS + rr] = __builtin_bit_cast(
                    Vec<T, V>, __builtin_amdgcn_raw_buffer_load_b128(rs_in[s], voff, uint32_t(rr) * kRowBytes, 2));
        }
    };
    // Each row of the tile: this thread's vector scanned, then across the
    // wave; every value becomes its result within the wave's 64 x V run
    // (inclusive, or exclusive with the identity first), and the wave's row
    // total goes to LDS.  Elements past the segment's end take the identity.
    auto scan_rows = [&](uint32_t t, int s) {
        int64_t start_, rem_;
        uint32_t seg_, j_;
        geom(t, start_, rem_, seg_, j_);
        const int64_t e_thread = int64_t(dt) * V;
#pragma unroll
        for (int rr = 0; rr < MS; rr++) {
            const int r = s * MS + rr;                    // register slot
            const uint32_t er = uint32_t(s) * rows + rr;  // (row, wave) entry row
            if (uint32_t(rr) < rows) {
                const int64_t e0 = int64_t(rr) * RE + e_thread;
                T inc[V];
                T acc = x[r].v[0];
#pragma unroll
                for (int c = 0; c < V; c++) {
                    T val = x[r].v[c];
                    if constexpr (!NOID) val = e0 + c < rem_ ? val : Op::template identity<T>();
                    acc = c == 0 ? val : Op::apply(acc, val);
                    inc[c] = acc;
                }
                if constexpr (NOID) {
                    // inclusive only; lane 0 has no lane before it
                    const T winc = wave_scan_incl_noid<Op>(acc);
                    const T wex = dpp_mov<kWaveShr1>(winc, winc);
#pragma unroll
                    for (int c = 0; c < V; c++) x[r].v[c] = lane > 0 ? Op::apply(wex, inc[c]) : inc[c];
                    if (lane == kWave - 1) ent[er * NDW + dw] = winc;
                } else {
                    const T id = Op::template identity<T>();
                    const T winc = wave_scan_incl<Op>(acc);
                    const T wex = wave_shr1(id, winc);
#pragma unroll
                    for (int c = 0; c < V; c++)
                        x[r].v[c] =
                            a.exclusive ? (c == 0 ? wex : Op::apply(wex, inc[c - 1])) : Op::apply(wex, inc[c]);
                    if (lane == kWave - 1) ent[er * NDW + dw] = winc;
                }
            }
        }
    };
    // Control wave: tile s's (row, wave) totals in tile order (lane l: KE
    // consecutive ones) scanned into their exclusive prefixes; returns the
    // tile's aggregate.
    auto scan_entries = [&](int s) -> C {
        const uint32_t ne = rows * NDW, b0 = uint32_t(s) * ne;
        T e[KE];
        if constexpr (NOID) {
            // lanes past the last entry hold whatever they read; they sit
            // above every lane with entries, so the inclusive scan carries
            // nothing from them down, and the aggregate is the last such
            // lane's result.  Entry 0 has nothing before it: its slot is left
            // as it is (the data waves do not read it).
            T acc = ent[b0 + (uint32_t(lane) * KE < ne ? uint32_t(lane) * KE : 0u)];
#pragma unroll
            for (int k = 0; k < KE; k++) {
                const uint32_t i = uint32_t(lane) * KE + k;
                e[k] = ent[b0 + (i < ne ? i : 0u)];
                if (k > 0 && i < ne) acc = Op::apply(acc, e[k]);
            }
            const T linc = wave_scan_incl_noid<Op>(acc);
            T run = dpp_mov<kWaveShr1>(linc, linc);
#pragma unroll
            for (int k = 0; k < KE; k++) {
                const uint32_t i = uint32_t(lane) * KE + k;
                if (i < ne) {
                    if (i > 0) ent[b0 + i] = run;
                    run = i > 0 ? Op::apply(run, e[k]) : e[k];
                }
            }
            return C(wave_read(linc, int((ne - 1) / KE)));
        } else {
            const T id = Op::template identity<T>();
            T acc = id;
#pragma unroll
            for (int k = 0; k < KE; k++) {
                const uint32_t i = uint32_t(lane) * KE + k;
                e[k] = i < ne ? ent[b0 + i] : id;
                acc = Op::apply(acc, e[k]);
            }
            const T linc = wave_scan_incl<Op>(acc);
            T run = wave_shr1(id, linc);
#pragma unroll
            for (int k = 0; k < KE; k++) {
                const uint32_t i = uint32_t(lane) * KE + k;
                if (i < ne) ent[b0 + i] = run;
                run = Op::apply(run, e[k]);
            }
            return C(wave_read(linc, kWave - 1));
        }
    };
    auto publish = [&](uint32_t t, const C &agg) {
        if (a.pipe.delay_stride > 0 && t % a.pipe.delay_stride == a.pipe.delay_stride - 1) {
            // a late publisher, so tests reach the look-back's re-polls
            for (uint32_t i = 0; i < a.pipe.delay_sleeps; i++) __builtin_amdgcn_s_sleep(64);
        }
        if (lane == 0) D::publish(desc + uint64_t(t) * D::kWords, s_epoch, kStateA, agg);
    };
    // The combination of the aggregates of tiles [lo, hi) (non-empty, all
    // published with a value), read kResMaxTiles at a time: one round trip
    // except for dynamic mode's first tiles of SW = 2 (up to twice as many).
    auto gap = [&](uint32_t lo, uint32_t hi) -> C {
        C acc{};
        for (uint32_t b = lo; b < hi; b += uint32_t(kResMaxTiles)) {
            const uint32_t e = hi - b > uint32_t(kResMaxTiles) ? b + uint32_t(kResMaxTiles) : hi;
            C part;
            if constexpr (NOID) {
                GapRead<Opt<C>, OptDesc<D>, NRW> g;
                g.issue(desc, int64_t(b), int64_t(e));
                part = g.template finish<OptOp<Op0>>(desc, s_epoch, hdr, a.pipe.spin_limit).v;
            } else {
                GapRead<C, D, NRW> g;
                g.issue(desc, int64_t(b), int64_t(e));
                part = g.template finish<Op>(desc, s_epoch, hdr, a.pipe.spin_limit);
            }
            acc = b == lo ? part : C(Op::apply(acc, part));
        }
        return acc;
    };
    // Tile s's results: (row, wave) prefix, then the tile's prefix (carry
    // type, one rounding); has_pre false for a segment's first tile.
    auto store = [&](int s, const C &pre, bool has_pre) {
#pragma unroll
        for (int rr = 0; rr < MS; rr++) {
            const int r = s * MS + rr;
            if (uint32_t(rr) < rows) {
                const T eb = ent[(uint32_t(s) * rows + rr) * NDW + dw];
                Vec<T, V> y;
                if constexpr (NOID) {
                    // entry (0, 0) has nothing before it in the tile, and a
                    // segment's first tile has nothing before it
                    const bool has_eb = rr > 0 || dw > 0;
#pragma unroll
                    for (int c = 0; c < V; c++) {
                        const T t = has_eb ? Op::apply(eb, x[r].v[c]) : x[r].v[c];
                        y.v[c] = has_pre ? T(Op::apply(pre, C(t))) : t;
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < V; c++) y.v[c] = T(Op::apply(pre, C(Op::apply(eb, x[r].v[c]))));
                }
                // the row step in the vector offset, the scalar offset a
                // constant 0 (see the column single pass: 128-bit buffer
                // stores with a scalar-register offset lost their data
                // registers)
                uint32_t vo = voff + uint32_t(rr) * kRowBytes;
                asm volatile("" : "+v"(vo));
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, y), rs_out[s], vo, 0, OUT_AUX);
            }
        }
    };

    // The control wave and the data waves run separate programs (the branch
    // is uniform within each wave) that meet at the same barriers, so the
    // control wave's code is not compiled around the data waves' tile
    // registers.  Barriers: B1 (the static first tile scanned), Bm (the
    // mode decided), in dynamic mode Bd (the claimed tiles loaded and their
    // first scanned), B2 (the first tile's prefix known; with two tiles,
    // the second scanned, after Bm so that its loads overlap the first
    // look-back), and with two tiles B3 (the second's prefix).
    //
    // With short tiles, the first one's aggregate is published before
    // the residency decision, which waits for every workgroup to start
    // (about 2 us of each call, longer than such a tile's loads), so the
    // look-backs that follow find their predecessors published.  A tile's
    // aggregate depends only on its data, so whoever processes the tile in
    // either mode publishes the same words; only waiting on predecessors
    // needs the decision.  Long first tiles, and the tiles of one-tile grids
    // of few workgroups, decide while they load (measured faster).
    uint32_t tl[SW];  // this workgroup's tiles: static, w (and w + G); dynamic, claim k's SW * k (and SW * k + 1)
    tl[0] = blockIdx.x;
    if constexpr (SW == 2) tl[1] = blockIdx.x + gridDim.x;
    int64_t start0, rem0;
    uint32_t seg0, j0;
    if (ctrl) {
        // short first tiles decide after publishing, long ones (and one-tile
        // grids of few workgroups) while loading
        const bool late = SW == 2 ? rows <= uint32_t(kResLateDecisionRows)
                                  : rows <= uint32_t(kResLateDecisionRows1) && n >= uint32_t(kResLateDecisionTiles);
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
        geom(tl[0], start0, rem0, seg0, j0);
        C agg = scan_entries(0);
        if (tps > 1) publish(tl[0], agg);
        if (lane == 0) {
            if (late) decide();
            s_dyn = dm;
            s_claim = ck;
        }
        dm = uint32_t(__builtin_amdgcn_readlane(int(dm), 0));
        ck = uint32_t(__builtin_amdgcn_readlane(int(ck), 0));
        __syncthreads();  // Bm
        if (dm != 0u) {
            tl[0] = uint32_t(SW) * ck;
            if constexpr (SW == 2) tl[1] = 2u * ck + 1u;
            __syncthreads();  // Bd
            geom(tl[0], start0, rem0, seg0, j0);
            agg = scan_entries(0);
            if (tps > 1) publish(tl[0], agg);
        }
        C pre{};
        if constexpr (!NOID) pre = Op::template identity<C>();
        if (tps > 1 && j0 > 0) pre = gap(tl[0] - j0, tl[0]);
        const C inc0 = j0 > 0 ? C(Op::apply(pre, agg)) : agg;
        if (lane == 0) {
            s_pre[0] = pre;
            if constexpr (!NOID) {
                if (a.total_out != nullptr && j0 == tps - 1) reinterpret_cast<T *>(a.total_out)[seg0] = T(inc0);
            }
        }
        __syncthreads();  // B2
        if constexpr (SW == 2) {
            // Second tile (same segment: whole arrays only): the first
            // tile's inclusive prefix and the aggregates of the tiles
            // between the two, while the data waves store the first tile.
            if (tl[1] < n) {
                const C agg1 = scan_entries(1);
                publish(tl[1], agg1);
                C pre1 = inc0;
                if (tl[1] > tl[0] + 1) pre1 = C(Op::apply(inc0, gap(tl[0] + 1, tl[1])));
                if (lane == 0) {
                    s_pre[1] = pre1;
                    if constexpr (!NOID) {
                        if (a.total_out != nullptr && tl[1] == n - 1)
                            reinterpret_cast<T *>(a.total_out)[0] = T(Op::apply(pre1, agg1));
                    }
                }
            }
            __syncthreads();  // B3
        }
    } else {
        load(tl[0], 0);
        if constexpr (SW == 2) load(tl[1], 1);
        scan_rows(tl[0], 0);
        __syncthreads();  // B1
        __syncthreads();  // Bm
        if (s_dyn != 0u) {
            const uint32_t ck = s_claim;
            tl[0] = uint32_t(SW) * ck;
            if constexpr (SW == 2) tl[1] = 2u * ck + 1u;
            load(tl[0], 0);
            if constexpr (SW == 2) load(tl[1], 1);
            scan_rows(tl[0], 0);
            __syncthreads();  // Bd
        }
        // the second tile is scanned while the control wave looks back for
        // the first (its loads overlap that look-back)
        if constexpr (SW == 2) scan_rows(tl[1], 1);
        geom(tl[0], start0, rem0, seg0, j0);
        __syncthreads();  // B2
        // The first tile's stores wait for the second tile's scan (above):
        // issued earlier, beside the second tile's loads, they slowed those
        // loads, which lead to the last look-back (fp32 1e7: 19.4 -> 22.0 us).
        store(0, s_pre[0], j0 > 0);
        if constexpr (SW == 2) {
            __syncthreads();  // B3
            store(1, s_pre[1], true);
        }
    }
    // end of the call (every thread: the clearing is strided over the
    // workgroup): in static mode every workgroup was counted before the
    // decision; in dynamic mode the holder of the last tile claimed last
    bool last = tl[0] == n - 1;
    if constexpr (SW == 2) last = last || tl[1] == n - 1;
    if (last) end_call(hdr, s_epoch, s_hw, s_cap, a.pipe.words_used, a.pipe.ws_words, desc);
}

template <class T, class Op, int OUT_AUX, bool NOID = false>
static int launch_resident_impl(const ScanArgs &a, int rows, int sweeps, hipStream_t s) {
    constexpr int V = 16 / int(sizeof(T));
    constexpr int MAXR = sizeof(T) == 8 ? kResMaxRows8 : kResMaxRows4;
    constexpr int MAXR2 = sizeof(T) == 8 ? kResMaxRows2x8 : kResMaxRows2x4;  // per tile, two tiles
    const uint32_t n = a.pipe.num_tiles;
    if (rows < 1 || sweeps < 1 || sweeps > 2 || rows > (sweeps == 2 ? MAXR2 : MAXR) || n < 1)
        return SCAN_ERR_UNSUPPORTED;
    const uint32_t grid = (n + uint32_t(sweeps) - 1) / uint32_t(sweeps);
    if (grid > uint32_t(kResMaxTiles)) return SCAN_ERR_UNSUPPORTED;
    if (sweeps == 2 && a.pipe.tiles_per_seg != n) return SCAN_ERR_UNSUPPORTED;  // whole arrays only
    if (NOID && (a.exclusive || a.total_out != nullptr)) return SCAN_ERR_UNSUPPORTED;
    if (sweeps == 2)
        hipLaunchKernelGGL((k_resident<T, Op, V, 2 * MAXR2, OUT_AUX, NOID, 2>), dim3(grid), dim3(kResWaves * kWave), 0,
                           s, a, uint32_t(rows));
    else
        hipLaunchKernelGGL((k_resident<T, Op, V, MAXR, OUT_AUX, NOID, 1>), dim3(grid), dim3(kResWaves * kWave), 0, s,
                           a, uint32_t(rows));
    return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
}

template <class T, bool NOID = false>
static ResLaunch pick_resident(scan_op_t op) {
    switch (op) {
    case SCAN_OP_SUM: return &launch_resident_impl<T, OpSum, 2, NOID>;
    case SCAN_OP_PROD: return &launch_resident_impl<T, OpProd, 2, NOID>;
    case SCAN_OP_MAX: return &launch_resident_impl<T, OpMax, 2, NOID>;
    case SCAN_OP_MIN: return &launch_resident_impl<T, OpMin, 2, NOID>;
    }
    return nullptr;
}

#if SW64_DT == 0
ResLaunch find_resident_i32(scan_op_t op) { return pick_resident<int32_t>(op); }
ResLaunch find_resident_noid_i32(scan_op_t op) { return pick_resident<int32_t, true>(op); }
// count-scan-emit's offsets: stores with the default cache policy, since the
// emit kernel reads them next
ResLaunch find_pack_resident() { return &launch_resident_impl<int32_t, OpSum, 0>; }
#elif SW64_DT == 1
ResLaunch find_resident_u32(scan_op_t op) { return pick_resident<uint32_t>(op); }
ResLaunch find_resident_noid_u32(scan_op_t op) { return pick_resident<uint32_t, true>(op); }
#elif SW64_DT == 2
ResLaunch find_resident_i64(scan_op_t op) { return pick_resident<int64_t>(op); }
ResLaunch find_resident_noid_i64(scan_op_t op) { return pick_resident<int64_t, true>(op); }
#elif SW64_DT == 3
ResLaunch find_resident_f32(scan_op_t op) { return pick_resident<float>(op); }
ResLaunch find_resident_noid_f32(scan_op_t op) { return pick_resident<float, true>(op); }
#elif SW64_DT == 4
ResLaunch find_resident_f64(scan_op_t op) { return pick_resident<double>(op); }
ResLaunch find_resident_noid_f64(scan_op_t op) { return pick_resident<double, true>(op); }
#else
#error "SW64_DT must select an element type (0..4)"
#endif

}  // namespace sw64
