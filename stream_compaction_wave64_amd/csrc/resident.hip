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
template <class T, class Op0, int V, int MAXR, int OUT_AUX, bool NOID = false>
__global__ __launch_bounds__(kResWaves *kWave) void k_resident(ScanArgs a, uint32_t rows) {
    using Op = std::conditional_t<NOID, NoId<Op0>, Op0>;
    using C = typename Carry<T, Op0>::type;
    using D = DescFor<T, C>;
    constexpr int NDW = kResWaves - 1;                       // data waves
    constexpr int RE = NDW * kWave * V;                      // elements per tile row
    constexpr int KE = (MAXR * NDW + kWave - 1) / kWave;     // (row, wave) totals per lane of the control wave
    static_assert(V * sizeof(T) == 16, "128-bit rows");
    __shared__ T ent[MAXR * NDW];        // (row, wave) totals, then their exclusive prefixes in the tile
    __shared__ C s_pre;                  // the tile's exclusive prefix (NOID: none for a segment's first tile)
    __shared__ uint32_t s_epoch, s_tile;
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
    // and drop their stores.
    Vec<T, V> x[MAXR];
    const uint32_t voff = dt * V * uint32_t(sizeof(T));
    constexpr uint32_t kRowBytes = uint32_t(RE) * sizeof(T);
    BufRsrc rs_in, rs_out;
    auto load = [&](uint32_t t) {
        int64_t start, rem;
        uint32_t seg, j;
        geom(t, start, rem, seg, j);
        const int64_t cnt = rem < tile_elems ? rem : tile_elems;
        rs_in = make_rsrc(in + start, cnt);
        rs_out = make_rsrc(out + start, cnt);
#pragma unroll
        for (int r = 0; r < MAXR; r++) {
            if (r < int(rows))
                x[r] = __builtin_bit_cast(Vec<T, V>,
                                          __builtin_amdgcn_raw_buffer_load_b128(rs_in, voff, r * kRowBytes, 2));
        }
    };
    // Each row of the tile: this thread's vector scanned, then across the
    // wave; every value becomes its result within the wave's 64 x V run
    // (inclusive, or exclusive with the identity first), and the wave's row
    // total goes to LDS.  Elements past the segment's end take the identity.
    auto scan_rows = [&](uint32_t t) {
        int64_t start_, rem_;
        uint32_t seg_, j_;
        geom(t, start_, rem_, seg_, j_);
        const int64_t e_thread = int64_t(dt) * V;
#pragma unroll
        for (int r = 0; r < MAXR; r++) {
            if (r < int(rows)) {
                const int64_t e0 = int64_t(r) * RE + e_thread;
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
                    if (lane == kWave - 1) ent[r * NDW + dw] = winc;
                } else {
                    const T id = Op::template identity<T>();
                    const T winc = wave_scan_incl<Op>(acc);
                    const T wex = wave_shr1(id, winc);
#pragma unroll
                    for (int c = 0; c < V; c++)
                        x[r].v[c] =
                            a.exclusive ? (c == 0 ? wex : Op::apply(wex, inc[c - 1])) : Op::apply(wex, inc[c]);
                    if (lane == kWave - 1) ent[r * NDW + dw] = winc;
                }
            }
        }
    };
    // The control wave runs the workspace protocol; the data waves load the
    // static tile and scan it meanwhile (each row as it arrives), and load and
    // scan again after the barrier if a dynamic-mode claim gave the workgroup
    // another tile.
    uint32_t tile = blockIdx.x;
    if (ctrl) {
        uint32_t tk = 0;
        if (lane == 0) {
            uint64_t hw = 0, cap = 0;
            const uint32_t e = begin_call(hdr, hw, cap);
            s_epoch = e;
            s_hw = hw;
            s_cap = cap;
            const uint32_t m = decide_mode(hdr, e, gridDim.x, a.pipe.mode_limit);
            tk = m == kModeStatic
                     ? uint32_t(blockIdx.x)
                     : __hip_atomic_fetch_add(&hdr->claim, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_tile = tk;
        }
        tile = uint32_t(__builtin_amdgcn_readlane(int(tk), 0));
    }
    if (!ctrl) {
        tile = blockIdx.x;
        load(tile);
        scan_rows(tile);
    }
    __syncthreads();
    if (s_tile != blockIdx.x) {
        // dynamic mode gave the workgroup another tile (every wave sees the
        // same s_tile, so all or none take this branch and its barrier)
        tile = s_tile;
        if (!ctrl) {
            load(tile);
            scan_rows(tile);
        }
        __syncthreads();
    }
    const uint32_t epoch = s_epoch;
    int64_t start, rem;
    uint32_t seg, j;
    geom(tile, start, rem, seg, j);
    // Control wave: the (row, wave) totals in tile order (lane l: KE
    // consecutive ones) scanned into their exclusive prefixes; the tile
    // aggregate published; the aggregates of the segment's earlier tiles
    // combined.
    if (ctrl) {
        const uint32_t ne = rows * NDW;
        T e[KE];
        T linc;
        C agg;
        if constexpr (NOID) {
            // lanes past the last entry hold whatever they read; they sit
            // above every lane with entries, so the inclusive scan carries
            // nothing from them down, and the aggregate is the last such
            // lane's result.  Entry 0 has nothing before it: its slot is left
            // as it is (the data waves do not read it).
            T acc = ent[uint32_t(lane) * KE < ne ? uint32_t(lane) * KE : 0u];
#pragma unroll
            for (int k = 0; k < KE; k++) {
                const uint32_t i = uint32_t(lane) * KE + k;
                e[k] = ent[i < ne ? i : 0u];
                if (k > 0 && i < ne) acc = Op::apply(acc, e[k]);
            }
            linc = wave_scan_incl_noid<Op>(acc);
            T run = dpp_mov<kWaveShr1>(linc, linc);
#pragma unroll
            for (int k = 0; k < KE; k++) {
                const uint32_t i = uint32_t(lane) * KE + k;
                if (i < ne) {
                    if (i > 0) ent[i] = run;
                    run = i > 0 ? Op::apply(run, e[k]) : e[k];
                }
            }
            agg = C(wave_read(linc, int((ne - 1) / KE)));
        } else {
            const T id = Op::template identity<T>();
            T acc = id;
#pragma unroll
            for (int k = 0; k < KE; k++) {
                const uint32_t i = uint32_t(lane) * KE + k;
                e[k] = i < ne ? ent[i] : id;
                acc = Op::apply(acc, e[k]);
            }
            linc = wave_scan_incl<Op>(acc);
            T run = wave_shr1(id, linc);
#pragma unroll
            for (int k = 0; k < KE; k++) {
                const uint32_t i = uint32_t(lane) * KE + k;
                if (i < ne) ent[i] = run;
                run = Op::apply(run, e[k]);
            }
            agg = C(wave_read(linc, kWave - 1));
        }
        C pre{};
        if constexpr (!NOID) pre = Op::template identity<C>();
        if (tps > 1) {
            if (a.pipe.delay_stride > 0 && tile % a.pipe.delay_stride == a.pipe.delay_stride - 1) {
                // a late publisher, so tests reach the look-back's re-polls
                for (uint32_t i = 0; i < a.pipe.delay_sleeps; i++) __builtin_amdgcn_s_sleep(64);
            }
            if (lane == 0) D::publish(desc + uint64_t(tile) * D::kWords, epoch, kStateA, agg);
            if (j > 0) {
                if constexpr (NOID) {
                    // j > 0 earlier tiles, all published with a value
                    GapRead<Opt<C>, OptDesc<D>, kResMaxTiles / kWave> g;
                    g.issue(desc, int64_t(tile) - j, int64_t(tile));
                    pre = g.template finish<OptOp<Op0>>(desc, epoch, hdr, a.pipe.spin_limit).v;
                } else {
                    GapRead<C, D, kResMaxTiles / kWave> g;
                    g.issue(desc, int64_t(tile) - j, int64_t(tile));
                    pre = g.template finish<Op>(desc, epoch, hdr, a.pipe.spin_limit);
                }
            }
        }
        if (lane == 0) {
            s_pre = pre;
            if constexpr (!NOID) {
                if (a.total_out != nullptr && j == tps - 1)
                    reinterpret_cast<T *>(a.total_out)[seg] = T(Op::apply(pre, agg));
            }
        }
    }
    __syncthreads();
    const C pre = s_pre;
#pragma unroll
    for (int r = 0; r < MAXR; r++) {
        if (!ctrl && r < int(rows)) {
            const T eb = ent[r * NDW + dw];
            Vec<T, V> y;
            if constexpr (NOID) {
                // entry (0, 0) has nothing before it in the tile, and a
                // segment's first tile has nothing before it
                const bool has_eb = r > 0 || dw > 0;
#pragma unroll
                for (int c = 0; c < V; c++) {
                    const T t = has_eb ? Op::apply(eb, x[r].v[c]) : x[r].v[c];
                    y.v[c] = j > 0 ? T(Op::apply(pre, C(t))) : t;
                }
            } else {
#pragma unroll
                for (int c = 0; c < V; c++) y.v[c] = T(Op::apply(pre, C(Op::apply(eb, x[r].v[c]))));
            }
            // the row step in the vector offset, the scalar offset a constant
            // 0 (see the column single pass: 128-bit buffer stores with a
            // scalar-register offset lost their data registers)
            uint32_t vo = voff + uint32_t(r) * kRowBytes;
            asm volatile("" : "+v"(vo));
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, y), rs_out, vo, 0, OUT_AUX);
        }
    }
    // end of the call: in static mode every workgroup was counted before the
    // decision; in dynamic mode the holder of the last ticket claimed last
    if (tile == n - 1) end_call(hdr, epoch, s_hw, s_cap, a.pipe.words_used, a.pipe.ws_words, desc);
}

template <class T, class Op, int OUT_AUX, bool NOID = false>
static int launch_resident_impl(const ScanArgs &a, int rows, hipStream_t s) {
    constexpr int V = 16 / int(sizeof(T));
    constexpr int MAXR = sizeof(T) == 8 ? kResMaxRows8 : kResMaxRows4;
    if (rows < 1 || rows > MAXR || a.pipe.num_tiles > uint32_t(kResMaxTiles)) return SCAN_ERR_UNSUPPORTED;
    if (NOID && (a.exclusive || a.total_out != nullptr)) return SCAN_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((k_resident<T, Op, V, MAXR, OUT_AUX, NOID>), dim3(a.pipe.num_tiles), dim3(kResWaves * kWave), 0,
                       s, a, uint32_t(rows));
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
