// segmented.hip -- scans of ragged segments: segment s is in[off[s] ..
// off[s+1]) and is scanned on its own (the packed lists of Merry, "Prefix
// sums on GPUs", slides "Output Format" and "Solution", whose offsets
// pack_offsets produces; AcceleratedKernels.jl PR #208's SliceScan with
// segments of any length).
//
// A segmented scan is a plain scan of (head flag, value) pairs under the
// operator that restarts at a head:
//   (fa, a) . (fb, b) = (fa | fb, fb ? b : a (+) b)        (a earlier)
// which is associative but not commutative, so every combination below keeps
// sequence order (the earlier operand on the left).  The structure is
// reduce-then-scan (The CUDA Handbook ch. 13 section 13.3.3), four launches:
//   1. map: for every tile whose first element lies in a segment, that
//      segment's index;
//   2. reduce: each workgroup finds its chunk's last head from the offsets
//      and folds only the elements from there to the chunk's end into one
//      (flag, value) partial (everything before a head is discarded);
//   3. partials: one workgroup scans the partials in order into each chunk's
//      exclusive prefix;
//   4. rescan: each workgroup scans its chunk, tile by tile, carrying the
//      prefix into the elements before the first head it meets.
// The rescan learns a tile's heads from the offsets: from the map it reads
// the segments that can start inside the tile and marks their starts in an
// LDS byte map, so no per-element flag array is ever materialised in HBM and
// the offsets are read once.  Traffic: one read of the data (plus the
// elements after each chunk's last head) and one write, one read of the
// offsets.
//
// Workspace: the map (one 64-bit word per tile, the index as a value below
// 2^32: a look-back descriptor reader sees such a word as unpublished, so it
// may stay), the head planes of the single pass (likewise below 2^32) and
// the chunk partials (zeroed by the rescan, as the other reduce-then-scan
// kernels leave theirs).
//
// Compiled once per element type (SW64_DT).
#include "launch.hpp"
#include "tile.hpp"

namespace sw64 {

template <class V>
struct SegVal {
    using value_type = V;
    V v;
    uint32_t f;  // a segment head lies in the combined range
};

template <class Op, class V>
__device__ __forceinline__ SegVal<V> seg_combine(const SegVal<V> &a, const SegVal<V> &b) {
    return {b.f ? b.v : Op::apply(a.v, b.v), a.f | b.f};
}

template <class Op, class V>
__device__ __forceinline__ SegVal<V> seg_identity() {
    return {Op::template identity<V>(), 0u};
}

// Inclusive segmented scan across the 64 lanes in lane order: the DPP
// Kogge-Stone rounds of wave_scan_incl (shift 1, 2, 4, 8 inside each
// 16-lane row, then lane 15 and lane 31 broadcasts), moving the value and the
// flag.  A lane whose source lies outside its row receives the identity pair
// (identity, no head), which combines as a no-op, as in the plain scan.
template <int CTRL, int ROW_MASK, class Op, class V>
__device__ __forceinline__ SegVal<V> seg_dpp_round(const SegVal<V> &x) {
    const SegVal<V> p{dpp_mov<CTRL, ROW_MASK>(Op::template identity<V>(), x.v), dpp_mov<CTRL, ROW_MASK>(0u, x.f)};
    return seg_combine<Op, V>(p, x);
}

template <class Op, class V>
__device__ __forceinline__ SegVal<V> wave_seg_scan_incl(SegVal<V> x) {
    x = seg_dpp_round<kRowShr1, 0xf, Op>(x);
    x = seg_dpp_round<kRowShr2, 0xf, Op>(x);
    x = seg_dpp_round<kRowShr4, 0xf, Op>(x);
    x = seg_dpp_round<kRowShr8, 0xf, Op>(x);
    x = seg_dpp_round<kRowBcast15, 0xa, Op>(x);
    x = seg_dpp_round<kRowBcast31, 0xc, Op>(x);
    return x;
}

// The lane before's inclusive value (the identity pair in lane 0).
template <class Op, class V>
__device__ __forceinline__ SegVal<V> wave_seg_shr1(const SegVal<V> &inc) {
    return SegVal<V>{wave_shr1(Op::template identity<V>(), inc.v), wave_shr1(0u, inc.f)};
}

// A tile of ROWS rows of B * VEC elements, laid out as TileScan's: thread t
// holds vector (r * B + t) of row r.
// PRELOAD: the scan reads a row's per-wave totals from LDS all at once
// before folding them (the single pass, where one workgroup per compute
// unit leaves the dependent reads exposed); otherwise one at a time (fewer
// registers, for the many-workgroup rescan).
template <class T, class Op, int B, int ROWS, int VEC, bool PRELOAD = false>
struct SegTile {
    using C = typename Carry<T, Op>::type;
    static constexpr int W = B / kWave;
    static constexpr int64_t TILE = int64_t(B) * ROWS * VEC;
    static_assert(TILE % 16 == 0 && ROWS * VEC <= 32, "16-byte clears of the head map, per-thread head bits");

    struct Shared {
        T tv[ROWS][W];  // per row and wave: inclusive segmented total
        uint32_t tf[ROWS][W];
    };
    struct Marks {
        alignas(16) uint8_t heads[TILE];  // nonzero: element e of the tile starts a segment
    };

    Vec<T, VEC> v[ROWS];
    uint32_t head;    // bit r*VEC+c: this thread's element starts a segment
    int64_t rem;      // elements of the tile in range
    SegVal<T> agg;    // tile aggregate

    __device__ __forceinline__ static int64_t elem(int r) { return (int64_t(r) * B + threadIdx.x) * VEC; }

    // Whole tiles load whole vectors; the last, partial tile loads element
    // by element (any n works with vector access; the identity fills the
    // rest).
    __device__ __forceinline__ void load(const T *src, int64_t remaining) {
        rem = remaining;
        const T id = Op::template identity<T>();
        if (remaining >= TILE) {
#pragma unroll
            for (int r = 0; r < ROWS; r++) v[r] = load_vec<T, VEC>(src + elem(r));
            return;
        }
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            const int64_t e = elem(r);
#pragma unroll
            for (int c = 0; c < VEC; c++) v[r].v[c] = e + c < remaining ? src[e + c] : id;
        }
    }

    // Mark the heads of tile t (elements [t0, t0 + TILE)) in LDS and read
    // this thread's.  The segments that can start in the tile are s0 (the
    // one holding t0) up to s1 (the one holding the next tile's first
    // element; nseg for the last tile), both clamped to nseg by the caller,
    // so invalid offsets give wrong results, never an access out of bounds.
    // A head is one byte in LDS written with a plain store (empty segments
    // write the same byte again), so no atomics: consecutive segment starts
    // a few elements apart would otherwise contend for the same word.  Each
    // thread issues its offset loads kMarkBatch at a time.  Contains two
    // barriers.
    static constexpr int kMarkBatch = 8;
    __device__ __forceinline__ void mark(Marks &sh, const SegArgs &a, uint32_t t, uint64_t s0, uint64_t s1) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        for (int i = threadIdx.x; i < int(TILE / 16); i += B)
            reinterpret_cast<u32x4 *>(sh.heads)[i] = u32x4{0u, 0u, 0u, 0u};
        __syncthreads();
        const int32_t t0 = int32_t(int64_t(t) * TILE);  // n <= INT32_MAX
        for (uint64_t base = s0 + threadIdx.x; base <= s1; base += uint64_t(kMarkBatch) * B) {
            int32_t o[kMarkBatch];  // offsets and tile starts are in [0, 2^31): the difference fits
            // unconditional loads (indices clamped to s1, a valid offset), so
            // the batch is in flight at once rather than one branch per load
#pragma unroll
            for (int u = 0; u < kMarkBatch; u++) {
                const uint64_t s = base + uint64_t(u) * B;
                o[u] = a.off[s <= s1 ? s : s1];
            }
#pragma unroll
            for (int u = 0; u < kMarkBatch; u++) o[u] = base + uint64_t(u) * B <= s1 ? o[u] - t0 : -1;
#pragma unroll
            for (int u = 0; u < kMarkBatch; u++)
                if (o[u] >= 0 && o[u] < TILE && o[u] < rem) sh.heads[o[u]] = 1;
        }
        __syncthreads();
        head = 0;
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            const int64_t e = elem(r);
            uint32_t bytes;  // this thread's VEC head bytes of row r, one LDS read
            if constexpr (VEC == 4) bytes = *reinterpret_cast<const uint32_t *>(sh.heads + e);
            else if constexpr (VEC == 2) bytes = *reinterpret_cast<const uint16_t *>(sh.heads + e);
            else bytes = sh.heads[e];
#pragma unroll
            for (int c = 0; c < VEC; c++) head |= uint32_t(((bytes >> (8 * c)) & 0xffu) != 0u) << (r * VEC + c);
        }
    }

    // This thread's head bits from an LDS byte map of the tile's elements
    // (nonzero: the element starts a segment).
    __device__ __forceinline__ void heads_from_map(const uint8_t *hm) {
        head = 0;
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            const int64_t e = elem(r);
            uint32_t bytes;  // this thread's VEC head bytes of row r, one LDS read
            if constexpr (VEC == 4) bytes = *reinterpret_cast<const uint32_t *>(hm + e);
            else if constexpr (VEC == 2) bytes = *reinterpret_cast<const uint16_t *>(hm + e);
            else bytes = hm[e];
#pragma unroll
            for (int c = 0; c < VEC; c++) head |= uint32_t(((bytes >> (8 * c)) & 0xffu) != 0u) << (r * VEC + c);
        }
    }

    // The tile's head bits for the rescan, as bit planes: plane j of wave w
    // holds bit j (row j / VEC, element j % VEC) of each lane's head mask, a
    // 64-lane ballot stored as two words holding 32 lanes each; a wave's
    // planes are contiguous, written by one store instruction.  Every word
    // stays below 2^32, which a look-back reader of a later call on this
    // workspace sees as unpublished, so the planes may stay.  TILE / 4 bytes
    // per tile.
    static constexpr int kPlanes = ROWS * VEC;
    static constexpr int64_t kPlaneWords = int64_t(kPlanes) * W * 2;
    __device__ __forceinline__ void save_heads(uint64_t *planes) const {
        const int wave = threadIdx.x / kWave, lane = lane_id();
        // one ballot per plane, stored at once by lane 0 (so the ballots do
        // not all stay live in scalar registers)
        uint64_t *dst = planes + int64_t(wave) * 2 * kPlanes;
#pragma unroll
        for (int j = 0; j < kPlanes; j++) {
            const uint64_t m = __ballot((head >> j) & 1u);
            if (lane == 0) {
                __builtin_nontemporal_store(m & 0xffffffffu, dst + 2 * j);
                __builtin_nontemporal_store(m >> 32, dst + 2 * j + 1);
            }
        }
    }

    // The plane words holding this lane's bits, loaded only (for a pipeline
    // that prefetches the next tile: computing the mask at once would wait
    // for the loads), and the mask from them.
    __device__ __forceinline__ static void issue_heads(const uint64_t *planes, uint32_t (&pw)[kPlanes]) {
        const uint32_t *p32 = reinterpret_cast<const uint32_t *>(planes);
        const int wave = threadIdx.x / kWave, lane = lane_id();
#pragma unroll
        for (int j = 0; j < kPlanes; j++) pw[j] = p32[((int64_t(wave) * kPlanes + j) * 2 + (lane >> 5)) * 2];
    }
    __device__ __forceinline__ void heads_from(const uint32_t (&pw)[kPlanes]) {
        const int lane = lane_id();
        head = 0;
#pragma unroll
        for (int j = 0; j < kPlanes; j++) head |= ((pw[j] >> (lane & 31)) & 1u) << j;
    }

    // This thread's head mask from the planes save_heads() wrote (the
    // addresses are uniform across the wave).
    __device__ __forceinline__ void load_heads(const uint64_t *planes) {
        const uint32_t wave = uniform(uint32_t(threadIdx.x / kWave));
        const int lane = lane_id();
        uint64_t w[kPlanes];
#pragma unroll
        for (int j = 0; j < kPlanes; j++) w[j] = planes[(int64_t(wave) * kPlanes + j) * 2 + (lane >> 5)];
        head = 0;
#pragma unroll
        for (int j = 0; j < kPlanes; j++) head |= uint32_t((w[j] >> (lane & 31)) & 1u) << j;
    }

    // Scan the tile within itself; afterwards v holds, per element, the
    // segmented inclusive value (or exclusive with `exclusive`) counted from
    // the tile's start, `cov` the elements with a head at or before them in
    // the tile (they ignore any carry), and agg the tile's aggregate.
    // Contains one barrier; the caller separates reuses of sh.
    __device__ __forceinline__ void scan(Shared &sh, bool exclusive, uint32_t &cov) {
        const int wave = threadIdx.x / kWave;
        SegVal<T> ex[ROWS];  // per row: the segmented value before this thread's vector, within its wave
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            SegVal<T> run = seg_identity<Op, T>();
#pragma unroll
            for (int c = 0; c < VEC; c++)
                run = seg_combine<Op, T>(run, SegVal<T>{v[r].v[c], (head >> (r * VEC + c)) & 1u});
            const SegVal<T> inc = wave_seg_scan_incl<Op, T>(run);
            if (lane_id() == kWave - 1) {
                sh.tv[r][wave] = inc.v;
                sh.tf[r][wave] = inc.f;
            }
            ex[r] = wave_seg_shr1<Op, T>(inc);
        }
        __syncthreads();
        SegVal<T> run = seg_identity<Op, T>();
        cov = 0;
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            SegVal<T> base = run;  // everything before this row, then before this wave
            if constexpr (PRELOAD) {
                SegVal<T> x[W];
#pragma unroll
                for (int w = 0; w < W; w++) x[w] = SegVal<T>{sh.tv[r][w], sh.tf[r][w]};
#pragma unroll
                for (int w = 0; w < W; w++) {
                    if (w < wave) base = seg_combine<Op, T>(base, x[w]);
                    run = seg_combine<Op, T>(run, x[w]);
                }
            } else {
#pragma unroll 1
                for (int w = 0; w < W; w++) {
                    const SegVal<T> x{sh.tv[r][w], sh.tf[r][w]};
                    if (w < wave) base = seg_combine<Op, T>(base, x);
                    run = seg_combine<Op, T>(run, x);
                }
            }
            SegVal<T> prev = seg_combine<Op, T>(base, ex[r]);  // before this thread's vector
#pragma unroll
            for (int c = 0; c < VEC; c++) {
                const SegVal<T> x{v[r].v[c], (head >> (r * VEC + c)) & 1u};
                const SegVal<T> inc = seg_combine<Op, T>(prev, x);
                const SegVal<T> out = exclusive ? (x.f ? SegVal<T>{Op::template identity<T>(), 1u} : prev) : inc;
                v[r].v[c] = out.v;
                cov |= out.f << (r * VEC + c);
                prev = inc;
            }
        }
        agg = run;
    }

    // Only the aggregate (the reduce pass).  Contains one barrier.
    __device__ __forceinline__ void reduce(Shared &sh) {
        const int wave = threadIdx.x / kWave;
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            SegVal<T> run = seg_identity<Op, T>();
#pragma unroll
            for (int c = 0; c < VEC; c++)
                run = seg_combine<Op, T>(run, SegVal<T>{v[r].v[c], (head >> (r * VEC + c)) & 1u});
            const SegVal<T> inc = wave_seg_scan_incl<Op, T>(run);
            if (lane_id() == kWave - 1) {
                sh.tv[r][wave] = inc.v;
                sh.tf[r][wave] = inc.f;
            }
        }
        __syncthreads();
        SegVal<T> run = seg_identity<Op, T>();
        for (int r = 0; r < ROWS; r++)
            for (int w = 0; w < W; w++) run = seg_combine<Op, T>(run, SegVal<T>{sh.tv[r][w], sh.tf[r][w]});
        agg = run;
    }

    // Store: elements without a head at or before them in the tile get the
    // carry in front (in the carry type, rounded once).
    // (Whole vectors for whole tiles, element by element in the last one.)
    __device__ __forceinline__ void store(T *dst, int64_t remaining, C carry, uint32_t cov) const {
        const BufRsrc rs = make_rsrc(dst, remaining < TILE ? (remaining > 0 ? remaining : 0) : TILE);
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            Vec<T, VEC> o;
#pragma unroll
            for (int c = 0; c < VEC; c++) {
                const bool own = (cov >> (r * VEC + c)) & 1u;
                o.v[c] = own ? v[r].v[c] : T(Op::apply(carry, C(v[r].v[c])));
            }
            if (remaining >= TILE) {
                store_vec_bounded<T, VEC>(rs, uint32_t(elem(r) * int64_t(sizeof(T))), o);
            } else {
#pragma unroll
                for (int c = 0; c < VEC; c++)
                    store_vec_bounded<T, 1>(rs, uint32_t((elem(r) + c) * int64_t(sizeof(T))), Vec<T, 1>{{o.v[c]}});
            }
        }
    }
};

// Pass 1: the tile -> segment map (templated on T only so that each element
// type's unit has its own instance; POW2: tiles are a power of two long).
// Each thread takes kMapSegs consecutive segments, whose kMapSegs + 1
// offsets it loads at once (one 16-byte load when aligned), so a thread
// waits for one round trip.
constexpr int kMapSegs = 4;

template <class T, bool POW2>
__global__ __launch_bounds__(256) void k_seg_map(SegArgs a) {
    typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
    static_assert(kMapSegs == 4, "one 16-byte load of offsets");
    const bool vec = (reinterpret_cast<uintptr_t>(a.off) & 15u) == 0;
    for (int64_t s0 = (int64_t(blockIdx.x) * 256 + threadIdx.x) * kMapSegs; s0 < a.nseg;
         s0 += int64_t(gridDim.x) * 256 * kMapSegs) {
        int32_t o[kMapSegs + 1];
        if (vec && s0 + kMapSegs <= a.nseg) {
            const i32x4 v = *reinterpret_cast<const i32x4 *>(a.off + s0);
            o[0] = v.x;
            o[1] = v.y;
            o[2] = v.z;
            o[3] = v.w;
            o[4] = a.off[s0 + kMapSegs];
        } else {
#pragma unroll
            for (int i = 0; i <= kMapSegs; i++) o[i] = s0 + i <= a.nseg ? a.off[s0 + i] : 0;
        }
#pragma unroll
        for (int i = 0; i < kMapSegs; i++) {
            const int64_t b = o[i], e = o[i + 1];
            if (s0 + i >= a.nseg || e <= b || b < 0) continue;
            // the first tile starting at or after b, and on while tiles start
            // before e (a shift for power-of-two tiles, else a 32-bit
            // division: offsets and the tile size are below 2^31)
            const uint32_t tile = uint32_t(a.tile);
            int64_t t0;
            if constexpr (POW2)
                t0 = int64_t((uint32_t(b) + tile - 1u) >> a.tile_log2);
            else
                t0 = int64_t((uint32_t(b) + tile - 1u) / tile);
            for (int64_t t = t0; t * a.tile < e && t < int64_t(a.num_tiles); t++) a.map[t] = uint64_t(s0 + i);
        }
    }
}

// The map entries a chunk's tiles need (its tiles and the next one), read
// once into LDS when they fit, each clamped to nseg.
constexpr int kSegMapCache = 64;

struct SegChunkMap {
    uint64_t m[kSegMapCache + 1];

    __device__ __forceinline__ void load(const SegArgs &a, uint64_t t0, uint64_t t1) {
        if (t1 - t0 <= uint64_t(kSegMapCache)) {
            for (uint64_t i = threadIdx.x; i <= t1 - t0; i += blockDim.x) {
                const uint64_t t = t0 + i;
                const uint64_t v = t < a.num_tiles ? a.map[t] : uint64_t(a.nseg);
                m[i] = v < uint64_t(a.nseg) ? v : uint64_t(a.nseg);
            }
        }
        __syncthreads();
    }
    __device__ __forceinline__ uint64_t get(const SegArgs &a, uint64_t t0, uint64_t t1, uint64_t t) const {
        if (t1 - t0 <= uint64_t(kSegMapCache)) return m[t - t0];
        const uint64_t v = t < a.num_tiles ? a.map[t] : uint64_t(a.nseg);
        return v < uint64_t(a.nseg) ? v : uint64_t(a.nseg);
    }
};

template <class T, class Op>
struct SegPartial {
    typename Carry<T, Op>::type v;
    uint32_t f, pad;
};

// Pass 2.  A chunk's partial depends only on its elements from its last
// head on: under the segmented operator a head discards everything before
// it, so the partial is (1, the fold of the elements from the last head to
// the chunk's end), or (0, the fold of the whole chunk) when no segment
// starts in it.  The last head is the start of the last segment starting at
// or before the chunk's last element; the offsets being non-decreasing, it
// is found among the segments the map gives for the chunk's last tile (the
// one holding its first element up to the one holding the next tile's), all
// read at once.  Then only the elements from that head on are read: with
// short segments a few per chunk instead of the whole chunk (Poisson(3)
// segments of 3e7 fp32: the pass that folded every tile read all 120 MB at
// 3.3 TB/s, 37.6 us).  The heads themselves are marked by the rescan.
template <class T, class Op, int B, int R, int V>
__global__ __launch_bounds__(B) void k_seg_reduce(SegArgs a) {
    using ST = SegTile<T, Op, B, R, V>;
    using C = typename ST::C;
    __shared__ int64_t s_last;  // index of the last segment starting at or before the chunk's end, or -1
    __shared__ C s_part[B / kWave];
    const uint64_t t0 = uint64_t(blockIdx.x) * a.chunk_tiles;
    const uint64_t t1 = t0 + a.chunk_tiles < a.num_tiles ? t0 + a.chunk_tiles : a.num_tiles;
    const int64_t e0 = int64_t(t0) * ST::TILE;                                          // the chunk's start
    const int64_t e1 = int64_t(t1) * ST::TILE < a.n ? int64_t(t1) * ST::TILE : a.n;  // and end
    auto seg_at = [&](uint64_t t) -> int64_t {  // the map: segment holding tile t's first element (clamped)
        const uint64_t v = t < a.num_tiles ? a.map[t] : uint64_t(a.nseg);
        return int64_t(v < uint64_t(a.nseg) ? v : uint64_t(a.nseg));
    };
    if (threadIdx.x == 0) s_last = -1;
    __syncthreads();
    {
        const int64_t lo = seg_at(t1 - 1), hi = seg_at(t1);  // candidates [lo, hi], within [0, nseg]
        int64_t best = -1;
        for (int64_t sidx = lo + threadIdx.x; sidx <= hi && sidx < a.nseg; sidx += B) {
            if (int64_t(a.off[sidx]) <= e1 - 1) best = sidx;  // non-decreasing: the last such is the largest
        }
        const int64_t wb = wave_reduce<OpMax>(best);
        if (lane_id() == 0 && wb >= 0) __hip_atomic_fetch_max(&s_last, wb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();
    const int64_t sl = s_last;
    const int64_t h = sl >= 0 ? int64_t(a.off[sl]) : -1;  // the last head at or before the chunk's end
    const bool has = h >= e0 && h < e1;
    const int64_t from = has ? h : e0;
    const T *in = reinterpret_cast<const T *>(a.in);
    C acc = Op::template identity<C>();
#pragma unroll 4
    for (int64_t i = from + threadIdx.x; i < e1; i += B) acc = Op::apply(acc, C(in[i]));
    acc = wave_reduce<Op>(acc);
    if (lane_id() == 0) s_part[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        C v = Op::template identity<C>();
        for (int w = 0; w < B / kWave; w++) v = Op::apply(v, s_part[w]);
        SegPartial<T, Op> *p = reinterpret_cast<SegPartial<T, Op> *>(a.partials);
        p[blockIdx.x].v = v;
        p[blockIdx.x].f = has ? 1u : 0u;
    }
}

// Pass 3: one workgroup of 1024 threads scans the chunk partials in order;
// thread k owns a run of up to kSegPartPer consecutive chunks.
constexpr int kSegPartThreads = 1024, kSegPartPer = 8;

template <class T, class Op>
__global__ __launch_bounds__(kSegPartThreads) void k_seg_partials(SegArgs a) {
    using C = typename Carry<T, Op>::type;
    __shared__ C wv[kSegPartThreads / kWave];
    __shared__ uint32_t wf[kSegPartThreads / kWave];
    SegPartial<T, Op> *p = reinterpret_cast<SegPartial<T, Op> *>(a.partials);
    const uint32_t per = (a.blocks + kSegPartThreads - 1) / kSegPartThreads;  // <= kSegPartPer
    const uint32_t c0 = threadIdx.x * per;
    SegVal<C> x[kSegPartPer];
    SegVal<C> run = seg_identity<Op, C>();
#pragma unroll
    for (int i = 0; i < kSegPartPer; i++) {
        x[i] = seg_identity<Op, C>();
        if (uint32_t(i) < per && c0 + i < a.blocks) x[i] = SegVal<C>{p[c0 + i].v, p[c0 + i].f};
        run = seg_combine<Op, C>(run, x[i]);
    }
    const int wave = threadIdx.x / kWave;
    const SegVal<C> inc = wave_seg_scan_incl<Op, C>(run);
    if (lane_id() == kWave - 1) {
        wv[wave] = inc.v;
        wf[wave] = inc.f;
    }
    __syncthreads();
    SegVal<C> pre = seg_identity<Op, C>();
    for (int w = 0; w < wave; w++) pre = seg_combine<Op, C>(pre, SegVal<C>{wv[w], wf[w]});
    pre = seg_combine<Op, C>(pre, wave_seg_shr1<Op, C>(inc));
#pragma unroll
    for (int i = 0; i < kSegPartPer; i++) {
        if (uint32_t(i) < per && c0 + i < a.blocks) {
            p[c0 + i].v = pre.v;  // the value carried into the chunk
            p[c0 + i].f = pre.f;
            pre = seg_combine<Op, C>(pre, x[i]);
        }
    }
}

// Pass 4.  The heads of up to kSegMarkTiles tiles are marked at once (one
// batch of offset loads per group: marking tile by tile put a dependent round
// trip and two barriers before every tile's scan), then each tile is scanned
// with the carry and stored.  The next tile's values are loaded while the
// current one is marked, scanned and stored (unconditional buffer loads, a
// range of zero when there is no next tile), so the tiles of a chunk do not
// each wait a full load latency.
constexpr int kSegMarkTiles = 8;

template <class T, class Op, int B, int R, int V>
__global__ __launch_bounds__(B) void k_seg_rescan(SegArgs a) {
    using ST = SegTile<T, Op, B, R, V>;
    using C = typename ST::C;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    __shared__ typename ST::Shared sh;
    __shared__ alignas(16) uint8_t hm[kSegMarkTiles * ST::TILE];  // the group's heads, one byte per element
    __shared__ SegChunkMap cm;
    __shared__ C s_carry;
    SegPartial<T, Op> *p = reinterpret_cast<SegPartial<T, Op> *>(a.partials);
    if (threadIdx.x == 0) s_carry = p[blockIdx.x].v;
    __syncthreads();
    C carry = s_carry;
    if (threadIdx.x == 0) p[blockIdx.x] = SegPartial<T, Op>{};  // leave the workspace zeroed
    const uint64_t t0 = uint64_t(blockIdx.x) * a.chunk_tiles;
    const uint64_t t1 = t0 + a.chunk_tiles < a.num_tiles ? t0 + a.chunk_tiles : a.num_tiles;
    cm.load(a, t0, t1);
    ST st;
    constexpr int VB = V * int(sizeof(T));  // bytes per vector
    static_assert(VB == 4 || VB == 8 || VB == 16, "vector access of 4, 8 or 16 bytes");
    Vec<T, V> nv[R];  // the next tile's values
    auto fetch = [&](uint64_t t) {
        const bool valid = t < t1;
        const int64_t start = valid ? int64_t(t) * ST::TILE : 0;
        const int64_t left = a.n - start;
        const BufRsrc rs =
            make_rsrc(reinterpret_cast<const T *>(a.in) + start, valid ? (left < ST::TILE ? left : ST::TILE) : 0);
#pragma unroll
        for (int r = 0; r < R; r++) {
            const uint32_t off = uint32_t(ST::elem(r) * int64_t(sizeof(T)));
            if constexpr (VB == 16)
                nv[r] = __builtin_bit_cast(Vec<T, V>, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 2));
            else if constexpr (VB == 8)
                nv[r] = __builtin_bit_cast(Vec<T, V>, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 2));
            else
                nv[r] = __builtin_bit_cast(Vec<T, V>, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 2));
        }
    };
    fetch(t0);
    for (uint64_t g0 = t0; g0 < t1; g0 += kSegMarkTiles) {
        const uint64_t g1 = g0 + kSegMarkTiles < t1 ? g0 + kSegMarkTiles : t1;
        const int64_t eg0 = int64_t(g0) * ST::TILE;
        const int64_t span = (int64_t(g1) * ST::TILE < a.n ? int64_t(g1) * ST::TILE : a.n) - eg0;  // elements in range
        for (int i = threadIdx.x; i < int((g1 - g0) * ST::TILE / 16); i += B)
            reinterpret_cast<u32x4 *>(hm)[i] = u32x4{0u, 0u, 0u, 0u};
        __syncthreads();
        // the segments that can start in the group: the one holding its first
        // element up to the one holding the next group's (clamped to nseg by
        // the map), so invalid offsets give wrong results, never an access
        // out of bounds
        const uint64_t s0 = cm.get(a, t0, t1, g0), s1 = cm.get(a, t0, t1, g1);
        const int32_t eg0_32 = int32_t(eg0);  // n <= INT32_MAX: offsets and group starts fit, so does their difference
        for (uint64_t base = s0 + threadIdx.x; base <= s1; base += uint64_t(ST::kMarkBatch) * B) {
            int32_t o[ST::kMarkBatch];
#pragma unroll
            for (int u = 0; u < ST::kMarkBatch; u++) {
                const uint64_t sidx = base + uint64_t(u) * B;
                o[u] = a.off[sidx <= s1 ? sidx : s1];
            }
#pragma unroll
            for (int u = 0; u < ST::kMarkBatch; u++) {
                const int32_t d = base + uint64_t(u) * B <= s1 ? o[u] - eg0_32 : -1;
                if (d >= 0 && d < span) hm[d] = 1;
            }
        }
        __syncthreads();
        for (uint64_t t = g0; t < g1; t++) {
            const int64_t start = int64_t(t) * ST::TILE;
            // a whole tile takes the prefetched values; the array's last,
            // partial tile (a vector may cross its end) is loaded element by
            // element as before
            if (a.n - start >= ST::TILE) {
                st.rem = a.n - start;
#pragma unroll
                for (int r = 0; r < R; r++) st.v[r] = nv[r];
            } else {
                st.load(reinterpret_cast<const T *>(a.in) + start, a.n - start);
            }
            fetch(t + 1);
            st.heads_from_map(hm + (t - g0) * ST::TILE);
            uint32_t cov;
            st.scan(sh, a.exclusive != 0, cov);
            st.store(reinterpret_cast<T *>(a.out) + start, a.n - start, carry, cov);
            carry = st.agg.f ? C(st.agg.v) : Op::apply(carry, C(st.agg.v));
            __syncthreads();
        }
    }
}

// ------------------------------------------------------------ single pass
// The same scan on the persistent look-back pipeline (pipeline.hpp): one
// read and one write of the data.  The carry between tiles is a (head flag,
// value) pair under the restarting operator, which the look-back combines in
// tile order (kOrderedOp).  Heads come from a heads pass (the marking of the
// reduce-then-scan rescan, without the data) as bit planes, laid out for the
// pipeline's data threads; the map pass runs first as before.

template <class BaseOp>
struct SegOp {
    static constexpr bool kOrdered = true;
    template <class X>
    __device__ __forceinline__ static X identity() {
        return X{BaseOp::template identity<typename X::value_type>(), 0u};
    }
    template <class X>
    __device__ __forceinline__ static X apply(const X &a, const X &b) {
        return seg_combine<BaseOp, typename X::value_type>(a, b);
    }
};

// A (flag, value) descriptor: the value in 32-bit chunks, one per word as
// Desc<C> does, and the flag in bit 32 of the first word (the payload has 54
// bits); accepted only when every word carries the same tag.
template <class V>
struct SegDesc {
    static constexpr int kWords = int(sizeof(V) / 4);
    struct Chunks { uint32_t w[kWords]; };

    __device__ __forceinline__ static void publish(uint64_t *d, uint32_t epoch, uint32_t state, SegVal<V> x) {
        const Chunks c = __builtin_bit_cast(Chunks, x.v);
        const uint64_t tag = desc_tag(epoch, state);
#pragma unroll
        for (int i = 0; i < kWords; i++) {
            const uint64_t flag = i == 0 ? uint64_t(x.f & 1u) << 32 : 0;
            __hip_atomic_store(d + i, tag | flag | c.w[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __device__ __forceinline__ static void fetch(const uint64_t *d, uint64_t (&w)[kWords]) {
#pragma unroll
        for (int i = 0; i < kWords; i++) w[i] = __hip_atomic_load(d + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __device__ __forceinline__ static uint32_t decode(const uint64_t (&w)[kWords], uint32_t epoch, SegVal<V> &x) {
        const uint32_t state = desc_state(w[0], epoch);
        bool ok = state != 0u;
        Chunks c;
#pragma unroll
        for (int i = 0; i < kWords; i++) {
            ok = ok && (w[i] >> kTagShift) == (w[0] >> kTagShift);
            c.w[i] = uint32_t(w[i]);
        }
        x.v = __builtin_bit_cast(V, c);
        x.f = uint32_t(w[0] >> 32) & 1u;
        return ok ? state : 0u;
    }
    __device__ __forceinline__ static uint32_t read(const uint64_t *d, uint32_t epoch, SegVal<V> &x) {
        uint64_t w[kWords];
        fetch(d, w);
        return decode(w, epoch, x);
    }
};

template <class T, class BaseOp, int BLOCK_, int ROWS, int VEC>
struct SegScanPolicy {
    using ST = SegTile<T, BaseOp, BLOCK_, ROWS, VEC, true>;
    using V = typename ST::C;  // carry value type
    using C = SegVal<V>;
    using Op = SegOp<BaseOp>;
    using D = SegDesc<V>;
    using Args = SegArgs;
    using Shared = typename ST::Shared;
    static constexpr int kDescWords = D::kWords;
    static constexpr int BLOCK = BLOCK_;

    // The tile's (flag, value) aggregate: rows, then waves, in order.
    __device__ __forceinline__ static C aggregate(const Shared &sh) {
        SegVal<T> run = seg_identity<BaseOp, T>();
        for (int r = 0; r < ROWS; r++)
            for (int w = 0; w < ST::W; w++) run = seg_combine<BaseOp, T>(run, SegVal<T>{sh.tv[r][w], sh.tf[r][w]});
        return C{V(run.v), run.f};
    }

    // A scanned tile waiting for its prefix: the tile-local results and
    // which of them have a head at or before them (own slots only).
    struct Stash {
        Vec<T, VEC> v[ROWS][BLOCK];
        uint32_t cov[BLOCK];
    };

    static constexpr bool kSetup = false;
    __device__ __forceinline__ static C setup(const Args &, const uint64_t *, uint32_t, WsHeader *) { return C{}; }

    // Elements with no head at or before them in the tile take the carry in
    // front (in the carry type, rounded once).
    __device__ __forceinline__ static void emit(const Stash &st, const Args &a, uint32_t tile, C pre, bool valid,
                                                C) {
        if (!valid) return;
        const int64_t start = int64_t(tile) * ST::TILE, remaining = a.n - start;
        T *dst = reinterpret_cast<T *>(a.out) + start;
        const BufRsrc rs = make_rsrc(dst, remaining < ST::TILE ? remaining : ST::TILE);
        const uint32_t cov = st.cov[threadIdx.x];
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            Vec<T, VEC> o = st.v[r][threadIdx.x];
#pragma unroll
            for (int c = 0; c < VEC; c++) {
                if (!((cov >> (r * VEC + c)) & 1u)) o.v[c] = T(BaseOp::apply(pre.v, V(o.v[c])));
            }
            if (remaining >= ST::TILE) {
                store_vec_bounded<T, VEC>(rs, uint32_t(ST::elem(r) * int64_t(sizeof(T))), o);
            } else {
#pragma unroll
                for (int c = 0; c < VEC; c++)
                    store_vec_bounded<T, 1>(rs, uint32_t((ST::elem(r) + c) * int64_t(sizeof(T))), Vec<T, 1>{{o.v[c]}});
            }
        }
    }

    __device__ __forceinline__ static void on_resolved(const Args &, uint32_t, C, C) {}

    struct Tile {
        ST st;
        uint32_t pw[ST::kPlanes];  // this lane's plane words, loaded with the data
        uint32_t cov;
        bool excl;

        // A tile past the end (the pipeline's prefetch) loads tile 0's data
        // and planes and is never scanned.  Loads are only issued here; the
        // head mask is formed in scan(), once the tile is due.
        __device__ __forceinline__ void load(const Args &a, uint32_t tile) {
            const bool valid = tile < a.pipe.num_tiles;
            const uint32_t t = valid ? tile : 0u;
            const int64_t start = int64_t(t) * ST::TILE;
            excl = a.exclusive != 0;
            st.load(reinterpret_cast<const T *>(a.in) + start, a.n - start);
            ST::issue_heads(a.heads + int64_t(t) * ST::kPlaneWords, pw);
        }
        __device__ __forceinline__ void scan(Shared &sh) {
            st.heads_from(pw);
            st.scan(sh, excl, cov);
        }
        __device__ __forceinline__ void stash(Stash &s, const Args &) const {
#pragma unroll
            for (int r = 0; r < ROWS; r++) s.v[r][threadIdx.x] = st.v[r];
            s.cov[threadIdx.x] = cov;
        }
    };
};

template <class P>
__global__ __launch_bounds__(CtrlPipeline<P>::THREADS) void k_seg_scan(typename P::Args a) {
    CtrlPipeline<P>::run(a);
}

// The heads pass: the reduce pass's marking and plane stores, without the
// data, for tiles of B threads (the pipeline's data threads).
template <class T, class Op, int B, int R, int V>
__global__ __launch_bounds__(B) void k_seg_heads(SegArgs a) {
    using ST = SegTile<T, Op, B, R, V>;
    __shared__ typename ST::Marks mk;
    __shared__ SegChunkMap cm;
    const uint64_t t0 = uint64_t(blockIdx.x) * a.chunk_tiles;
    const uint64_t t1 = t0 + a.chunk_tiles < a.num_tiles ? t0 + a.chunk_tiles : a.num_tiles;
    cm.load(a, t0, t1);
    ST st;
    for (uint64_t t = t0; t < t1; t++) {
        st.rem = a.n - int64_t(t) * ST::TILE;
        st.mark(mk, a, uint32_t(t), cm.get(a, t0, t1, t), cm.get(a, t0, t1, t + 1));
        st.save_heads(a.heads + int64_t(t) * ST::kPlaneWords);
        __syncthreads();  // the marks are rewritten by the next tile
    }
}

// B threads per workgroup: B - 64 data threads and the control wave.
template <class T, class Op, int B, int R, int V>
static int launch_seg_pipe_impl(const SegArgs &a, hipStream_t s) {
    using P = SegScanPolicy<T, Op, B - kWave, R, V>;
    if (a.tile != P::ST::TILE || a.blocks < 1) return SCAN_ERR_UNSUPPORTED;
    const int64_t mg = (a.nseg + 256 * kMapSegs - 1) / (256 * kMapSegs);
    const dim3 mgrid(unsigned(mg < 16384 ? (mg > 0 ? mg : 1) : 16384));
    if (a.tile_log2 >= 0)
        hipLaunchKernelGGL((k_seg_map<T, true>), mgrid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((k_seg_map<T, false>), mgrid, dim3(256), 0, s, a);
    if (hipGetLastError() != hipSuccess) return SCAN_ERR_HIP;
    hipLaunchKernelGGL((k_seg_heads<T, Op, B - kWave, R, V>), dim3(a.blocks), dim3(B - kWave), 0, s, a);
    if (hipGetLastError() != hipSuccess) return SCAN_ERR_HIP;
    const int g = pipeline_grid(reinterpret_cast<const void *>(&k_seg_scan<P>), B, a.pipe.num_tiles, a.grid_cap);
    if (g <= 0) return SCAN_ERR_HIP;
    hipLaunchKernelGGL((k_seg_scan<P>), dim3(g), dim3(B), 0, s, a);
    return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
}

template <class T, class Op, int B, int R, int V>
static int launch_seg_impl(const SegArgs &a, hipStream_t s) {
    if (a.blocks < 1 || a.blocks > uint32_t(kSegPartThreads * kSegPartPer)) return SCAN_ERR_UNSUPPORTED;
    if (a.tile != SegTile<T, Op, B, R, V>::TILE) return SCAN_ERR_UNSUPPORTED;
    const int64_t mg = (a.nseg + 256 * kMapSegs - 1) / (256 * kMapSegs);
    const dim3 mgrid(unsigned(mg < 16384 ? (mg > 0 ? mg : 1) : 16384));
    if (a.tile_log2 >= 0)
        hipLaunchKernelGGL((k_seg_map<T, true>), mgrid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((k_seg_map<T, false>), mgrid, dim3(256), 0, s, a);
    if (hipGetLastError() != hipSuccess) return SCAN_ERR_HIP;
    hipLaunchKernelGGL((k_seg_reduce<T, Op, B, R, V>), dim3(a.blocks), dim3(B), 0, s, a);
    if (hipGetLastError() != hipSuccess) return SCAN_ERR_HIP;
    hipLaunchKernelGGL((k_seg_partials<T, Op>), dim3(1), dim3(kSegPartThreads), 0, s, a);
    if (hipGetLastError() != hipSuccess) return SCAN_ERR_HIP;
    hipLaunchKernelGGL((k_seg_rescan<T, Op, B, R, V>), dim3(a.blocks), dim3(B), 0, s, a);
    return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
}

// Shapes: the default 256 threads x 2 rows, the ones the tuning sweep
// visits, and 256 x 1 (the smallest tiles, for tests); element-wide
// variants of each.
// Single-pass shapes: 512 threads (448 data) x 8 rows, and 256 x 1 (small
// tiles for tests); element-wide variants of each.
template <class T, class Op, int V>
static SegLaunch pick_seg_pipe_shape(int block, int rows) {
    if (block == 512 && rows == 4) return &launch_seg_pipe_impl<T, Op, 512, 4, V>;
    if (block == 512 && rows == 2) return &launch_seg_pipe_impl<T, Op, 512, 2, V>;
    if (block == 768 && rows == 2) return &launch_seg_pipe_impl<T, Op, 768, 2, V>;
    if (block == 256 && rows == 1) return &launch_seg_pipe_impl<T, Op, 256, 1, V>;
    return nullptr;
}

template <class T, class Op, int V>
static SegLaunch pick_seg_shape(int block, int rows) {
    if (block == 256 && rows == 1) return &launch_seg_impl<T, Op, 256, 1, V>;
    if (block == 256 && rows == 2) return &launch_seg_impl<T, Op, 256, 2, V>;
    if (block == 256 && rows == 4) return &launch_seg_impl<T, Op, 256, 4, V>;
    if (block == 512 && rows == 1) return &launch_seg_impl<T, Op, 512, 1, V>;
    if (block == 512 && rows == 2) return &launch_seg_impl<T, Op, 512, 2, V>;
    if (block == 128 && rows == 2) return &launch_seg_impl<T, Op, 128, 2, V>;
    if constexpr (sizeof(T) == 4) {
        if (block == 512 && rows == 8) return &launch_seg_impl<T, Op, 512, 8, V>;
        if (block == 512 && rows == 4) return &launch_seg_impl<T, Op, 512, 4, V>;
    } else {
        if (block == 512 && rows == 4) return &launch_seg_impl<T, Op, 512, 4, V>;
    }
    return nullptr;
}

template <class T, class Op, bool PIPE>
static SegLaunch pick_seg_vec(int block, int rows, int vec) {
    constexpr int VMAX = 16 / int(sizeof(T));
    if constexpr (PIPE) {
        if (vec == VMAX) return pick_seg_pipe_shape<T, Op, VMAX>(block, rows);
        if (vec == 1) return pick_seg_pipe_shape<T, Op, 1>(block, rows);
    } else {
        if (vec == VMAX) return pick_seg_shape<T, Op, VMAX>(block, rows);
        if (vec == 1) return pick_seg_shape<T, Op, 1>(block, rows);
    }
    return nullptr;
}

template <class T, bool PIPE>
static SegLaunch pick_seg_op(scan_op_t op, int block, int rows, int vec) {
    switch (op) {
    case SCAN_OP_SUM: return pick_seg_vec<T, OpSum, PIPE>(block, rows, vec);
    case SCAN_OP_PROD: return pick_seg_vec<T, OpProd, PIPE>(block, rows, vec);
    case SCAN_OP_MAX: return pick_seg_vec<T, OpMax, PIPE>(block, rows, vec);
    case SCAN_OP_MIN: return pick_seg_vec<T, OpMin, PIPE>(block, rows, vec);
    }
    return nullptr;
}

#if SW64_DT == 0
SegLaunch find_seg_i32(scan_op_t op, int b, int r, int v) { return pick_seg_op<int32_t, false>(op, b, r, v); }
SegLaunch find_seg_pipe_i32(scan_op_t op, int b, int r, int v) { return pick_seg_op<int32_t, true>(op, b, r, v); }
#elif SW64_DT == 1
SegLaunch find_seg_u32(scan_op_t op, int b, int r, int v) { return pick_seg_op<uint32_t, false>(op, b, r, v); }
SegLaunch find_seg_pipe_u32(scan_op_t op, int b, int r, int v) { return pick_seg_op<uint32_t, true>(op, b, r, v); }
#elif SW64_DT == 2
SegLaunch find_seg_i64(scan_op_t op, int b, int r, int v) { return pick_seg_op<int64_t, false>(op, b, r, v); }
SegLaunch find_seg_pipe_i64(scan_op_t op, int b, int r, int v) { return pick_seg_op<int64_t, true>(op, b, r, v); }
#elif SW64_DT == 3
SegLaunch find_seg_f32(scan_op_t op, int b, int r, int v) { return pick_seg_op<float, false>(op, b, r, v); }
SegLaunch find_seg_pipe_f32(scan_op_t op, int b, int r, int v) { return pick_seg_op<float, true>(op, b, r, v); }
#elif SW64_DT == 4
SegLaunch find_seg_f64(scan_op_t op, int b, int r, int v) { return pick_seg_op<double, false>(op, b, r, v); }
SegLaunch find_seg_pipe_f64(scan_op_t op, int b, int r, int v) { return pick_seg_op<double, true>(op, b, r, v); }
#else
#error "SW64_DT must select an element type (0..4)"
#endif

}  // namespace sw64
