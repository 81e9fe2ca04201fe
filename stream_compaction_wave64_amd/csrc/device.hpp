// device.hpp -- device primitives for the gfx950 scan kernels.
//
//  * operators with identities and wrap-around integer arithmetic;
//  * the wavefront scan: Kogge-Stone doubling over the 64 lanes of a wave
//    with DPP row shifts and row broadcasts (Merry, "Prefix sums on GPUs",
//    slide "Kogge-Stone"; The CUDA Handbook ch. 13, section 13.3.1, where the
//    warp scan is the innermost step of every scan);
//  * the workgroup scan of per-wave totals through one LDS slot per wave
//    (AcceleratedKernels.jl PR #208, second bullet: one slot per sub-group);
//  * tile descriptors and the decoupled look-back (The CUDA Handbook ch. 13,
//    decoupled look-back section, Figure 13-11 and Listing 13-13).
#pragma once

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <type_traits>

namespace sw64 {

constexpr int kWave = 64;

// ------------------------------------------------------------- operators --

template <class T>
struct Limits;
template <> struct Limits<int32_t> {
    __device__ static int32_t lowest() { return INT32_MIN; }
    __device__ static int32_t highest() { return INT32_MAX; }
};
template <> struct Limits<uint32_t> {
    __device__ static uint32_t lowest() { return 0u; }
    __device__ static uint32_t highest() { return UINT32_MAX; }
};
template <> struct Limits<int64_t> {
    __device__ static int64_t lowest() { return INT64_MIN; }
    __device__ static int64_t highest() { return INT64_MAX; }
};
template <> struct Limits<float> {
    __device__ static float lowest() { return -__builtin_huge_valf(); }
    __device__ static float highest() { return __builtin_huge_valf(); }
};
template <> struct Limits<double> {
    __device__ static double lowest() { return -__builtin_huge_val(); }
    __device__ static double highest() { return __builtin_huge_val(); }
};

// Integer sum and product wrap modulo 2^bits: computed in the unsigned type
// of the same width (signed overflow is undefined in C++).
struct OpSum {
    static constexpr int id = 0;
    template <class T> __device__ __forceinline__ static T identity() { return T(0); }
    template <class T> __device__ __forceinline__ static T apply(T a, T b) {
        if constexpr (std::is_integral_v<T>) {
            using U = std::make_unsigned_t<T>;
            return T(U(a) + U(b));
        } else {
            return a + b;
        }
    }
};

struct OpProd {
    static constexpr int id = 1;
    template <class T> __device__ __forceinline__ static T identity() { return T(1); }
    template <class T> __device__ __forceinline__ static T apply(T a, T b) {
        if constexpr (std::is_integral_v<T>) {
            using U = std::make_unsigned_t<T>;
            return T(U(a) * U(b));
        } else {
            return a * b;
        }
    }
};

struct OpMax {
    static constexpr int id = 2;
    template <class T> __device__ __forceinline__ static T identity() { return Limits<T>::lowest(); }
    template <class T> __device__ __forceinline__ static T apply(T a, T b) { return a > b ? a : b; }
};

struct OpMin {
    static constexpr int id = 3;
    template <class T> __device__ __forceinline__ static T identity() { return Limits<T>::highest(); }
    template <class T> __device__ __forceinline__ static T apply(T a, T b) { return a < b ? a : b; }
};

// Type in which a tile's aggregate and prefix travel between workgroups.
// fp32 sums and products carry in fp64: a prefix that crosses ~1e5 tiles in
// fp32 would spend a large share of the fp32 tolerance on that chain alone.
template <class T, class Op> struct Carry { using type = T; };
template <> struct Carry<float, OpSum> { using type = double; };
template <> struct Carry<float, OpProd> { using type = double; };

// -------------------------------------------------------------- cross-lane --

// DPP move of a 32-bit-multiple value.  Lanes whose source is outside the
// row (or that the row mask disables) receive `old`, the operator identity.
template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf, class T>
__device__ __forceinline__ T dpp_mov(T old, T src) {
    static_assert(sizeof(T) % 4 == 0, "DPP moves 32-bit words");
    if constexpr (sizeof(T) == 4) {
        return __builtin_bit_cast(
            T, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, src),
                                           CTRL, ROW_MASK, BANK_MASK, false));
    } else {
        struct W { int w[sizeof(T) / 4]; };
        W o = __builtin_bit_cast(W, old), s = __builtin_bit_cast(W, src), r;
#pragma unroll
        for (int i = 0; i < int(sizeof(T) / 4); i++)
            r.w[i] = __builtin_amdgcn_update_dpp(o.w[i], s.w[i], CTRL, ROW_MASK, BANK_MASK, false);
        return __builtin_bit_cast(T, r);
    }
}

// DPP control codes (GFX9 family, valid on gfx950).
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143, kWaveShr1 = 0x138;

// Inclusive scan over the 64 lanes: four Kogge-Stone doubling rounds inside
// each 16-lane row (shift 1, 2, 4, 8), then lane 15 of rows 0/2 feeds rows
// 1/3 and lane 31 feeds rows 2/3.  Earlier lanes are the left operand.
template <class Op, class T>
__device__ __forceinline__ T wave_scan_incl(T x) {
    const T id = Op::template identity<T>();
    x = Op::apply(dpp_mov<kRowShr1>(id, x), x);
    x = Op::apply(dpp_mov<kRowShr2>(id, x), x);
    x = Op::apply(dpp_mov<kRowShr4>(id, x), x);
    x = Op::apply(dpp_mov<kRowShr8>(id, x), x);
    x = Op::apply(dpp_mov<kRowBcast15, 0xa>(id, x), x);
    x = Op::apply(dpp_mov<kRowBcast31, 0xc>(id, x), x);
    return x;
}

// Shift every lane's value to the next lane; lane 0 receives `id`.
template <class T>
__device__ __forceinline__ T wave_shr1(T id, T x) {
    return dpp_mov<kWaveShr1>(id, x);
}

// Value of lane `lane` broadcast to the whole wave (a scalar register).
template <class T>
__device__ __forceinline__ T wave_read(T x, int lane) {
    static_assert(sizeof(T) % 4 == 0, "readlane moves 32-bit words");
    struct W { int w[sizeof(T) / 4]; };
    W s = __builtin_bit_cast(W, x), r;
#pragma unroll
    for (int i = 0; i < int(sizeof(T) / 4); i++) r.w[i] = __builtin_amdgcn_readlane(s.w[i], lane);
    return __builtin_bit_cast(T, r);
}

template <class Op, class T>
__device__ __forceinline__ T wave_reduce(T x) {
    return wave_read(wave_scan_incl<Op>(x), kWave - 1);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// A wave-uniform value moved to scalar registers, so that branches on it are
// scalar branches rather than exec-mask regions.
// (The builtin returns a signed int: each half is widened as unsigned.)
__device__ __forceinline__ uint32_t uniform(uint32_t x) { return uint32_t(__builtin_amdgcn_readfirstlane(x)); }
__device__ __forceinline__ int64_t uniform(int64_t x) {
    const uint64_t u = uint64_t(x);
    const uint64_t hi = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(u >> 32)));
    const uint64_t lo = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(u)));
    return int64_t((hi << 32) | lo);
}

// Operators that are associative but not commutative (the segmented scan's
// (head flag, value) operator) declare kOrdered; every combination of
// look-back values then keeps tile order, earlier tiles on the left.
template <class Op>
inline constexpr bool kOrderedOp = requires { Op::kOrdered; };

// Lane l receives lane 63 - l's value (one cross-lane read per 32-bit word).
template <class T>
__device__ __forceinline__ T wave_reverse(T x) {
    static_assert(sizeof(T) % 4 == 0, "cross-lane reads move 32-bit words");
    struct W { int w[sizeof(T) / 4]; };
    W s = __builtin_bit_cast(W, x), r;
    const int addr = (kWave - 1 - lane_id()) * 4;
#pragma unroll
    for (int i = 0; i < int(sizeof(T) / 4); i++) r.w[i] = __builtin_amdgcn_ds_bpermute(addr, s.w[i]);
    return __builtin_bit_cast(T, r);
}

// --------------------------------------------------------- tile descriptors --
//
// A tile publishes its aggregate (state A) and later its inclusive prefix
// (state P) in 64-bit descriptor words written with agent-scope atomic
// stores.  Every word carries in its top 10 bits the tag (epoch mod 256) << 2
// | state and a payload in the low 54 bits.  A word whose tag is not the
// running call's reads as X (nothing published yet).  Each call rewrites
// every word it uses and, at its end, clears the words above its own up to
// the previous high-water mark (end_call), so every word of the workspace
// carries the last call's tag or none: consecutive calls need only distinct
// tags.
//
// Desc<C>: C split into 32-bit chunks, one per word, written one after
// another; a reader accepts the value only when every word carries the same
// tag, which is unambiguous because each state is written exactly once per
// call.  DescTrunc: a double in one word, its low 10 mantissa bits dropped
// (42 of 52 kept, relative change below 2^-42) -- the inter-tile carry of
// fp32 sums and products, which only needs to be far more precise than the
// fp32 outputs.  Plain agent-scope atomic loads and stores suffice: no fence
// is needed, since a reader never combines a tag with a value from another
// write.

constexpr uint32_t kStateA = 1u, kStateP = 2u;
constexpr uint32_t kEpochMask = 0x3fffffffu;  // the header's epoch counter
constexpr int kTagShift = 54;

__device__ __forceinline__ uint64_t desc_tag(uint32_t epoch, uint32_t state) {
    return uint64_t(((epoch & 0xffu) << 2) | state) << kTagShift;
}

// The state a word shows to a call at `epoch`: kStateA / kStateP, or 0 (X).
// An epoch outside the counter's range (a corrupted header) matches no tag,
// so every look-back times out and reports it.
__device__ __forceinline__ uint32_t desc_state(uint64_t w, uint32_t epoch) {
    const uint32_t tag = uint32_t(w >> kTagShift);
    const uint32_t want = epoch <= kEpochMask ? (epoch & 0xffu) : 0x400u;
    return (tag >> 2) == want ? (tag & 3u) : 0u;
}

template <class C>
struct Desc {
    static constexpr int kWords = int(sizeof(C) / 4);
    struct Chunks { uint32_t w[kWords]; };

    __device__ __forceinline__ static void publish(uint64_t *d, uint32_t epoch, uint32_t state, C value) {
        const Chunks c = __builtin_bit_cast(Chunks, value);
        const uint64_t tag = desc_tag(epoch, state);
#pragma unroll
        for (int i = 0; i < kWords; i++)
            __hip_atomic_store(d + i, tag | c.w[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // The words of one descriptor, loaded (decode() reads them later).
    __device__ __forceinline__ static void fetch(const uint64_t *d, uint64_t (&w)[kWords]) {
#pragma unroll
        for (int i = 0; i < kWords; i++)
            w[i] = __hip_atomic_load(d + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // kStateA / kStateP when all words carry that state of `epoch`, 0
    // otherwise (not yet published, or caught between two word writes).
    __device__ __forceinline__ static uint32_t read(const uint64_t *d, uint32_t epoch, C &value) {
        uint64_t w[kWords];
        fetch(d, w);
        return decode(w, epoch, value);
    }

    __device__ __forceinline__ static uint32_t decode(const uint64_t (&w)[kWords], uint32_t epoch, C &value) {
        const uint32_t state = desc_state(w[0], epoch);
        bool ok = state != 0u;
        Chunks c;
#pragma unroll
        for (int i = 0; i < kWords; i++) {
            ok = ok && (w[i] >> kTagShift) == (w[0] >> kTagShift);
            c.w[i] = uint32_t(w[i]);
        }
        value = __builtin_bit_cast(C, c);
        return ok ? state : 0u;
    }
};

struct DescTrunc {
    static constexpr int kWords = 1;
    __device__ __forceinline__ static void publish(uint64_t *d, uint32_t epoch, uint32_t state, double value) {
        __hip_atomic_store(d, desc_tag(epoch, state) | (__builtin_bit_cast(uint64_t, value) >> (64 - kTagShift)),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __device__ __forceinline__ static void fetch(const uint64_t *d, uint64_t (&w)[1]) {
        w[0] = __hip_atomic_load(d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __device__ __forceinline__ static uint32_t decode(const uint64_t (&w)[1], uint32_t epoch, double &value) {
        value = __builtin_bit_cast(double, w[0] << (64 - kTagShift));
        return desc_state(w[0], epoch);
    }
    __device__ __forceinline__ static uint32_t read(const uint64_t *d, uint32_t epoch, double &value) {
        uint64_t w[1];
        fetch(d, w);
        return decode(w, epoch, value);
    }
};

// The descriptor format of a scalar carry: fp32 data carried in fp64 packs
// into one word; everything else is carried exactly.
template <class T, class C>
using DescFor = std::conditional_t<std::is_same_v<T, float> && std::is_same_v<C, double>, DescTrunc, Desc<C>>;

// Workspace header.  Counters that many workgroups update at once sit in
// separate 128-byte lines: same-address agent-scope atomics serialize at about
// 11.5 ns each on MI355X, sixteen addresses give about 1 ns each.
struct WsHeader {
    uint32_t epoch;       // tag of the running call's descriptors
    uint32_t error;       // kErr* bits (see flag_error)
    uint64_t high_water;  // descriptor words the last call left tagged
    uint32_t mode;        // (epoch << 2) | kModeStatic or kModeDynamic: the call that decided it
    uint32_t claim;       // next tile ticket in dynamic mode
    uint64_t capacity;    // descriptor words of the buffer scan_workspace_init zeroed (0: not recorded)
    uint32_t pad0[24];
    struct {
        uint32_t count;   // workgroups of the running call counted in this slot
        uint32_t pad[31];
    } started[16];
};
constexpr size_t kWsHeaderBytes = 4096;
static_assert(sizeof(WsHeader) <= kWsHeaderBytes, "header fits its reserved bytes");
static_assert(offsetof(WsHeader, capacity) == 24 && offsetof(WsHeader, started) == 128, "header layout");
constexpr uint32_t kErrSpin = 1u, kErrFallback = 4u;  // bit 1 is no longer used
constexpr uint32_t kModeStatic = 1u, kModeDynamic = 2u;

__device__ __forceinline__ void flag_error(WsHeader *hdr, uint32_t code) {
    __hip_atomic_fetch_or(&hdr->error, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class U>
__device__ __forceinline__ U ld(const U *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class U>
__device__ __forceinline__ void st(U *p, U v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Start of a call that publishes descriptors (thread 0 only): read the epoch,
// the high-water mark and the recorded capacity (one round trip), then count
// this workgroup with a fire-and-forget atomic whose operand depends on the
// loaded epoch, so the read has returned before the count is made.  Whoever
// later sees every workgroup counted knows that none will read the epoch
// again.  The high-water mark changes only at a call's end, after every
// workgroup is counted, so the value read here is the one end_call needs.
__device__ __forceinline__ uint32_t begin_call(WsHeader *hdr, uint64_t &high_water, uint64_t &capacity) {
    const uint32_t e = ld(&hdr->epoch);
    high_water = ld(&hdr->high_water);
    capacity = ld(&hdr->capacity);
    __hip_atomic_fetch_add(&hdr->started[blockIdx.x & 15].count, 1u + (e >> 30), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    return e;
}

__device__ __forceinline__ uint32_t started_sum(const WsHeader *hdr) {
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) s += ld(&hdr->started[i].count);
    return s;
}

// Decide, once per call, how tiles are assigned (thread 0 only).  The static
// round-robin (workgroup w takes tiles w, w+G, ...) needs all G workgroups
// resident at once: a resident workgroup may wait on a tile of one that has
// not started.  The occupancy the runtime reports is not a guarantee (other
// work may hold compute units, and at full register occupancy it was measured
// to overstate), so the first workgroup that sees all G counted selects
// static mode; one that waits `limit` polls without seeing them selects
// dynamic mode, where tiles are claimed in order from a counter -- slower
// (one same-address atomic per tile), but deadlock-free with any number of
// resident workgroups.  No tile waits on another before the decision; the
// resident passes publish their static first tile's aggregate before it,
// which is safe because a tile's aggregate depends only on its data, so the
// workgroup that processes the tile in either mode publishes the same words
// (aggregates only: a word never changes state within a call).
// Each poll reads the mode word and the counters in one round trip; the
// compare-and-swap returns the decided mode whether or not it won.  The
// mode word carries the epoch it was decided in ((epoch << 2) | mode) and
// is never reset: a word from another call reads as undecided, and a
// workgroup still polling after this call's end (which resets the counters)
// still finds this call's decision.
__device__ __forceinline__ uint32_t decide_mode(WsHeader *hdr, uint32_t epoch, uint32_t G, uint32_t limit) {
    const uint32_t tag = (epoch & kEpochMask) << 2;
    auto decided = [&](uint32_t m) { return (m & ~3u) == tag && (m & 3u) != 0u; };
    uint32_t m = ld(&hdr->mode);
    for (uint32_t polls = 0;; polls++) {
        const uint32_t started = started_sum(hdr);
        if (decided(m)) return m & 3u;
        const uint32_t want = started >= G ? kModeStatic : (polls >= limit ? kModeDynamic : 0u);
        if (want != 0u) {
            uint32_t expected = m;
            if (__hip_atomic_compare_exchange_strong(&hdr->mode, &expected, tag | want, __ATOMIC_RELAXED,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
                if (want == kModeDynamic) flag_error(hdr, kErrFallback);
                return want;
            }
            if (decided(expected)) return expected & 3u;  // another workgroup's decision
            m = expected;
            continue;
        }
        __builtin_amdgcn_s_sleep(2);
        m = ld(&hdr->mode);
    }
}

// End of a call, run by one workgroup once every workgroup is known to have
// read the epoch: reset the per-call words, advance the epoch for the next
// call on this workspace, and clear the descriptor words above this call's
// up to the previous high-water mark `hw` (begin_call's): words below
// `words_used` were all rewritten by this call, so afterwards every word
// carries this call's tag or none.  The clearing reaches as far as the buffer
// goes: the call's own `ws_words`, or the capacity scan_workspace_init
// recorded when the caller passes a smaller size on the same buffer.  Words
// beyond both (a buffer zeroed by other means, then passed with shrinking
// sizes) keep the high-water mark up, so the next call that sees them clears
// them.  In static mode every workgroup was counted before the mode was
// decided; in dynamic mode the caller holds the last claim.  Whole workgroup
// (no barrier).
__device__ __forceinline__ void end_call(WsHeader *hdr, uint32_t epoch, uint64_t hw, uint64_t capacity,
                                         uint64_t words_used, uint64_t ws_words, uint64_t *desc) {
    const uint64_t room = ws_words > capacity ? ws_words : capacity;
    const uint64_t clear_end = hw < room ? hw : room;
    if (threadIdx.x == 0) {
        st(&hdr->high_water, clear_end < hw ? hw : words_used);
#pragma unroll
        for (int i = 0; i < 16; i++) st(&hdr->started[i].count, 0u);
        st(&hdr->claim, 0u);
        st(&hdr->epoch, (epoch + 1u) & kEpochMask);
    }
    for (uint64_t i = words_used + threadIdx.x; i < clear_end; i += blockDim.x) st(desc + i, uint64_t(0));
}

// Decoupled look-back by one wave (The CUDA Handbook ch. 13, Figure 13-11),
// widened for MI355X.  The page's warp inspects the 32 nearest predecessors
// per step; here every lane reads DEPTH descriptors at once, so one round
// trip covers the 64*DEPTH nearest predecessors: slot (lane, k) holds tile
// frontier - lane - 64*k, i.e. distance d = lane + 64*k.  A descriptor read
// crosses XCDs (~1.3 us), and the frontier of published prefixes advances at
// most one window per round trip, so the window must span more tiles than
// the grid finishes per round trip; 64 does not at HBM rate.
//
// The window is re-read while any slot nearer than the nearest P is still X.
// Then the values of slots 0..nearest P (aggregates, then that prefix) are
// combined; with no P in the window, all of them are combined and the
// window moves 64*DEPTH tiles back.  Tiles before `first` (the start of the
// segment) count as P with the identity.  Returns the exclusive prefix of
// `tile`, the same in every lane.  A commutative operator combines the
// window in lane order; an ordered one (kOrderedOp) in tile order.
//
// Every wait is bounded: after `spin_limit` polls of one window the wave
// flags kErrSpin in the header and takes the unpublished slots as P with the
// identity, so the kernel always finishes (with a wrong result that the
// flag reports) instead of spinning forever on a tile that never runs.
template <class Op, class C, int DEPTH, class D = Desc<C>>
__device__ __forceinline__ C lookback(const uint64_t *desc, uint32_t epoch, int64_t tile, int64_t first,
                                      WsHeader *hdr, uint32_t spin_limit) {
    constexpr int kSpan = kWave * DEPTH;
    const int lane = lane_id();
    const C id = Op::template identity<C>();
    C excl = id;
    int64_t frontier = tile - 1;
    for (;;) {
        uint32_t st[DEPTH];
        C v[DEPTH];
        int near_p = kSpan;  // distance of the nearest P (kSpan: none)
        for (uint32_t polls = 0;; polls++) {
#pragma unroll
            for (int k = 0; k < DEPTH; k++) {
                const int64_t p = frontier - lane - int64_t(kWave) * k;
                if (p >= first) {
                    st[k] = D::read(desc + p * D::kWords, epoch, v[k]);
                } else {
                    st[k] = kStateP;
                    v[k] = id;
                }
            }
            int near_x = kSpan;
            near_p = kSpan;
#pragma unroll
            for (int k = DEPTH - 1; k >= 0; k--) {
                const uint64_t xm = __ballot(st[k] == 0u);
                const uint64_t pm = __ballot(st[k] == kStateP);
                if (xm) near_x = kWave * k + __builtin_ctzll(xm);
                if (pm) near_p = kWave * k + __builtin_ctzll(pm);
            }
            if (near_x == kSpan || near_p < near_x) break;
            if (polls >= spin_limit) {
                if (lane == 0) flag_error(hdr, kErrSpin);
#pragma unroll
                for (int k = 0; k < DEPTH; k++) {
                    if (st[k] == 0u) v[k] = id;
                }
                near_p = near_x;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if constexpr (kOrderedOp<Op>) {
            // tile order is distance order reversed: per block of 64 slots,
            // reverse the lanes and reduce; older blocks on the left
            C win = id;
#pragma unroll
            for (int k = DEPTH - 1; k >= 0; k--) {
                const C x = lane + kWave * k <= near_p ? v[k] : id;
                win = Op::apply(win, wave_reduce<Op>(wave_reverse(x)));
            }
            excl = Op::apply(win, excl);
        } else {
            C contrib = id;
#pragma unroll
            for (int k = 0; k < DEPTH; k++) {
                if (lane + kWave * k <= near_p) contrib = Op::apply(v[k], contrib);
            }
            excl = Op::apply(wave_reduce<Op>(contrib), excl);
        }
        if (near_p < kSpan) break;
        frontier -= kSpan;
    }
    return excl;
}

// Look-back of the static order by aggregates only (an MI355X design).  The
// page's look-back finds a predecessor's inclusive prefix, so the prefixes
// form a chain through the workgroups of a round: with 64 predecessors per
// round trip, the last of G = 256 workgroups needs four dependent round
// trips.  In the static order workgroup w owns tiles w, w + G, ..., so it
// already knows the inclusive prefix of its own previous tile t - G; tile
// t's exclusive prefix is that value combined with the aggregates of the
// G - 1 tiles between them, which their owners published a step or more
// earlier.  One round trip, which issue() starts and finish() completes
// after the caller's other work, and no tile waits for another's prefix.
// The G - 1 reads per tile (64 * NR at most) are the price.
//
// Slot (lane, k) reads tile lo + lane + 64k for tiles in [lo, hi).  A slot
// still X at finish() is re-read until published; after `spin_limit` polls
// the wave flags kErrSpin and counts it as the identity, so the wait always
// ends.  Commutative operators combine slots as they arrive; ordered ones
// (kOrderedOp) keep tile order.
template <class C, class D, int NR>
struct GapRead {
    uint64_t w[NR][D::kWords];
    int64_t lo, hi;

    __device__ __forceinline__ void issue(const uint64_t *desc, int64_t lo_, int64_t hi_) {
        lo = lo_;
        hi = hi_;
#pragma unroll
        for (int k = 0; k < NR; k++) {
            const int64_t p = lo + lane_id() + int64_t(kWave) * k;
            if (p < hi) D::fetch(desc + p * D::kWords, w[k]);
        }
    }

    // Every still-unpublished slot read again, all loads issued before any
    // is decoded: one memory round trip per poll however many slots wait
    // (a load and its decode per slot made one round trip per slot).
    __device__ __forceinline__ void refetch(const uint64_t *desc, uint32_t pending) {
#pragma unroll
        for (int k = 0; k < NR; k++) {
            const int64_t p = lo + lane_id() + int64_t(kWave) * k;
            if (pending & (1u << k)) D::fetch(desc + p * D::kWords, w[k]);
        }
    }

    // The combination of the aggregates of [lo, hi), the same in every lane.
    template <class Op>
    __device__ __forceinline__ C finish(const uint64_t *desc, uint32_t epoch, WsHeader *hdr, uint32_t spin_limit) {
        if constexpr (kOrderedOp<Op>) return finish_ordered<Op>(desc, epoch, hdr, spin_limit);
        const C id = Op::template identity<C>();
        C acc = id;
        uint32_t pending = 0;  // bit k: slot k not yet published
#pragma unroll
        for (int k = 0; k < NR; k++) {
            const int64_t p = lo + lane_id() + int64_t(kWave) * k;
            C v;
            if (p < hi) {
                if (D::decode(w[k], epoch, v) != 0u)
                    acc = Op::apply(v, acc);
                else
                    pending |= 1u << k;
            }
        }
        for (uint32_t polls = 0; __ballot(pending != 0u) != 0ull; polls++) {
            if (polls >= spin_limit) {
                if (lane_id() == 0) flag_error(hdr, kErrSpin);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
            refetch(desc, pending);
#pragma unroll
            for (int k = 0; k < NR; k++) {
                C v;
                if ((pending & (1u << k)) && D::decode(w[k], epoch, v) != 0u) {
                    acc = Op::apply(v, acc);
                    pending &= ~(1u << k);
                }
            }
        }
        return wave_reduce<Op>(acc);
    }

    // The same for an ordered operator: every slot's value is kept until all
    // are published, then block k (tiles lo + 64k .. lo + 64k + 63, in lane
    // order) is reduced across the wave and the blocks combined in order.
    template <class Op>
    __device__ __forceinline__ C finish_ordered(const uint64_t *desc, uint32_t epoch, WsHeader *hdr,
                                                uint32_t spin_limit) {
        const C id = Op::template identity<C>();
        C v[NR];
        uint32_t pending = 0;  // bit k: slot k not yet published
#pragma unroll
        for (int k = 0; k < NR; k++) {
            const int64_t p = lo + lane_id() + int64_t(kWave) * k;
            v[k] = id;
            if (p < hi && D::decode(w[k], epoch, v[k]) == 0u) {
                v[k] = id;
                pending |= 1u << k;
            }
        }
        for (uint32_t polls = 0; __ballot(pending != 0u) != 0ull; polls++) {
            if (polls >= spin_limit) {
                if (lane_id() == 0) flag_error(hdr, kErrSpin);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
            refetch(desc, pending);
#pragma unroll
            for (int k = 0; k < NR; k++) {
                if (pending & (1u << k)) {
                    if (D::decode(w[k], epoch, v[k]) != 0u)
                        pending &= ~(1u << k);
                    else
                        v[k] = id;
                }
            }
        }
        C acc = id;
#pragma unroll
        for (int k = 0; k < NR; k++) {
            if (lo + int64_t(kWave) * k < hi) acc = Op::apply(acc, wave_reduce<Op>(v[k]));
        }
        return acc;
    }
};

// ---------------------------------------------------------- vector access --

template <class T, int V>
struct alignas(sizeof(T) * V) Vec {
    T v[V];
};

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 128-bit (or element-wide) accesses that bypass cache allocation: every
// input is read once and every output written once, so streaming through
// the caches only evicts data others could use.
template <class T, int V>
__device__ __forceinline__ Vec<T, V> load_vec(const T *p) {
    constexpr int B = int(sizeof(T)) * V;
    if constexpr (B == 16) {
        return __builtin_bit_cast(Vec<T, V>, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p)));
    } else if constexpr (B == 8) {
        return __builtin_bit_cast(Vec<T, V>, __builtin_nontemporal_load(reinterpret_cast<const uint64_t *>(p)));
    } else {
        static_assert(B == 4, "vector access of 4, 8 or 16 bytes");
        return __builtin_bit_cast(Vec<T, V>, __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p)));
    }
}

// Buffer resource over `count` elements at `base` (a wave-uniform pointer):
// accesses at byte offsets past the range read 0 / are dropped by the
// hardware, so a tile's ragged end needs no branch.  Word 3 is the gfx9
// family's raw-buffer configuration (no swizzle, no format conversion).
using BufRsrc = __amdgpu_buffer_rsrc_t;
// The operands are moved to scalar registers explicitly: a resource the
// compiler cannot prove uniform would be wrapped in a per-lane loop.
template <class T>
__device__ __forceinline__ BufRsrc make_rsrc(const T *base, int64_t count) {
    T *b = reinterpret_cast<T *>(uniform(int64_t(reinterpret_cast<uintptr_t>(base))));
    const uint32_t bytes = uniform(uint32_t(count * int64_t(sizeof(T))));
    return __builtin_amdgcn_make_buffer_rsrc(b, 0, int(bytes), 0x00020000);
}

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// Store of one vector through a buffer resource; AUX is the cache policy
// (2: nontemporal, streaming, the default; 0: the default policy, for an
// output the next kernel reads right away).
template <class T, int V, int AUX = 2>
__device__ __forceinline__ void store_vec_bounded(BufRsrc rs, uint32_t byte_off, const Vec<T, V> &x) {
    constexpr int B = int(sizeof(T)) * V;
    constexpr int kNT = AUX;
    if constexpr (B == 16) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, x), rs, byte_off, 0, kNT);
    } else if constexpr (B == 8) {
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, x), rs, byte_off, 0, kNT);
    } else {
        static_assert(B == 4, "vector access of 4, 8 or 16 bytes");
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), rs, byte_off, 0, kNT);
    }
}

template <class T, int V>
__device__ __forceinline__ void store_vec(T *p, const Vec<T, V> &x) {
    constexpr int B = int(sizeof(T)) * V;
    if constexpr (B == 16) {
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, x), reinterpret_cast<u32x4_t *>(p));
    } else if constexpr (B == 8) {
        __builtin_nontemporal_store(__builtin_bit_cast(uint64_t, x), reinterpret_cast<uint64_t *>(p));
    } else {
        static_assert(B == 4, "vector access of 4, 8 or 16 bytes");
        __builtin_nontemporal_store(__builtin_bit_cast(uint32_t, x), reinterpret_cast<uint32_t *>(p));
    }
}

}  // namespace sw64
