// element.hip -- scans of large elements: each element is W consecutive
// components combined component-wise (AcceleratedKernels.jl PR #208: scans
// of structs and of ForwardDiff duals, value + 16 partials = 136 bytes).  The
// same kernel scans along the long axis of an (outer, len, W) array, i.e.
// scan_dim with a small inner extent (1e6 x 8 along dim 0 is 1e6 elements of
// 8 components).
//
// Design: one element per thread, held in registers as W components; the W
// component scans of a tile run side by side (W wave scans on DPP, one LDS
// slot per wave and component), and the tile's carry is the W-component
// aggregate, whose descriptor spans W x (carry bytes / 4) words.  Tiles are
// `block` elements, chosen on the host by the PR's rule for large element
// types (largest power of two whose one-item-per-thread tile plus per-thread
// totals fits the local-memory budget); this kernel keeps less than that in
// LDS (one slot per wave, the PR's second bullet), so the rule is a safe
// bound here.  The loads of one element are consecutive 128-bit accesses
// (lanes at a stride of one element): the cache lines a wave touches are
// shared by its few consecutive accesses, so they go through the caches
// (no nontemporal hint) and HBM sees each byte once.  Ordering, descriptors
// and look-back come from the persistent pipeline (pipeline.hpp).
//
// Compiled once per element type (SW64_DT).
#include "launch.hpp"
#include "tile.hpp"

namespace sw64 {

constexpr int kElemMaxWaves = 4;  // block <= 256 elements

template <class C1, int W>
struct Agg {
    C1 c[W];
};

template <class Op>
struct ElemOp {
    template <class A>
    __device__ __forceinline__ static A identity() {
        A r;
#pragma unroll
        for (int k = 0; k < int(sizeof(A::c) / sizeof(A::c[0])); k++)
            r.c[k] = Op::template identity<std::remove_reference_t<decltype(r.c[0])>>();
        return r;
    }
    template <class A>
    __device__ __forceinline__ static A apply(const A &a, const A &b) {
        A r;
#pragma unroll
        for (int k = 0; k < int(sizeof(A::c) / sizeof(A::c[0])); k++) r.c[k] = Op::apply(a.c[k], b.c[k]);
        return r;
    }
};

template <class T_, class Op_, int W>
struct ElemPolicy {
    using T = T_;
    using Op = Op_;
    using C1 = typename Carry<T, Op>::type;
    using C = Agg<C1, W>;
    static constexpr int BLOCK = 256;  // launch bound; blockDim.x is 64, 128 or 256
    static constexpr int kDescWords = Desc<C>::kWords;
    static constexpr int kBytes = W * int(sizeof(T));
    using Args = ElemArgs;

    struct Shared {
        T tot[W][kElemMaxWaves];
        C agg[3];
    };

    static constexpr int kCW = Desc<C1>::kWords;  // descriptor words per component

    // Component by component, so the registers in use do not grow with W.
    template <class TileT>
    __device__ __forceinline__ static void publish_aggregate(const TileT &ts, uint64_t *d, uint32_t epoch,
                                                             uint32_t state) {
#pragma unroll 1
        for (int k = 0; k < W; k++) Desc<C1>::publish(d + k * kCW, epoch, state, ts.aggp->c[k]);
    }

    __device__ __forceinline__ static void set_identity(C *prefix) {
        if (lane_id() == 0) {
#pragma unroll 1
            for (int k = 0; k < W; k++) prefix->c[k] = Op::template identity<C1>();
        }
    }

    // The decoupled look-back of the pipeline, component-serial (wave 0).
    // Phase 1 polls word 0 of each window slot for its state, as in the
    // scalar look-back.  Phase 2 reduces the slots up to the nearest P one
    // component at a time into LDS; every word read must carry the tag seen
    // in phase 1, otherwise that descriptor advanced from A to P between the
    // reads and the window is read again (states only move forward, so this
    // repeats at most once per slot).  The exclusive prefix accumulates in
    // LDS; lane 0 then publishes P component-wise.
    template <class TileT>
    __device__ static void resolve(const TileT &ts, const uint64_t *desc, uint32_t epoch, uint32_t tile,
                                   int64_t first, WsHeader *hdr, uint32_t spin_limit, C *prefix) {
        __shared__ C1 win[W];
        const int lane = lane_id();
        const C1 id = Op::template identity<C1>();
        if (lane == 0) {
#pragma unroll 1
            for (int k = 0; k < W; k++) prefix->c[k] = id;
        }
        int64_t frontier = int64_t(tile) - 1;
        for (;;) {
            const int64_t p = frontier - lane;
            const uint64_t *dl = desc + p * kDescWords;
            uint64_t tag = 0;
            uint32_t st = kStateP;
            int near_p = kWave, near_x = kWave;
            for (uint32_t polls = 0;; polls++) {
                if (p >= first) {
                    const uint64_t w0 = ld(dl);
                    tag = w0 >> kTagShift;
                    st = desc_state(w0, epoch);
                } else {
                    st = kStateP;
                }
                const uint64_t xm = __ballot(st == 0u), pm = __ballot(st == kStateP);
                near_x = xm ? __builtin_ctzll(xm) : kWave;
                near_p = pm ? __builtin_ctzll(pm) : kWave;
                if (near_x == kWave || near_p < near_x) break;
                if (polls >= spin_limit) {
                    if (lane == 0) flag_error(hdr, kErrSpin);
                    near_p = near_x;  // unpublished slots count as P with the identity
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            const bool reads = p >= first && st != 0u && lane <= near_p;
            bool torn = false;
#pragma unroll 1
            for (int k = 0; k < W; k++) {
                C1 v = id;
                bool bad = false;
                if (reads) {
                    struct Chunks { uint32_t w[kCW]; } c;
#pragma unroll
                    for (int i = 0; i < kCW; i++) {
                        const uint64_t word = ld(dl + k * kCW + i);
                        bad = bad || (word >> kTagShift) != tag;
                        c.w[i] = uint32_t(word);
                    }
                    v = __builtin_bit_cast(C1, c);
                }
                if (__any(bad)) {
                    torn = true;
                    break;
                }
                const C1 sum = wave_reduce<Op>(v);
                if (lane == 0) win[k] = sum;
            }
            if (torn) continue;
            if (lane == 0) {
#pragma unroll 1
                for (int k = 0; k < W; k++) prefix->c[k] = Op::apply(win[k], prefix->c[k]);
            }
            if (near_p < kWave) break;
            frontier -= kWave;
        }
        if (lane == 0) {
            uint64_t *d = const_cast<uint64_t *>(desc) + uint64_t(tile) * kDescWords;
#pragma unroll 1
            for (int k = 0; k < W; k++)
                Desc<C1>::publish(d + k * kCW, epoch, kStateP, Op::apply(prefix->c[k], ts.aggp->c[k]));
        }
    }

    struct Tile {
        T x[W];          // the element; after scan(), its tile-local scan
        int slot;
        bool excl;
        const C *aggp;   // this buffer's aggregate slot in LDS

        __device__ __forceinline__ void set_slot(int s) { slot = s; }

        __device__ __forceinline__ static void geom(const Args &a, uint32_t tile, int64_t &start,
                                                    int64_t &remaining) {
            const uint32_t seg = tile / a.pipe.tiles_per_seg;
            const uint32_t j = tile - seg * a.pipe.tiles_per_seg;
            start = int64_t(seg) * a.seg_len + int64_t(j) * blockDim.x;
            remaining = a.seg_len - int64_t(j) * blockDim.x;
        }

        __device__ __forceinline__ void load(const Args &a, uint32_t tile) {
            int64_t start, remaining;
            geom(a, tile, start, remaining);
            excl = a.exclusive != 0;
            const int64_t e = start + threadIdx.x;
            const T *src = reinterpret_cast<const T *>(a.in) + e * W;
            if (threadIdx.x < remaining) {
                if constexpr (kBytes % 16 == 0) {
                    if (a.vec16) {
#pragma unroll
                        for (int q = 0; q < kBytes / 16; q++) {
                            const u32x4_t w = reinterpret_cast<const u32x4_t *>(src)[q];
                            struct Q { T t[16 / sizeof(T)]; };
                            const Q qq = __builtin_bit_cast(Q, w);
#pragma unroll
                            for (int i = 0; i < int(16 / sizeof(T)); i++) x[q * (16 / sizeof(T)) + i] = qq.t[i];
                        }
                        return;
                    }
                }
#pragma unroll
                for (int k = 0; k < W; k++) x[k] = src[k];
            } else {
#pragma unroll
                for (int k = 0; k < W; k++) x[k] = Op::template identity<T>();
            }
        }

        // W wave scans, one LDS slot per wave and component, then every
        // thread combines the per-wave totals.  One barrier.
        __device__ __forceinline__ void scan(Shared &sh) {
            const T id = Op::template identity<T>();
            const int lane = lane_id(), wave = threadIdx.x / kWave, waves = blockDim.x / kWave;
#pragma unroll
            for (int k = 0; k < W; k++) x[k] = wave_scan_incl<Op>(x[k]);
            if (lane == kWave - 1) {
#pragma unroll
                for (int k = 0; k < W; k++) sh.tot[k][wave] = x[k];
            }
            __syncthreads();
            C agg;
#pragma unroll
            for (int k = 0; k < W; k++) {
                T base = id, run = id;
                for (int w = 0; w < waves; w++) {
                    const T t = sh.tot[k][w];
                    if (w < wave) base = Op::apply(base, t);
                    run = Op::apply(run, t);
                }
                const T mine = excl ? wave_shr1(id, x[k]) : x[k];
                x[k] = Op::apply(base, mine);
                agg.c[k] = C1(run);
            }
            if (threadIdx.x == 0) sh.agg[slot] = agg;
            aggp = &sh.agg[slot];
        }

        __device__ __forceinline__ C aggregate() const { return *aggp; }

        __device__ __forceinline__ void emit(const Args &a, uint32_t tile, const C *prefix) const {
            int64_t start, remaining;
            geom(a, tile, start, remaining);
            if (threadIdx.x >= remaining) return;
            const C pre = *prefix;
            T *dst = reinterpret_cast<T *>(a.out) + (start + threadIdx.x) * W;
            T y[W];
#pragma unroll
            for (int k = 0; k < W; k++) y[k] = T(Op::apply(pre.c[k], C1(x[k])));
            if constexpr (kBytes % 16 == 0) {
                if (a.vec16) {
#pragma unroll
                    for (int q = 0; q < kBytes / 16; q++) {
                        struct Q { T t[16 / sizeof(T)]; } qq;
#pragma unroll
                        for (int i = 0; i < int(16 / sizeof(T)); i++) qq.t[i] = y[q * (16 / sizeof(T)) + i];
                        reinterpret_cast<u32x4_t *>(dst)[q] = __builtin_bit_cast(u32x4_t, qq);
                    }
                    return;
                }
            }
#pragma unroll
            for (int k = 0; k < W; k++) dst[k] = y[k];
        }
    };
};

template <class P>
__global__ __launch_bounds__(P::BLOCK) void k_element(typename P::Args a) {
    Pipeline<P>::run(a);
}

template <class T, class Op, int W>
static int launch_element_impl(const ElemArgs &a, int block, uint32_t grid_cap, hipStream_t s) {
    using P = ElemPolicy<T, Op, W>;
    const int g = pipeline_grid(reinterpret_cast<const void *>(&k_element<P>), block, a.pipe.num_tiles, grid_cap);
    if (g <= 0) return SCAN_ERR_HIP;
    hipLaunchKernelGGL((k_element<P>), dim3(g), dim3(block), 0, s, a);
    return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
}

// Built widths: small vectors and the struct shapes of the measured configs
// (24 x fp32 = 96 B, 17 x fp64 = 136 B); any other width is scanned by the
// column kernel.
template <class T, class Op>
static ElemLaunch pick_width(int w) {
    switch (w) {
    case 2: return &launch_element_impl<T, Op, 2>;
    case 3: return &launch_element_impl<T, Op, 3>;
    case 4: return &launch_element_impl<T, Op, 4>;
    case 8: return &launch_element_impl<T, Op, 8>;
    case 16: return &launch_element_impl<T, Op, 16>;
    case 17: return &launch_element_impl<T, Op, 17>;
    case 24: return &launch_element_impl<T, Op, 24>;
    }
    return nullptr;
}

template <class T>
static ElemLaunch pick_elem_op(scan_op_t op, int w) {
    switch (op) {
    case SCAN_OP_SUM: return pick_width<T, OpSum>(w);
    case SCAN_OP_PROD: return pick_width<T, OpProd>(w);
    case SCAN_OP_MAX: return pick_width<T, OpMax>(w);
    case SCAN_OP_MIN: return pick_width<T, OpMin>(w);
    }
    return nullptr;
}

#if SW64_DT == 0
ElemLaunch find_element_i32(scan_op_t op, int w) { return pick_elem_op<int32_t>(op, w); }
#elif SW64_DT == 1
ElemLaunch find_element_u32(scan_op_t op, int w) { return pick_elem_op<uint32_t>(op, w); }
#elif SW64_DT == 2
ElemLaunch find_element_i64(scan_op_t op, int w) { return pick_elem_op<int64_t>(op, w); }
#elif SW64_DT == 3
ElemLaunch find_element_f32(scan_op_t op, int w) { return pick_elem_op<float>(op, w); }
#elif SW64_DT == 4
ElemLaunch find_element_f64(scan_op_t op, int w) { return pick_elem_op<double>(op, w); }
#else
#error "SW64_DT must select an element type (0..4)"
#endif

}  // namespace sw64
