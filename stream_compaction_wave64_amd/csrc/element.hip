// element.hip -- scans of large elements: each element is W consecutive
// components combined component-wise (AcceleratedKernels.jl PR #208: scans
// of structs and of ForwardDiff duals, value + 16 partials = 136 bytes).  The
// same kernels scan along the long axis of an (outer, len, W) array, i.e.
// scan_dim with a small inner extent (1e6 x 8 along dim 0 is 1e6 elements of
// 8 components).
//
// Reduce-then-scan over chunks of tiles (The CUDA Handbook ch. 13 section
// 13.3.3; Merry, "Prefix sums on GPUs", slide "Reduce-then-Scan strategy"),
// chosen over the single-pass look-back here because a carry of W components
// makes every look-back window W times as expensive to read, while the second
// read of a chunk mostly hits the 256 MB Infinity Cache at these sizes.
//   1. reduce: each workgroup folds its chunk into W component partials;
//   2. partials: per segment and component, an exclusive scan over chunks;
//   3. rescan: each workgroup scans its chunk again from those prefixes,
//      tile by tile with a running carry, and zeroes its partials (the
//      workspace's descriptor area is left zeroed).
//
// A tile is `threads` x E elements.  It is moved between HBM and LDS with
// coalesced accesses (consecutive lanes, consecutive 16-byte vectors, or
// element-wide values when the data is not 16-byte aligned) and transposed
// through LDS so that each thread owns E consecutive elements: the W
// component scans are then thread-serial over E elements, W wave scans on
// DPP, and one LDS slot per wave and component (the PR's second bullet).  A
// thread's LDS slots are padded to an odd number of accesses so the
// transposed reads are free of bank conflicts.  `threads` comes from the
// PR's LDS-budget rule for large elements and E fills the rest of the budget
// (see plan_element in api.hip).
//
// Compiled once per element type (SW64_DT).
#include "launch.hpp"

namespace sw64 {

constexpr int kElemMaxThreads = 512;
constexpr int kElemMaxWaves = kElemMaxThreads / kWave;

template <class T, class Op, int W, int E, int LG>
struct ElemTile {
    using C = typename Carry<T, Op>::type;
    static constexpr int S = int(sizeof(T));
    static constexpr int LV = LG / S;       // values per global access
    static constexpr int VPT = E * W;       // values a thread owns per tile
    static_assert(LG % S == 0 && VPT % LV == 0, "whole accesses per thread");
    static constexpr int UPT = VPT / LV;    // accesses per thread per tile
    static constexpr int STRIDE = VPT + (UPT % 2 == 0 ? LV : 0);  // LDS values per thread

    // tile + per-wave totals (reduce: in C, rescan: in T) + W carries (rescan)
    static constexpr size_t lds_bytes(int threads) {
        return size_t(threads) * STRIDE * S + size_t(kElemMaxWaves) * W * sizeof(C);
    }
    static constexpr size_t lds_bytes_rescan(int threads) { return lds_bytes(threads) + W * sizeof(C); }

    using Acc = Vec<T, LV>;  // one global access

    // Geometry of tile `j` of segment `seg`.
    struct Geo {
        int64_t e0;     // first element of the tile within its segment
        int64_t valid;  // elements of the tile in range (<= threads * E)
        BufRsrc rs;     // the tile's bytes in the (input or output) array
    };

    __device__ __forceinline__ static Geo geo(const ElemArgs &a, const void *base, uint32_t seg, int64_t j) {
        Geo g;
        const int64_t tile = int64_t(blockDim.x) * E;
        g.e0 = j * tile;
        const int64_t rem = a.len - g.e0;
        g.valid = uniform(rem < tile ? rem : tile);
        const T *p = reinterpret_cast<const T *>(base) + (int64_t(seg) * a.len + g.e0) * W;
        g.rs = make_rsrc(p, g.valid * W);
        return g;
    }

    // Global -> registers: access u = r * threads + thread of the tile
    // (value u * LV), r < UPT; accesses past the range read zero.
    // AUX: the loads' cache policy (2: nontemporal; 0: the reduce pass, whose
    // data the rescan reads again soon after and may find in the caches).
    template <int AUX = 2>
    __device__ __forceinline__ static void load_regs(const Geo &g, Acc (&x)[UPT]) {
#pragma unroll
        for (int r = 0; r < UPT; r++) {
            const uint32_t u = uint32_t(r) * blockDim.x + threadIdx.x;
            if constexpr (LG == 16)
                x[r] = __builtin_bit_cast(Acc, __builtin_amdgcn_raw_buffer_load_b128(g.rs, u * 16u, 0, AUX));
            else if constexpr (LG == 8)
                x[r] = __builtin_bit_cast(Acc, __builtin_amdgcn_raw_buffer_load_b64(g.rs, u * 8u, 0, AUX));
            else
                x[r] = __builtin_bit_cast(Acc, __builtin_amdgcn_raw_buffer_load_b32(g.rs, u * 4u, 0, AUX));
        }
    }

    // Registers -> LDS in the owner layout: access u belongs to thread
    // u / UPT at its slot (u % UPT) * LV.
    __device__ __forceinline__ static void regs_to_lds(const Acc (&x)[UPT], T *lds) {
#pragma unroll
        for (int r = 0; r < UPT; r++) {
            const uint32_t u = uint32_t(r) * blockDim.x + threadIdx.x;
            *reinterpret_cast<Acc *>(lds + (u / UPT) * STRIDE + (u % UPT) * LV) = x[r];
        }
    }

    // LDS (owner layout) -> global, dropping values past the tile's range.
    __device__ __forceinline__ static void store_tile(const Geo &g, const T *lds) {
#pragma unroll
        for (int r = 0; r < UPT; r++) {
            const uint32_t u = uint32_t(r) * blockDim.x + threadIdx.x;
            const Acc x = *reinterpret_cast<const Acc *>(lds + (u / UPT) * STRIDE + (u % UPT) * LV);
            store_vec_bounded<T, LV>(g.rs, u * uint32_t(LG), x);
        }
    }

    // This thread's E elements from LDS; elements past the range hold the
    // identity.
    __device__ __forceinline__ static void read_own(const Geo &g, const T *lds, T (&v)[VPT]) {
        const T *src = lds + threadIdx.x * STRIDE;
#pragma unroll
        for (int q = 0; q < UPT; q++) {
            const Acc x = *reinterpret_cast<const Acc *>(src + q * LV);
#pragma unroll
            for (int i = 0; i < LV; i++) v[q * LV + i] = x.v[i];
        }
        const T id = Op::template identity<T>();
#pragma unroll
        for (int e = 0; e < E; e++) {
            const bool in = int64_t(threadIdx.x) * E + e < g.valid;
#pragma unroll
            for (int c = 0; c < W; c++) v[e * W + c] = in ? v[e * W + c] : id;
        }
    }

    __device__ __forceinline__ static void write_own(T *lds, const T (&v)[VPT]) {
        T *dst = lds + threadIdx.x * STRIDE;
#pragma unroll
        for (int q = 0; q < UPT; q++) {
            Acc x;
#pragma unroll
            for (int i = 0; i < LV; i++) x.v[i] = v[q * LV + i];
            *reinterpret_cast<Acc *>(dst + q * LV) = x;
        }
    }

    __device__ __forceinline__ static uint32_t tiles_of(const ElemArgs &a, uint32_t chunk, int64_t &j0) {
        const int64_t tiles = (a.len + int64_t(blockDim.x) * E - 1) / (int64_t(blockDim.x) * E);
        j0 = int64_t(chunk) * a.tiles_per_chunk;
        const int64_t left = tiles - j0;
        return uint32_t(left < int64_t(a.tiles_per_chunk) ? (left > 0 ? left : 0) : a.tiles_per_chunk);
    }

    // Pass 1: the W component partials of each chunk.
    __device__ static void reduce(const ElemArgs &a) {
        extern __shared__ __align__(16) char smem[];
        T *lds = reinterpret_cast<T *>(smem);
        C *red = reinterpret_cast<C *>(smem + size_t(blockDim.x) * STRIDE * S);
        const uint32_t seg = blockIdx.x / a.chunks, chunk = blockIdx.x % a.chunks;
        const C cid = Op::template identity<C>();
        C acc[W];
#pragma unroll
        for (int c = 0; c < W; c++) acc[c] = cid;
        int64_t j0;
        const uint32_t nt = tiles_of(a, chunk, j0);
        // the next tile's loads are in flight while this one is folded
        Acc nx[UPT];
        if (nt > 0) load_regs<0>(geo(a, a.in, seg, j0), nx);
        for (uint32_t k = 0; k < nt; k++) {
            const Geo g = geo(a, a.in, seg, j0 + k);
            if (k > 0) __syncthreads();  // previous tile's reads are done
            regs_to_lds(nx, lds);
            if (k + 1 < nt) load_regs<0>(geo(a, a.in, seg, j0 + k + 1), nx);
            __syncthreads();
            T v[VPT];
            read_own(g, lds, v);
#pragma unroll
            for (int e = 0; e < E; e++) {
#pragma unroll
                for (int c = 0; c < W; c++) acc[c] = Op::apply(acc[c], C(v[e * W + c]));
            }
        }
        const int wave = threadIdx.x / kWave, waves = blockDim.x / kWave;
#pragma unroll
        for (int c = 0; c < W; c++) {
            const C r = wave_reduce<Op>(acc[c]);
            if (lane_id() == 0) red[wave * W + c] = r;
        }
        __syncthreads();
        if (threadIdx.x < W) {
            C t = cid;
            for (int w = 0; w < waves; w++) t = Op::apply(t, red[w * W + threadIdx.x]);
            reinterpret_cast<C *>(a.partials)[(int64_t(seg) * a.chunks + chunk) * W + threadIdx.x] = t;
        }
    }

    // Pass 3: scan each tile of the chunk from the chunk's prefix.  The
    // tile's values stay in LDS, read twice by their owner thread: once for
    // its W component totals, once to replace them by their results; the
    // registers hold the W running offsets and the next tile's loads (issued
    // as soon as this tile is in LDS, so a workgroup's tiles do not each wait
    // a full load latency: 1e6 elements of 24 fp32, 65.9 -> 61.8 us per
    // call), and the chunk's W carries sit in LDS.
    __device__ static void rescan(const ElemArgs &a) {
        extern __shared__ __align__(16) char smem[];
        T *lds = reinterpret_cast<T *>(smem);
        T *wt = reinterpret_cast<T *>(smem + size_t(blockDim.x) * STRIDE * S);
        C *carry = reinterpret_cast<C *>(smem + lds_bytes(int(blockDim.x)));  // W running prefixes
        const uint32_t seg = blockIdx.x / a.chunks, chunk = blockIdx.x % a.chunks;
        const int lane = lane_id(), wave = threadIdx.x / kWave, waves = blockDim.x / kWave;
        const T id = Op::template identity<T>();
        C *part = reinterpret_cast<C *>(a.partials) + (int64_t(seg) * a.chunks + chunk) * W;
        if (threadIdx.x < W) {
            carry[threadIdx.x] = part[threadIdx.x];
            part[threadIdx.x] = C{};  // leave the workspace zeroed
        }
        int64_t j0;
        const uint32_t nt = tiles_of(a, chunk, j0);
        T *own = lds + threadIdx.x * STRIDE;
        // the next tile's loads are in flight while this one is scanned and
        // stored
        Acc nx[UPT];
        if (nt > 0) load_regs(geo(a, a.in, seg, j0), nx);
        for (uint32_t k = 0; k < nt; k++) {
            const Geo gi = geo(a, a.in, seg, j0 + k);
            __syncthreads();  // carry written; previous tile's stores have read LDS
            regs_to_lds(nx, lds);
            if (k + 1 < nt) load_regs(geo(a, a.in, seg, j0 + k + 1), nx);
            __syncthreads();
            // this thread's component totals (elements past the range: identity)
            T off[W];
#pragma unroll
            for (int c = 0; c < W; c++) off[c] = id;
#pragma unroll
            for (int q = 0; q < UPT; q++) {
                const Acc x = *reinterpret_cast<const Acc *>(own + q * LV);
#pragma unroll
                for (int i = 0; i < LV; i++) {
                    const int idx = q * LV + i, e = idx / W, c = idx % W;
                    if (int64_t(threadIdx.x) * E + e < gi.valid) off[c] = Op::apply(off[c], x.v[i]);
                }
            }
            // wave scans of the totals: off[c] becomes the thread's exclusive
            // offset within its wave
#pragma unroll
            for (int c = 0; c < W; c++) {
                const T inc = wave_scan_incl<Op>(off[c]);
                if (lane == kWave - 1) wt[wave * W + c] = inc;
                off[c] = wave_shr1(id, inc);
            }
            __syncthreads();
#pragma unroll
            for (int c = 0; c < W; c++) {
                T base = id;
                for (int w = 0; w < wave; w++) base = Op::apply(base, wt[w * W + c]);
                off[c] = Op::apply(base, off[c]);
            }
            // results in place: carry (+) inclusive (or exclusive) tile-local value
#pragma unroll
            for (int q = 0; q < UPT; q++) {
                Acc x = *reinterpret_cast<const Acc *>(own + q * LV);
#pragma unroll
                for (int i = 0; i < LV; i++) {
                    const int c = (q * LV + i) % W;
                    const T inc = Op::apply(off[c], x.v[i]);
                    x.v[i] = T(Op::apply(carry[c], C(a.exclusive ? off[c] : inc)));
                    off[c] = inc;
                }
                *reinterpret_cast<Acc *>(own + q * LV) = x;
            }
            __syncthreads();  // every thread has read the carry and written its results
            if (threadIdx.x < W) {
                T tot = id;
                for (int w = 0; w < waves; w++) tot = Op::apply(tot, wt[w * W + threadIdx.x]);
                carry[threadIdx.x] = Op::apply(carry[threadIdx.x], C(tot));
            }
            store_tile(geo(a, a.out, seg, j0 + k), lds);
        }
    }
};

template <class K>
__global__ __launch_bounds__(kElemMaxThreads) void k_elem_reduce(ElemArgs a) {
    K::reduce(a);
}

template <class K>
__global__ __launch_bounds__(kElemMaxThreads) void k_elem_rescan(ElemArgs a) {
    K::rescan(a);
}

// Pass 2: one workgroup per (segment, component) scans the chunk partials
// into exclusive prefixes: each thread loads a run of up to kElemPartPer
// consecutive chunks at once (one round trip), folds it, then a workgroup
// scan of the runs, and writes the run's prefixes back from registers.
constexpr int kElemPartThreads = 1024, kElemPartPer = 8;
constexpr int kElemMaxChunks = kElemPartThreads * kElemPartPer;

template <class T, class Op, int W>
__global__ __launch_bounds__(kElemPartThreads) void k_elem_partials(ElemArgs a) {
    using C = typename Carry<T, Op>::type;
    __shared__ C tot[kElemPartThreads / kWave];
    const uint32_t seg = blockIdx.x / W, comp = blockIdx.x % W;
    C *part = reinterpret_cast<C *>(a.partials) + int64_t(seg) * a.chunks * W + comp;
    const C id = Op::template identity<C>();
    const uint32_t per = (a.chunks + kElemPartThreads - 1) / kElemPartThreads;  // <= kElemPartPer
    const uint32_t c0 = threadIdx.x * per;
    C x[kElemPartPer];
#pragma unroll
    for (int i = 0; i < kElemPartPer; i++)
        x[i] = (uint32_t(i) < per && c0 + i < a.chunks) ? part[int64_t(c0 + i) * W] : id;
    C run = id;
#pragma unroll
    for (int i = 0; i < kElemPartPer; i++) run = Op::apply(run, x[i]);
    const int wave = threadIdx.x / kWave;
    const C inc = wave_scan_incl<Op>(run);
    if (lane_id() == kWave - 1) tot[wave] = inc;
    __syncthreads();
    C base = id;
    for (int w = 0; w < wave; w++) base = Op::apply(base, tot[w]);
    C ex = Op::apply(base, wave_shr1(id, inc));
#pragma unroll
    for (int i = 0; i < kElemPartPer; i++) {
        if (uint32_t(i) < per && c0 + i < a.chunks) {
            part[int64_t(c0 + i) * W] = ex;
            ex = Op::apply(ex, x[i]);
        }
    }
}

template <class T, class Op, int W, int E, int LG>
static int launch_elem_impl(const ElemArgs &a, int threads, hipStream_t s) {
    using K = ElemTile<T, Op, W, E, LG>;
    if (threads < kWave || threads > kElemMaxThreads || threads % kWave) return SCAN_ERR_UNSUPPORTED;
    if (a.chunks > uint32_t(kElemMaxChunks)) return SCAN_ERR_UNSUPPORTED;
    const uint32_t blocks = a.outer * a.chunks;
    const size_t lds = K::lds_bytes(threads), lds_r = K::lds_bytes_rescan(threads);
    if (lds_r > 65536) {  // above the default dynamic LDS limit (gfx950 has 160 KiB per workgroup)
        if (hipFuncSetAttribute(reinterpret_cast<const void *>(&k_elem_reduce<K>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) != hipSuccess ||
            hipFuncSetAttribute(reinterpret_cast<const void *>(&k_elem_rescan<K>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(lds_r)) != hipSuccess)
            return SCAN_ERR_HIP;
    }
    hipLaunchKernelGGL((k_elem_reduce<K>), dim3(blocks), dim3(threads), lds, s, a);
    if (hipGetLastError() != hipSuccess) return SCAN_ERR_HIP;
    hipLaunchKernelGGL((k_elem_partials<T, Op, W>), dim3(a.outer * W), dim3(kElemPartThreads), 0, s, a);
    if (hipGetLastError() != hipSuccess) return SCAN_ERR_HIP;
    hipLaunchKernelGGL((k_elem_rescan<K>), dim3(blocks), dim3(threads), lds_r, s, a);
    return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
}

// Variants per width: E = elem_e_max(W) or 1, 16-byte accesses (when W
// components span whole 16-byte vectors) or element-wide ones.
template <class T, class Op, int W>
static ElemLaunch pick_elem_variant(int e, bool vec) {
    constexpr int EM = elem_e_max(W);
    constexpr bool kVecOk = (W * int(sizeof(T))) % 16 == 0;
    if (vec) {
        if constexpr (kVecOk) {
            if (e == EM) return &launch_elem_impl<T, Op, W, EM, 16>;
            if (e == 1) return &launch_elem_impl<T, Op, W, 1, 16>;
        }
        return nullptr;
    }
    if (e == EM) return &launch_elem_impl<T, Op, W, EM, int(sizeof(T))>;
    if (e == 1) return &launch_elem_impl<T, Op, W, 1, int(sizeof(T))>;
    return nullptr;
}

// Built widths: small vectors and the struct shapes of the measured configs
// (24 x fp32 = 96 B, 17 x fp64 = 136 B); any other width is scanned by the
// column kernel.
template <class T, class Op>
static ElemLaunch pick_width(int w, int e, bool vec) {
    switch (w) {
    case 2: return pick_elem_variant<T, Op, 2>(e, vec);
    case 3: return pick_elem_variant<T, Op, 3>(e, vec);
    case 4: return pick_elem_variant<T, Op, 4>(e, vec);
    case 8: return pick_elem_variant<T, Op, 8>(e, vec);
    case 16: return pick_elem_variant<T, Op, 16>(e, vec);
    case 17: return pick_elem_variant<T, Op, 17>(e, vec);
    case 24: return pick_elem_variant<T, Op, 24>(e, vec);
    }
    return nullptr;
}

template <class T>
static ElemLaunch pick_elem_op(scan_op_t op, int w, int e, bool vec) {
    switch (op) {
    case SCAN_OP_SUM: return pick_width<T, OpSum>(w, e, vec);
    case SCAN_OP_PROD: return pick_width<T, OpProd>(w, e, vec);
    case SCAN_OP_MAX: return pick_width<T, OpMax>(w, e, vec);
    case SCAN_OP_MIN: return pick_width<T, OpMin>(w, e, vec);
    }
    return nullptr;
}

#if SW64_DT == 0
ElemLaunch find_element_i32(scan_op_t op, int w, int e, bool vec) { return pick_elem_op<int32_t>(op, w, e, vec); }
#elif SW64_DT == 1
ElemLaunch find_element_u32(scan_op_t op, int w, int e, bool vec) { return pick_elem_op<uint32_t>(op, w, e, vec); }
#elif SW64_DT == 2
ElemLaunch find_element_i64(scan_op_t op, int w, int e, bool vec) { return pick_elem_op<int64_t>(op, w, e, vec); }
#elif SW64_DT == 3
ElemLaunch find_element_f32(scan_op_t op, int w, int e, bool vec) { return pick_elem_op<float>(op, w, e, vec); }
#elif SW64_DT == 4
ElemLaunch find_element_f64(scan_op_t op, int w, int e, bool vec) { return pick_elem_op<double>(op, w, e, vec); }
#else
#error "SW64_DT must select an element type (0..4)"
#endif

}  // namespace sw64
