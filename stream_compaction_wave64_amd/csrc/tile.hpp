// tile.hpp -- the per-tile body shared by the look-back and reduce-then-scan
// kernels.
//
// A tile is ROWS rows of BLOCK*VEC consecutive elements.  Row r of the tile
// is read by one vector instruction per thread: thread t holds elements
// [(r*BLOCK + t)*VEC, +VEC), so each wave instruction moves 64 contiguous
// 128-bit vectors (1 KiB) and every access is fully coalesced.  The tile is
// scanned in three levels, all in registers except one LDS slot per wave and
// row:
//   1. each thread scans its VEC elements serially (items-per-thread
//      register blocking, The CUDA Handbook ch. 13 section 13.3.5);
//   2. the per-thread totals of each row are scanned across the wave with
//      the DPP Kogge-Stone scan (ROWS independent scans, interleaved);
//   3. the last lane of each wave stores its row totals to LDS; after one
//      barrier every thread combines the ROWS x W totals in tile order to
//      get its row offsets and the tile aggregate (one slot per wave, as in
//      AcceleratedKernels.jl PR #208, second bullet).
// Unlike the page's kernel, no LDS transpose is needed: every element keeps
// the register it was loaded into until it is stored.
#pragma once

#include "device.hpp"

namespace sw64 {

template <class T, class Op, int BLOCK, int ROWS, int VEC>
struct TileScan {
    static_assert(BLOCK % kWave == 0 && BLOCK <= 1024, "block must be whole waves");
    static constexpr int W = BLOCK / kWave;
    static constexpr int64_t TILE = int64_t(BLOCK) * ROWS * VEC;
    using C = typename Carry<T, Op>::type;

    struct Shared {
        T tot[ROWS][W];
    };

    Vec<T, VEC> v[ROWS];  // loaded values, then their in-vector inclusive scan
    T off[ROWS];          // exclusive offset of this thread's vector in each row
    T agg;                // tile aggregate

    __device__ __forceinline__ static int64_t elem(int r) {
        return (int64_t(r) * BLOCK + threadIdx.x) * VEC;
    }

    // Load the tile; vectors at or past `remaining` hold the identity.  The
    // caller guarantees remaining is a multiple of VEC.
    __device__ __forceinline__ void load(const T *src, int64_t remaining) {
        // Out-of-range rows re-read the tile's first vector (always in range)
        // so every load is unconditional and all of them are in flight at once.
        const T id = Op::template identity<T>();
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            const int64_t e = elem(r);
            const bool in = e < remaining;
            const Vec<T, VEC> x = load_vec<T, VEC>(src + (in ? e : 0));
#pragma unroll
            for (int c = 0; c < VEC; c++) v[r].v[c] = in ? x.v[c] : id;
        }
    }

    // Levels 1-3 above.  Contains one __syncthreads().
    __device__ __forceinline__ void scan(Shared &sh) {
        const T id = Op::template identity<T>();
        const int lane = lane_id();
        const int wave = threadIdx.x / kWave;
        T tot[ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            T acc = v[r].v[0];
#pragma unroll
            for (int c = 1; c < VEC; c++) {
                acc = Op::apply(acc, v[r].v[c]);
                v[r].v[c] = acc;
            }
            tot[r] = acc;
        }
        T winc[ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; r++) winc[r] = wave_scan_incl<Op>(tot[r]);
        if (lane == kWave - 1) {
#pragma unroll
            for (int r = 0; r < ROWS; r++) sh.tot[r][wave] = winc[r];
        }
        __syncthreads();
        T run = id;
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            const T row_start = run;
            T wbase = id;
#pragma unroll
            for (int w = 0; w < W; w++) {
                const T t = sh.tot[r][w];
                if (w < wave) wbase = Op::apply(wbase, t);
                run = Op::apply(run, t);
            }
            off[r] = Op::apply(Op::apply(row_start, wbase), wave_shr1(id, winc[r]));
        }
        agg = run;
    }

    // Tile aggregate only (the reduce pass of reduce-then-scan): per-thread
    // reduction of all its elements, wave reduction, one LDS slot per wave.
    // Contains one __syncthreads(); the caller separates reuses of `sh`.
    __device__ __forceinline__ void reduce(Shared &sh) {
        const T id = Op::template identity<T>();
        T acc = id;
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
#pragma unroll
            for (int c = 0; c < VEC; c++) acc = Op::apply(acc, v[r].v[c]);
        }
        const T w = wave_reduce<Op>(acc);
        if (lane_id() == 0) sh.tot[0][threadIdx.x / kWave] = w;
        __syncthreads();
        T run = id;
#pragma unroll
        for (int k = 0; k < W; k++) run = Op::apply(run, sh.tot[0][k]);
        agg = run;
    }

    // Add the tile's exclusive prefix `pre` and store; inclusive or exclusive.
    __device__ __forceinline__ void store(T *dst, int64_t remaining, C pre, bool exclusive) const {
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            const T base = T(Op::apply(pre, C(off[r])));
            Vec<T, VEC> o;
            T prev = Op::template identity<T>();
#pragma unroll
            for (int c = 0; c < VEC; c++) {
                const T cur = v[r].v[c];
                o.v[c] = Op::apply(base, exclusive ? prev : cur);
                prev = cur;
            }
            const int64_t e = elem(r);
            if (e < remaining) store_vec<T, VEC>(dst + e, o);
        }
    }
};

}  // namespace sw64
