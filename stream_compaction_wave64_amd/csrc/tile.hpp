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
    int64_t rem;          // elements of the tile in range (>= TILE: all)

    __device__ __forceinline__ static int64_t elem(int r) {
        return (int64_t(r) * BLOCK + threadIdx.x) * VEC;
    }

    // Issue the tile's loads.  No loaded value is read here: the registers
    // are first touched by scan() or reduce(), so a pipelined caller keeps
    // the loads in flight while it works on other tiles (a select applied at
    // load time would make the compiler wait for the data right away).
    // Out-of-range rows re-read the tile's first vector (always in range), so
    // every load is unconditional.  The caller guarantees `remaining` is a
    // multiple of VEC.
    __device__ __forceinline__ void load(const T *src, int64_t remaining) {
        rem = remaining;
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            const int64_t e = elem(r);
            v[r] = load_vec<T, VEC>(src + (e < remaining ? e : 0));
        }
    }

    // Identity in every vector at or past the end (only the last tile of a
    // segment has any).
    __device__ __forceinline__ void mask_tail() {
        if (rem >= TILE) return;
        const T id = Op::template identity<T>();
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            const bool in = elem(r) < rem;
#pragma unroll
            for (int c = 0; c < VEC; c++) v[r].v[c] = in ? v[r].v[c] : id;
        }
    }

    // Levels 1-3 above.  Contains one __syncthreads().
    __device__ __forceinline__ void scan(Shared &sh) {
        mask_tail();
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

    // The tile aggregate from the per-wave totals scan() left in LDS, in the
    // carry type, computed by any one whole wave after scan()'s barrier (the
    // same value in every lane).  Operators are commutative.
    template <class C2>
    __device__ __forceinline__ static C2 aggregate_from(const Shared &sh) {
        C2 acc = Op::template identity<C2>();
        for (int i = lane_id(); i < ROWS * W; i += kWave) acc = Op::apply(acc, C2(sh.tot[i / W][i % W]));
        return wave_reduce<Op>(acc);
    }

    // Tile aggregate only (the reduce pass of reduce-then-scan): per-thread
    // reduction of all its elements, wave reduction, one LDS slot per wave.
    // Contains one __syncthreads(); the caller separates reuses of `sh`.
    __device__ __forceinline__ void reduce(Shared &sh) {
        mask_tail();
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

    // After scan(): replace every value by its tile-local result (inclusive,
    // or exclusive with the identity before the tile's first element), i.e.
    // the output less the tile's prefix.
    __device__ __forceinline__ void fold(bool exclusive) {
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            T prev = off[r];
#pragma unroll
            for (int c = 0; c < VEC; c++) {
                const T inc = Op::apply(off[r], v[r].v[c]);
                v[r].v[c] = exclusive ? prev : inc;
                prev = inc;
            }
        }
    }

    // Store fold()ed values with the tile's prefix `pre` applied (in the
    // carry type, rounded once).  Rows at or past `remaining` are dropped.
    template <int AUX = 2>  // the stores' cache policy (see store_vec_bounded)
    __device__ __forceinline__ static void store_folded(const Vec<T, VEC> (&w)[ROWS], T *dst, int64_t remaining,
                                                        C pre) {
        const BufRsrc rs = make_rsrc(dst, remaining < TILE ? (remaining > 0 ? remaining : 0) : TILE);
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            Vec<T, VEC> o;
#pragma unroll
            for (int c = 0; c < VEC; c++) o.v[c] = T(Op::apply(pre, C(w[r].v[c])));
            store_vec_bounded<T, VEC, AUX>(rs, uint32_t(elem(r) * int64_t(sizeof(T))), o);
        }
    }

    // Add the tile's exclusive prefix `pre` and store; inclusive or exclusive.
    // Every store is issued (no branch): rows at or past `remaining` fall
    // outside the buffer resource's range and the hardware drops them.
    __device__ __forceinline__ void store(T *dst, int64_t remaining, C pre, bool exclusive) const {
        const BufRsrc rs = make_rsrc(dst, remaining < TILE ? (remaining > 0 ? remaining : 0) : TILE);
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
            store_vec_bounded<T, VEC>(rs, uint32_t(elem(r) * int64_t(sizeof(T))), o);
        }
    }
};

}  // namespace sw64
