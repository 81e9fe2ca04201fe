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
#include "launch.hpp"
#include "tile.hpp"

namespace sw64 {

template <class X, int CMP>
__device__ __forceinline__ bool keep(X v, X t) {
    if constexpr (CMP == SCAN_CMP_GT) return v > t;
    else if constexpr (CMP == SCAN_CMP_GE) return v >= t;
    else if constexpr (CMP == SCAN_CMP_LT) return v < t;
    else if constexpr (CMP == SCAN_CMP_LE) return v <= t;
    else if constexpr (CMP == SCAN_CMP_EQ) return v == t;
    else return v != t;
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

    // A scanned tile waiting for its prefix: every thread's row offsets and
    // selection bits.
    struct Stash {
        int32_t off[ROWS][BLOCK];
        uint32_t bits[BLOCK];
    };

    // Each selected element's index at its position.
    __device__ __forceinline__ static void emit(const Stash &st, const Args &a, uint32_t tile, C pre, bool valid) {
        if (!valid) return;
        const int64_t start = int64_t(tile) * TS::TILE;
        const uint32_t bits = st.bits[threadIdx.x];
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
            const int64_t e = TS::elem(r);
            int32_t pos = pre + st.off[r][threadIdx.x];
#pragma unroll
            for (int c = 0; c < VEC; c++) {
                if (bits & (1u << (r * VEC + c))) {
                    a.out_idx[pos] = int32_t(start + e + c);
                    pos++;
                }
            }
        }
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
            for (int r = 0; r < ROWS; r++) st.off[r][threadIdx.x] = ts.off[r];
            st.bits[threadIdx.x] = bits;
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

// Shapes: the default 512 x 8 rows of 4 (tile 16384) and 256 x 1 (small
// tiles for tests); element-wide variants for misaligned x.
template <class X, int CMP>
static CompactLaunch pick_compact_shape(int block, int rows, int vec) {
    if (vec == 4) {
        if (block == 512 && rows == 8) return &launch_compact_impl<X, CMP, 512, 8, 4>;
        if (block == 256 && rows == 1) return &launch_compact_impl<X, CMP, 256, 1, 4>;
    } else if (vec == 1) {
        if (block == 512 && rows == 8) return &launch_compact_impl<X, CMP, 512, 8, 1>;
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
    }
    return nullptr;
}

CompactLaunch find_compact(scan_dtype_t dt, scan_cmp_t cmp, int block, int rows, int vec) {
    if (dt == SCAN_F32) return pick_compact_cmp<float>(cmp, block, rows, vec);
    if (dt == SCAN_I32) return pick_compact_cmp<int32_t>(cmp, block, rows, vec);
    return nullptr;
}

// ------------------------------------------------------------------- emit
// One thread per object; the record value starts at (i + 1) mod n and wraps
// at n without a division per record.
__global__ __launch_bounds__(256) void k_emit_neighbors(const int32_t *offsets, int64_t n, int32_t *out) {
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
        const int32_t b = offsets[i], e = offsets[i + 1];
        int64_t r = (i + 1 == n) ? 0 : i + 1;
        for (int32_t k = b; k < e; k++) {
            out[k] = int32_t(r);
            r = (r + 1 == n) ? 0 : r + 1;
        }
    }
}

int launch_emit_neighbors(const int32_t *offsets, int64_t n, int32_t *out, hipStream_t s) {
    if (n <= 0) return SCAN_OK;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(k_emit_neighbors, dim3(unsigned(blocks)), dim3(256), 0, s, offsets, n, out);
    return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
}

}  // namespace sw64
