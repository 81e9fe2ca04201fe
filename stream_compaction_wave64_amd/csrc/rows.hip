// rows.hip -- scans of many rows that each fit one tile: scan_dim along the
// contiguous axis of an (outer, len) array (AcceleratedKernels.jl PR #208:
// accumulate along a dimension; the 4096 x 4096 "along rows" case), and the
// segmented scan of The CUDA Handbook ch. 13 in its simplest form, where a
// segment never spans two tiles.
//
// One workgroup per row, with no inter-workgroup traffic at all: it loads the
// row with 128-bit accesses, scans it with the register tile of tile.hpp
// (thread-serial, DPP wave scans, one LDS slot per wave and tile row), and
// stores it.  No descriptors, no control wave, no persistent grid: the
// memory system sees the traffic of a plain copy, and the many workgroups per
// compute unit hide each other's load latency.  The look-back pipeline would
// treat each row as one tile whose prefix is the identity, and pay for its
// stash, barriers and idle control wave (4096 x 4096 fp32: 26.3 -> 24.1 us
// per call).  Two rows per workgroup, both rows' loads issued before either
// scan, measured the same.
//
// This file is compiled once per element type (SW64_DT selects it).
#include "launch.hpp"
#include "tile.hpp"

namespace sw64 {

template <class T, class Op, int ROWS>
__global__ __launch_bounds__(kRowsBlock) void k_rows(RowsArgs a) {
    constexpr int VEC = 16 / int(sizeof(T));
    using TS = TileScan<T, Op, kRowsBlock, ROWS, VEC>;
    __shared__ typename TS::Shared sh;
    const int64_t base = int64_t(blockIdx.x) * a.len;
    TS ts;
    ts.load(reinterpret_cast<const T *>(a.in) + base, a.len);
    ts.scan(sh);
    // the row's results: no prefix before its first element; vectors past
    // its end fall outside the buffer resource and are dropped
    const BufRsrc rs = make_rsrc(reinterpret_cast<T *>(a.out) + base, a.len);
    const T id = Op::template identity<T>();
#pragma unroll
    for (int r = 0; r < ROWS; r++) {
        Vec<T, VEC> o;
        T prev = id;
#pragma unroll
        for (int c = 0; c < VEC; c++) {
            const T cur = ts.v[r].v[c];
            o.v[c] = Op::apply(ts.off[r], a.exclusive ? prev : cur);
            prev = cur;
        }
        // the row step in the vector offset, the scalar offset a constant 0
        // (128-bit buffer stores with a scalar-register offset lost their
        // data registers)
        uint32_t vo = uint32_t(TS::elem(r) * int64_t(sizeof(T)));
        asm volatile("" : "+v"(vo));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, o), rs, vo, 0, 2);
    }
}

template <class T, class Op, int ROWS>
static int launch_rows_impl(const RowsArgs &a, hipStream_t s) {
    constexpr int VEC = 16 / int(sizeof(T));
    if (a.len < 1 || a.len > int64_t(kRowsBlock) * ROWS * VEC || a.len % VEC != 0 || a.rows < 1 ||
        a.rows > uint64_t(INT32_MAX))
        return SCAN_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((k_rows<T, Op, ROWS>), dim3(uint32_t(a.rows)), dim3(kRowsBlock), 0, s, a);
    return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
}

template <class T, class Op>
static RowsLaunch pick_rows_shape(int rows) {
    switch (rows) {
    case 1: return &launch_rows_impl<T, Op, 1>;
    case 2: return &launch_rows_impl<T, Op, 2>;
    case 4: return &launch_rows_impl<T, Op, 4>;
    case 8: return &launch_rows_impl<T, Op, 8>;
    }
    return nullptr;
}

template <class T>
static RowsLaunch pick_rows(scan_op_t op, int rows) {
    switch (op) {
    case SCAN_OP_SUM: return pick_rows_shape<T, OpSum>(rows);
    case SCAN_OP_PROD: return pick_rows_shape<T, OpProd>(rows);
    case SCAN_OP_MAX: return pick_rows_shape<T, OpMax>(rows);
    case SCAN_OP_MIN: return pick_rows_shape<T, OpMin>(rows);
    }
    return nullptr;
}

#if SW64_DT == 0
RowsLaunch find_rows_i32(scan_op_t op, int rows) { return pick_rows<int32_t>(op, rows); }
#elif SW64_DT == 1
RowsLaunch find_rows_u32(scan_op_t op, int rows) { return pick_rows<uint32_t>(op, rows); }
#elif SW64_DT == 2
RowsLaunch find_rows_i64(scan_op_t op, int rows) { return pick_rows<int64_t>(op, rows); }
#elif SW64_DT == 3
RowsLaunch find_rows_f32(scan_op_t op, int rows) { return pick_rows<float>(op, rows); }
#elif SW64_DT == 4
RowsLaunch find_rows_f64(scan_op_t op, int rows) { return pick_rows<double>(op, rows); }
#else
#error "SW64_DT must select an element type (0..4)"
#endif

}  // namespace sw64
