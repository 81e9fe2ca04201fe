// util.hip -- fill kernels (workspace initialisation, empty outputs) and the
// copy kernel that measures the attainable read+write bandwidth of the part:
// the fastest plain copy measured on MI355X.
#include <mutex>

#include "device.hpp"
#include "launch.hpp"

namespace sw64 {

int resident_blocks(const void *kernel, int waves_per_block) {
    static std::mutex mu;
    static const void *keys[512];
    static int devs[512], vals[512], count = 0;
    const int block = waves_per_block * kWave;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < count; i++)
        if (keys[i] == kernel && devs[i] == dev) return vals[i];
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    // At most 6 waves per SIMD (24 per compute unit).  A grid at the bound
    // the kernel's resources set was measured not to start at once: 8 waves
    // per SIMD for small 4-byte kernels, 7 for the 64-bit look-back kernels
    // of 256 threads (102-104 scalar registers, 64-71 vector registers; every
    // call fell back to dynamic claiming until the grid was capped here).
    // Default shapes hold one large workgroup per compute unit and are not
    // affected.
    if (per_cu * waves_per_block > 24) per_cu = 24 / waves_per_block > 0 ? 24 / waves_per_block : 1;
    const int v = per_cu * cus;
    if (count < 512) {
        keys[count] = kernel;
        devs[count] = dev;
        vals[count] = v;
        count++;
    }
    return v;
}

// Fill `words` 64-bit words with `value`, except word `at` (if < words),
// which gets `at_value`.
__global__ __launch_bounds__(256) void k_fill_u64(uint64_t *p, uint64_t words, uint64_t value, uint64_t at,
                                                   uint64_t at_value) {
    for (uint64_t i = uint64_t(blockIdx.x) * 256 + threadIdx.x; i < words; i += uint64_t(gridDim.x) * 256)
        p[i] = i == at ? at_value : value;
}

__global__ __launch_bounds__(256) void k_fill_i32(int32_t *p, int64_t count, int32_t value) {
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < count; i += int64_t(gridDim.x) * 256)
        p[i] = value;
}

int launch_fill_u64(void *p, uint64_t words, uint64_t value, hipStream_t s, uint64_t at, uint64_t at_value) {
    if (words == 0) return SCAN_OK;
    const uint64_t blocks = (words + 255) / 256;
    hipLaunchKernelGGL(k_fill_u64, dim3(unsigned(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s,
                       reinterpret_cast<uint64_t *>(p), words, value, at, at_value);
    return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
}

int launch_fill_i32(int32_t *p, int64_t count, int32_t value, hipStream_t s) {
    if (count <= 0) return SCAN_OK;
    const int64_t blocks = (count + 255) / 256;
    hipLaunchKernelGGL(k_fill_i32, dim3(unsigned(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s, p, count,
                       value);
    return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
}

// Copy ceiling: one 16-byte vector per thread, 256 threads (4 KiB) per
// workgroup, nontemporal loads and stores.  Among the copies measured on
// MI355X (400 MB each way) this was the fastest, about 81 % of 8 TB/s:
// workgroups of 8 rows (32 KiB) reached 74-76 %, the scan's 77 KiB tiles
// 73 %, persistent grids 66-77 %.  Writes are what suffers: a write-only
// pass ran at 80 % with one vector per thread and 65 % with eight.
constexpr int kCopyBlock = 256, kCopyRows = 1;

__global__ __launch_bounds__(kCopyBlock) void k_copy16(const uint32_t *in, uint32_t *out, int64_t vecs) {
    const int64_t base = int64_t(blockIdx.x) * kCopyBlock * kCopyRows;
    Vec<uint32_t, 4> x[kCopyRows];
#pragma unroll
    for (int r = 0; r < kCopyRows; r++) {
        const int64_t i = base + int64_t(r) * kCopyBlock + threadIdx.x;
        x[r] = load_vec<uint32_t, 4>(in + 4 * (i < vecs ? i : base));
    }
#pragma unroll
    for (int r = 0; r < kCopyRows; r++) {
        const int64_t i = base + int64_t(r) * kCopyBlock + threadIdx.x;
        if (i < vecs) store_vec<uint32_t, 4>(out + 4 * i, x[r]);
    }
}

int launch_copy(const void *in, void *out, size_t bytes, hipStream_t s) {
    const int64_t vecs = int64_t(bytes / 16);
    if (vecs == 0) return SCAN_OK;
    const int64_t per = int64_t(kCopyBlock) * kCopyRows;
    const int64_t blocks = (vecs + per - 1) / per;
    hipLaunchKernelGGL(k_copy16, dim3(unsigned(blocks)), dim3(kCopyBlock), 0, s,
                       reinterpret_cast<const uint32_t *>(in), reinterpret_cast<uint32_t *>(out), vecs);
    return hipGetLastError() == hipSuccess ? SCAN_OK : SCAN_ERR_HIP;
}

}  // namespace sw64
