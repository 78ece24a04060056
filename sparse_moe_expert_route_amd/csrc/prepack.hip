// Packed weight layout (moe.h, MOE_WEIGHTS_PACKED): a pure byte permutation
// of the e2m1 code bytes and of their e8m0 scale bytes, done once when
// weights are loaded.  Each output 1 KB code block holds 16 rows x 64 bytes
// so that a 64-lane load of 16 bytes per lane covers whole cache lines; the
// canonical layout gives the same load only 16 or 32 bytes of each of 16-32
// lines.  Each 64-byte scale block holds the 4 scale bytes of those 16 rows
// for the same 128 columns, so that the scales a wave needs for a stretch of
// K are a few whole lines.
#include "moe_internal.h"

namespace moe {

// one 16-byte unit per thread, destination order (coalesced writes)
__global__ void __launch_bounds__(256) prepack_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                      int64_t units, int K) {
    const int64_t steps = K / 128;                 // 1 KB blocks per 16-row group
    const int64_t row_units = K / 32;              // 16-byte units per row
    for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < units;
         d += (int64_t)gridDim.x * blockDim.x) {
        const int64_t block = d >> 6;
        const int within = (int)(d & 63), p = within >> 4, r = within & 15;
        const int64_t q = block / steps, c = block - q * steps;
        dst[d] = src[(16 * q + r) * row_units + 4 * c + p];
    }
}

// one scale dword (4 bytes = one row's scales of 128 columns) per thread,
// destination order
__global__ void __launch_bounds__(256) prepack_scales_kernel(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst,
                                                             int64_t units, int K) {
    const int64_t steps = K / 128;                 // 64-byte blocks per 16-row group
    for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < units;
         d += (int64_t)gridDim.x * blockDim.x) {
        const int64_t block = d >> 4;
        const int r = (int)(d & 15);
        const int64_t q = block / steps, c = block - q * steps;
        dst[d] = src[(16 * q + r) * steps + c];
    }
}

static unsigned grid_for(int64_t units) {
    const int64_t blocks = (units + 255) / 256;
    return (unsigned)(blocks < 65536 ? blocks : 65536);
}

hipError_t launch_prepack(const uint8_t* src, uint8_t* dst, int64_t rows, int K, hipStream_t stream) {
    const int64_t units = rows * (K / 32);
    hipLaunchKernelGGL(prepack_kernel, dim3(grid_for(units)), dim3(256), 0, stream, (const uint4*)src, (uint4*)dst, units, K);
    return hipGetLastError();
}

hipError_t launch_prepack_scales(const uint8_t* src, uint8_t* dst, int64_t rows, int K, hipStream_t stream) {
    const int64_t units = rows * (K / 128);
    hipLaunchKernelGGL(prepack_scales_kernel, dim3(grid_for(units)), dim3(256), 0, stream, (const uint32_t*)src,
                       (uint32_t*)dst, units, K);
    return hipGetLastError();
}

}  // namespace moe
