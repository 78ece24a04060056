// Weighted combine: y[t] = sum_j w[t][j] * y_perm[row_of_slot[t*k + j]].
//
// There is no shared expert (teardown, "How Is the Backbone Built?"; devupai
// "No shared expert"), so the routed sum is the whole layer output.
#include "moe_internal.h"

namespace moe {

__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ y_perm,
                                                      const int32_t* __restrict__ row_of_slot,
                                                      const float* __restrict__ w, void* __restrict__ y,
                                                      int out_bf16, int T, int H, int k) {
    const int t = blockIdx.x;
    int rows[8];
    float ws[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        rows[j] = j < k ? row_of_slot[(size_t)t * k + j] : -1;
        ws[j] = j < k ? w[(size_t)t * k + j] : 0.0f;
    }
    // workgroup (t, b) covers channels [1024 b, 1024 b + 1024): a decode step
    // with few tokens still spreads over the whole chip
    for (int c = (blockIdx.y * 256 + threadIdx.x) * 4; c < H; c += gridDim.y * 256 * 4) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j < k && rows[j] >= 0) {
                const v4f v = *(const v4f*)(y_perm + (size_t)rows[j] * H + c);
                acc[0] = fmaf(ws[j], v[0], acc[0]);
                acc[1] = fmaf(ws[j], v[1], acc[1]);
                acc[2] = fmaf(ws[j], v[2], acc[2]);
                acc[3] = fmaf(ws[j], v[3], acc[3]);
            }
        }
        if (out_bf16) {
            uint2 o;
            o.x = (uint32_t)float_to_bf16_rne(acc[0]) | ((uint32_t)float_to_bf16_rne(acc[1]) << 16);
            o.y = (uint32_t)float_to_bf16_rne(acc[2]) | ((uint32_t)float_to_bf16_rne(acc[3]) << 16);
            *(uint2*)((uint16_t*)y + (size_t)t * H + c) = o;
        } else {
            *(v4f*)((float*)y + (size_t)t * H + c) = acc;
        }
    }
}

hipError_t launch_combine(const float* y_perm, const int32_t* row_of_slot, const float* w, void* y, int out_bf16,
                          int64_t T, int H, int k, hipStream_t stream) {
    const unsigned cb = (unsigned)((H + 1023) / 1024);
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)T, cb), dim3(256), 0, stream, y_perm, row_of_slot, w, y, out_bf16,
                       (int)T, H, k);
    return hipGetLastError();
}

}  // namespace moe
