// Weighted combine: y[t] = sum_j w[t][j] * y_perm[row_of_slot[t*k + j]].
//
// There is no shared expert (teardown, "How Is the Backbone Built?"; devupai
// "No shared expert"), so the routed sum is the whole layer output.
#include "moe_internal.h"

namespace moe {

typedef uint32_t v2u __attribute__((ext_vector_type(2)));

__global__ void __launch_bounds__(512) combine_kernel(const float* __restrict__ y_perm,
                                                      const int32_t* __restrict__ row_of_slot,
                                                      const float* __restrict__ w, void* __restrict__ y,
                                                      int out_bf16, int T, int H, int k) {
    const int t = blockIdx.x;
    int rows[8];
    float ws[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        rows[j] = row_of_slot[(size_t)t * k + min(j, k - 1)];
        ws[j] = j < k ? w[(size_t)t * k + j] : 0.0f;
    }
    // a slot without a row (row -1: moe_permute was given an expert id out of
    // range, which its error word reports), or with a row outside the T*k rows
    // of y_perm, adds nothing and is not loaded
    bool has[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) has[j] = (unsigned)rows[j] < (unsigned)(T * k);
    // workgroup (t, b) covers channels [2048 b, 2048 b + 2048): a decode step
    // with few tokens still spreads over the whole chip.  All eight loads are
    // issued before the first FMA (slots past k re-read slot k-1 with weight
    // 0, which leaves the sum unchanged but for the sign of an all-zero sum),
    // and they bypass the caches: y_perm is read once.  The stores of y bypass
    // them too (on Pro skewed prefill, 384 MiB of y: combine 732 -> 687 us).
    for (int c = (blockIdx.y * 512 + threadIdx.x) * 4; c < H; c += gridDim.y * 512 * 4) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        v4f v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            v[j] = has[j] ? __builtin_nontemporal_load((const v4f*)(y_perm + (size_t)rows[j] * H + c))
                          : v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            acc[0] = fmaf(ws[j], v[j][0], acc[0]);
            acc[1] = fmaf(ws[j], v[j][1], acc[1]);
            acc[2] = fmaf(ws[j], v[j][2], acc[2]);
            acc[3] = fmaf(ws[j], v[j][3], acc[3]);
        }
        if (out_bf16) {
            v2u o;
            o.x = (uint32_t)float_to_bf16_rne(acc[0]) | ((uint32_t)float_to_bf16_rne(acc[1]) << 16);
            o.y = (uint32_t)float_to_bf16_rne(acc[2]) | ((uint32_t)float_to_bf16_rne(acc[3]) << 16);
            __builtin_nontemporal_store(o, (v2u*)((uint16_t*)y + (size_t)t * H + c));
        } else {
            __builtin_nontemporal_store(acc, (v4f*)((float*)y + (size_t)t * H + c));
        }
    }
}

hipError_t launch_combine(const float* y_perm, const int32_t* row_of_slot, const float* w, void* y, int out_bf16,
                          int64_t T, int H, int k, hipStream_t stream) {
    // few tokens (decode): spread each token over channel blocks of 2048 so
    // the combine still covers the chip; many tokens: one workgroup per token
    // (fewer, longer workgroups: Flash prefill 238 -> 222 us), of 512 threads
    // (Pro skewed prefill 679 -> 667 us against 256 threads)
    const unsigned cb = T >= 2048 ? 1u : (unsigned)((H + 2047) / 2048);
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)T, cb), dim3(512), 0, stream, y_perm, row_of_slot, w, y, out_bf16,
                       (int)T, H, k);
    return hipGetLastError();
}

}  // namespace moe
