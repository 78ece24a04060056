// FP8 quantisation of one bf16 row by one 256-thread workgroup, shared by the
// quant-gather kernel and the decode router launch.
//
// 8 channels (one 16-byte bf16 load) per thread, so a 128-channel block is 16
// consecutive lanes: amax by xor-shuffles within the 16, then the shared block
// exponent, then RNE e4m3 codes of x * 2^-e (an exact power-of-two scaling).
// F32S (FP8 block-scaled experts): the block's float32 scale amax / 448 and
// RNE e4m3 codes of x / scale.
#pragma once

#include "moe_internal.h"

namespace moe {

template <bool F32S>
__device__ __forceinline__ void quantise_row(const uint16_t* __restrict__ xr, uint8_t* __restrict__ xq,
                                             void* __restrict__ xs, int r, int H) {
    uint8_t* qr = xq + (size_t)r * H;
    for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
        const uint4 raw = *(const uint4*)(xr + c);
        float v[8];
        v[0] = bf16_bits_to_float(raw.x & 0xFFFFu); v[1] = bf16_bits_to_float(raw.x >> 16);
        v[2] = bf16_bits_to_float(raw.y & 0xFFFFu); v[3] = bf16_bits_to_float(raw.y >> 16);
        v[4] = bf16_bits_to_float(raw.z & 0xFFFFu); v[5] = bf16_bits_to_float(raw.z >> 16);
        v[6] = bf16_bits_to_float(raw.w & 0xFFFFu); v[7] = bf16_bits_to_float(raw.w >> 16);
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
        float q[8];
        if constexpr (F32S) {
            // float32 scale amax / 448 (FP8 block-scaled experts)
            const float sc = fp8_f32_scale(amax);
            const float d = amax > 0.0f ? sc : 1.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = fp8_f32_quotient(v[i], d);
            if ((threadIdx.x & 15) == 0) ((float*)xs)[(size_t)r * (H / kFp8Block) + c / kFp8Block] = sc;
        } else {
            const int e = fp8_block_exponent(amax);
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = __builtin_amdgcn_ldexpf(v[i], -e);
            if ((threadIdx.x & 15) == 0) ((uint8_t*)xs)[(size_t)r * (H / kFp8Block) + c / kFp8Block] = (uint8_t)(e + 127);
        }
        uint2 codes;
        codes.x = pack_fp8x4(q[0], q[1], q[2], q[3]);
        codes.y = pack_fp8x4(q[4], q[5], q[6], q[7]);
        *(uint2*)(qr + c) = codes;
    }
}

}  // namespace moe
