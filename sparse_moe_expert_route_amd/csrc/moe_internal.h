// Internal declarations of the HIP translation units of the MoE library:
// the host-side launch interface (moe_launch.h) plus the device helpers the
// kernels share.  Not part of the public ABI (include/moe.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_launch.h"

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// FP8 block quantisation rule (shared by the activation quantiser and the
// SwiGLU epilogue): scale 2^e with e the smallest integer such that
// amax / 2^e <= 448 = 1.75 * 2^8; written as e8m0 byte e + 127.  With
// amax = m * 2^x, m in [0.5, 1): e = x - 9 if m <= 0.875, else x - 8.
// An all-zero block gets e = -127 (byte 0).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int fp8_block_exponent(float amax) {
    if (!(amax > 0.0f)) return -127;
    int x = __builtin_amdgcn_frexp_expf(amax);
    float m = __builtin_amdgcn_frexp_mantf(amax);
    int e = (m <= 0.875f) ? x - 9 : x - 8;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// FP8 quantisation with a float32 scale (FP8 block-scaled experts): the
// scale of a 128-channel block is amax / 448 and each code is the e4m3
// rounding of v / scale, both IEEE binary32 divisions (hipcc's default fp32
// division is correctly rounded).  The quotient can exceed 448 by one
// rounding; such values round to 448 anyway, and the clamp keeps the
// conversion away from its saturation path.  An all-zero block stores scale
// 0 and divides by 1.
__device__ __forceinline__ float fp8_f32_scale(float amax) { return amax / 448.0f; }
__device__ __forceinline__ float fp8_f32_quotient(float v, float d) { return fminf(fmaxf(v / d, -448.0f), 448.0f); }

// Four floats (already divided by their block scale, |v| <= 448) -> four
// e4m3 bytes, round to nearest even (v_cvt_pk_fp8_f32), byte i = v[i].
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    return (uint32_t)r;
}

// silu(z) = z / (1 + e^-z), with the hardware exponential and reciprocal
// (v_exp_f32, v_rcp_f32: a few ulp) instead of the correctly rounded
// division sequence, which cost the SwiGLU epilogues about ten instructions
// per element.  e^-z overflowing to +inf gives -0, as the division would.
__device__ __forceinline__ float silu_f32(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

__device__ __forceinline__ uint16_t float_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Block-scaled MFMA, A = FP4 (e2m1) weights, B = FP8 (e4m3) activations:
// D[16 weight rows][16 tokens] += sum_k A[row][k] * B[token][k] over 128 k.
// OPSEL_A / OPSEL_B pick the scale byte within each lane's scale register.
template <int OPSEL_A, int OPSEL_B = 0>
__device__ __forceinline__ v4f mfma_w4a8(v8i a, v8i b, v4f c, int scale_a, int scale_b) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, OPSEL_A, scale_a, OPSEL_B, scale_b);
}

// Error bits of caller-given expert offsets (kErrExpertOffsets unless
// 0 = o[0] <= o[1] <= ... <= o[E] = N), evaluated by one wave; every lane
// returns the same value.
__device__ __forceinline__ uint32_t offsets_error(const int32_t* __restrict__ offsets, int E, int64_t N) {
    const int lane = threadIdx.x & 63;
    bool bad = false;
    for (int e = lane; e < E; e += 64) bad |= offsets[e] > offsets[e + 1];
    if (lane == 0) bad |= offsets[0] != 0 || (int64_t)offsets[E] != N;
    return __ballot(bad) ? kErrExpertOffsets : 0u;
}

// M-tile t of kRowsPerTile rows, looked up from the expert offsets alone
// (expert e owns ceil(n_e / 16) tiles, in expert order), so the streaming
// GEMMs need no tile plan.  One wave: lane l sums the tiles of its run of
// ceil(E/64) <= 8 experts, a wave scan finds the lane whose run holds t, and
// that lane's walk over its run gives the expert.  Every lane returns the
// same {expert, first row, rows, 0}, expert -1 for t past the last tile.
// Offsets are clamped to [0, N] and a decreasing pair counts as an empty
// expert, so invalid offsets (reported through offsets_error) still give
// tiles inside the N rows.  Needs E <= 512.
__device__ __forceinline__ int4 find_stream_tile(const int32_t* __restrict__ offsets, int E, int N, int t) {
    const int lane = threadIdx.x & 63;
    const int c = (E + 63) >> 6;
    const int e0 = min(lane * c, E), e1 = min(e0 + c, E);
    int o[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) o[i] = (e0 + i <= e1) ? min(max(offsets[e0 + i], 0), N) : 0;
    int n = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (e0 + i < e1) n += max(o[i + 1] - o[i] + kRowsPerTile - 1, 0) / kRowsPerTile;
    int incl = n;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d, 64);
        if (lane >= d) incl += v;
    }
    const int total = __shfl(incl, 63, 64);
    if (t >= total) return int4{-1, 0, 0, 0};
    const int excl = incl - n;
    int e = -1, row0 = 0, rows = 0, before = excl;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (e0 + i < e1) {
            const int nt = max(o[i + 1] - o[i] + kRowsPerTile - 1, 0) / kRowsPerTile;
            if (t >= before && t < before + nt) {
                e = e0 + i;
                row0 = o[i] + (t - before) * kRowsPerTile;
                rows = min(kRowsPerTile, o[i + 1] - row0);
            }
            before += nt;
        }
    }
    // exactly one lane's run holds t (runs without tiles are empty ranges)
    const int src = __builtin_ctzll(__ballot(e >= 0));
    return int4{__builtin_amdgcn_readfirstlane(__shfl(e, src, 64)), __builtin_amdgcn_readfirstlane(__shfl(row0, src, 64)),
                __builtin_amdgcn_readfirstlane(__shfl(rows, src, 64)), 0};
}

}  // namespace moe
