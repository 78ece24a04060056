// Router logits (bf16 x . W_r^T, fp32 accumulation) and top-k selection.
//
// The router is BF16 ("Why Are the V2.6 Files Half the Size of V2.5?", row
// "Router") and picks 8 experts per token ("How Big Is Each Expert?"), both
// on the teardown page.
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------------------
// Router logits on the bf16 MFMA (16x16x32).  A operand = 16 router rows
// (experts), B operand = 16 token rows; D[4g+i][r] lands in lane (g, r) as
// expert e0+4g+i, token t0+r, so each lane stores 4 consecutive logits.
// Both operands share one lane->k mapping (8 consecutive k per lane), which is
// all a dot product needs.
//
// Work split: a workgroup of 4 waves covers 16*TT tokens and 16*(4/KS)
// experts; KS waves split the K range of one 16-expert tile and are reduced
// through LDS (decode shapes: few tokens, so split K for parallelism).
// ---------------------------------------------------------------------------
template <int TT, int KS>
__global__ void __launch_bounds__(256) router_logits_kernel(const uint16_t* __restrict__ x,
                                                             const uint16_t* __restrict__ wr,
                                                             float* __restrict__ logits,
                                                             int T, int H, int E) {
    constexpr int kGroups = 4 / KS;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int ks = wave % KS;
    const int eg = wave / KS;
    const int g = lane >> 4, r = lane & 15;
    const int e0 = (blockIdx.x * kGroups + eg) * 16;
    const int t0 = blockIdx.y * (16 * TT);

    const int erow = min(e0 + r, E - 1);
    const uint16_t* wp = wr + (size_t)erow * H;
    const uint16_t* xp[TT];
#pragma unroll
    for (int j = 0; j < TT; ++j) xp[j] = x + (size_t)min(t0 + 16 * j + r, T - 1) * H;

    v4f acc[TT];
#pragma unroll
    for (int j = 0; j < TT; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int kspan = H / KS;
    const int kbeg = ks * kspan, kend = kbeg + kspan;
    // kspan is a multiple of 32; unroll by 4 steps of 32 where possible
    int kk = kbeg;
    for (; kk + 128 <= kend; kk += 128) {
        v8bf a[4], b[4][TT];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            a[u] = *(const v8bf*)(wp + kk + 32 * u + 8 * g);
#pragma unroll
            for (int j = 0; j < TT; ++j) b[u][j] = *(const v8bf*)(xp[j] + kk + 32 * u + 8 * g);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < TT; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b[u][j], acc[j], 0, 0, 0);
    }
    for (; kk < kend; kk += 32) {
        v8bf a = *(const v8bf*)(wp + kk + 8 * g);
#pragma unroll
        for (int j = 0; j < TT; ++j) {
            v8bf b = *(const v8bf*)(xp[j] + kk + 8 * g);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
        }
    }

    if constexpr (KS > 1) {
        __shared__ v4f red[4][TT][64];
#pragma unroll
        for (int j = 0; j < TT; ++j) red[wave][j][lane] = acc[j];
        __syncthreads();
        if (ks != 0) return;
#pragma unroll
        for (int j = 0; j < TT; ++j) {
            v4f s = red[wave][j][lane];
#pragma unroll
            for (int q = 1; q < KS; ++q) s += red[wave + q][j][lane];
            acc[j] = s;
        }
    }

    const int e = e0 + 4 * g;
#pragma unroll
    for (int j = 0; j < TT; ++j) {
        const int t = t0 + 16 * j + r;
        if (t >= T) continue;
        float* o = logits + (size_t)t * E + e;
        if (e + 3 < E && (E & 3) == 0) {
            *(v4f*)o = acc[j];
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (e + i < E) o[i] = acc[j][i];
        }
    }
}

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* w_router, float* logits,
                                int64_t T, int H, int E, hipStream_t stream) {
    if (T <= 256) {
        // decode shapes: 16 tokens x 16 experts per workgroup, K split over 4 waves
        dim3 grid((E + 15) / 16, (unsigned)((T + 15) / 16));
        hipLaunchKernelGGL((router_logits_kernel<1, 4>), grid, dim3(256), 0, stream, x, w_router, logits,
                           (int)T, H, E);
    } else {
        // prefill shapes: 64 tokens x 64 experts per workgroup
        dim3 grid((E + 63) / 64, (unsigned)((T + 63) / 64));
        hipLaunchKernelGGL((router_logits_kernel<4, 1>), grid, dim3(256), 0, stream, x, w_router, logits,
                           (int)T, H, E);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k selection + softmax weights: one wave per token.
//
// key = fp32(L + b).  Each key is mapped to an unsigned integer that orders
// like the float (after -0 -> +0) and packed with ~id in the low word, so a
// single 64-bit max picks the largest key and, among equal keys, the lowest
// expert id.  k rounds of a wave-wide max; the winning lane retires its key.
// Weights: softmax over the k selected *unbiased* logits, max-subtracted.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ordered_key(float f) {
    if (f == 0.0f) f = 0.0f;   // -0 == +0
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        unsigned long long o = __shfl_xor(v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

template <int EJ>
__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias,
                                                    int32_t* __restrict__ ids, float* __restrict__ w,
                                                    int T, int E, int k) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float* L = logits + (size_t)t * E;

    float lv[EJ];
    unsigned long long key[EJ];
#pragma unroll
    for (int j = 0; j < EJ; ++j) {
        const int e = lane + 64 * j;
        if (e < E) {
            float l = L[e];
            float kf = bias ? l + bias[e] : l;
            lv[j] = l;
            key[j] = ((unsigned long long)ordered_key(kf) << 32) | (uint32_t)(~(uint32_t)e);
        } else {
            lv[j] = 0.0f;
            key[j] = 0;
        }
    }

    float sel = 0.0f;   // lane j (< k) keeps the j-th selected logit
    int sid = 0;
    for (int j = 0; j < k; ++j) {
        unsigned long long best = 0;
#pragma unroll
        for (int q = 0; q < EJ; ++q) best = key[q] > best ? key[q] : best;
        best = wave_max_u64(best);
        const int e = (int)(~(uint32_t)best);
        const int owner = e & 63, slot = e >> 6;
        float lsel = 0.0f;
        if (lane == owner) {
#pragma unroll
            for (int q = 0; q < EJ; ++q)
                if (q == slot) { key[q] = 0; lsel = lv[q]; }
        }
        lsel = __shfl(lsel, owner, 64);
        if (lane == j) { sel = lsel; sid = e; }
    }

    // softmax over the k selected logits held by lanes 0..k-1
    float m = lane < k ? sel : -__builtin_inff();
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    float z = lane < k ? expf(sel - m) : 0.0f;
    float s = z;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    if (lane < k) {
        ids[(size_t)t * k + lane] = sid;
        w[(size_t)t * k + lane] = z / s;
    }
}

hipError_t launch_topk(const float* logits, const float* bias, int32_t* ids, float* w, int64_t T, int E,
                       int k, hipStream_t stream) {
    dim3 grid((unsigned)((T + 3) / 4)), block(256);
    const int ej = (E + 63) / 64;
#define MOE_TOPK_CASE(n) \
    case n: hipLaunchKernelGGL((topk_kernel<n>), grid, block, 0, stream, logits, bias, ids, w, (int)T, E, k); break;
    switch (ej) {
        MOE_TOPK_CASE(1) MOE_TOPK_CASE(2) MOE_TOPK_CASE(3) MOE_TOPK_CASE(4)
        MOE_TOPK_CASE(5) MOE_TOPK_CASE(6) MOE_TOPK_CASE(7) MOE_TOPK_CASE(8)
        default: return hipErrorInvalidValue;
    }
#undef MOE_TOPK_CASE
    return hipGetLastError();
}

}  // namespace moe
