// Router logits (bf16 x . W_r^T, fp32 accumulation) and top-k selection.
//
// The router is BF16 ("Why Are the V2.6 Files Half the Size of V2.5?", row
// "Router") and picks 8 experts per token ("How Big Is Each Expert?"), both
// on the teardown page.
#include "moe_internal.h"
#include "fp8_rows.h"

#include <type_traits>

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
__device__ __forceinline__ void router_logits_block(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                                                    float* __restrict__ logits, int T, int H, int E, int bx,
                                                    int by) {
    constexpr int kGroups = 4 / KS;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int ks = wave % KS;
    const int eg = wave / KS;
    const int g = lane >> 4, r = lane & 15;
    const int e0 = (bx * kGroups + eg) * 16;
    const int t0 = by * (16 * TT);

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
    // kspan is a multiple of 32.  Chunks of 16 steps of 32: the 32 loads of a
    // chunk go out together, so a decode-sized K range costs two or three
    // memory round trips rather than one per step (same MFMA order, so the
    // same sums).
    int kk = kbeg;
    constexpr int U = 16;
    for (; kk + 32 * U <= kend; kk += 32 * U) {
        v8bf a[U], b[U][TT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            a[u] = *(const v8bf*)(wp + kk + 32 * u + 8 * g);
#pragma unroll
            for (int j = 0; j < TT; ++j) b[u][j] = *(const v8bf*)(xp[j] + kk + 32 * u + 8 * g);
        }
        __builtin_amdgcn_sched_barrier(0);   // every load of the chunk before its first MFMA
#pragma unroll
        for (int u = 0; u < U; ++u)
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

template <int TT, int KS>
__global__ void __launch_bounds__(256) router_logits_kernel(const uint16_t* __restrict__ x,
                                                             const uint16_t* __restrict__ wr,
                                                             float* __restrict__ logits,
                                                             int T, int H, int E) {
    router_logits_block<TT, KS>(x, wr, logits, T, H, E, blockIdx.x, blockIdx.y);
}

// Decode forward: the router logits and the token-order FP8 copy of x in one
// launch.  Block rows y < gy compute logits as router_logits_kernel does; the
// rows after them quantise token rows, one per workgroup.  The two parts
// share nothing, so no workgroup waits for another.
template <bool F32S>
__global__ void __launch_bounds__(256) router_quant_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ wr,
                                                           float* __restrict__ logits, int T, int H, int E,
                                                           int gy, uint8_t* __restrict__ xq,
                                                           void* __restrict__ xs) {
    if ((int)blockIdx.y < gy) {
        router_logits_block<1, 4>(x, wr, logits, T, H, E, blockIdx.x, blockIdx.y);
        return;
    }
    const int r = ((int)blockIdx.y - gy) * (int)gridDim.x + (int)blockIdx.x;
    if (r < T) quantise_row<F32S>(x + (size_t)r * H, xq, xs, r, H);
}

// ---------------------------------------------------------------------------
// Router logits for many tokens (prefill): an LDS-tiled bf16 GEMM on
// v_mfma_f32_32x32x16_bf16.  A workgroup of 4 waves computes 64 tokens x 128
// experts (small enough for two workgroups per CU and, on the prefill
// shapes, at least one workgroup per CU); wave (wm, wn) owns 32 tokens x 64
// experts (1 x 2 MFMA tiles).  K is walked in stages of 64 (128 bytes of a
// bf16 row); each stage's 64 x rows and 128 W_r rows (24 KB) are copied by
// direct global->LDS loads into a three-buffer ring, two stages ahead of
// their use, with the 16-byte chunk c of row p stored at slot
// c ^ ((p / 2) mod 8): LDS serves a 16-byte read 16 lanes at a time across
// 64 banks (256 bytes), and two 128-byte rows share one such window, so the
// row's parity picks the half and (p / 2) mod 8 spreads the 8 rows of each
// parity over the 8 slots; the 16 rows of a phase then hit distinct banks.  Both operands use the same lane -> k mapping
// (8 consecutive k per lane), which is all a dot product needs.  Rows past T
// or E are clamped for loading and not stored.  H % 64 == 0.
// ---------------------------------------------------------------------------
typedef float v16f_r __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_r;

constexpr int kRtTok = 64;           // tokens per workgroup
constexpr int kRtExp = 128;          // experts per workgroup
constexpr int kRtStageK = 64;        // bf16 elements of K per stage
constexpr int kRtRowBytes = 2 * kRtStageK;
constexpr int kRtBuf = (kRtTok + kRtExp) * kRtRowBytes;   // x rows, then W_r rows
constexpr int kRtLoads = (kRtTok + kRtExp) / 32;          // direct loads per wave per stage (8 rows each)

__shared__ __attribute__((aligned(16))) uint8_t rt_buf0[kRtBuf];
__shared__ __attribute__((aligned(16))) uint8_t rt_buf1[kRtBuf];
__shared__ __attribute__((aligned(16))) uint8_t rt_buf2[kRtBuf];

__device__ __forceinline__ int rt_swz(int row, int chunk) { return row * kRtRowBytes + ((chunk ^ ((row >> 1) & 7)) << 4); }
__device__ __forceinline__ constexpr int rt_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// The K loop; the three LDS buffers are separate objects, which the
// compiler's wait tracking for direct-to-LDS loads tells apart.
__device__ __forceinline__ void router_tiled_kloop(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                                                   int T, int H, int E, int t0, int e0, v16f_r (&acc)[2],
                                                   uint8_t* __restrict__ b0, uint8_t* __restrict__ b1,
                                                   uint8_t* __restrict__ b2) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 5, r = lane & 31;
    const int wm = wave & 1, wn = wave >> 1;
    const int nstage = H / kRtStageK;
    auto buf = [&](auto bc) -> uint8_t* {
        constexpr int B = decltype(bc)::value;
        if constexpr (B == 0) return b0; else if constexpr (B == 1) return b1; else return b2;
    };
    // stage st: 192 rows (64 x rows, then 128 W_r rows) x 128 bytes; each
    // load moves 8 rows (8 lanes of 16 bytes per row); wave w moves rows
    // 48w .. 48w+47
    auto load_stage = [&](auto bc, int st) {
        uint8_t* lds = buf(bc);
#pragma unroll
        for (int p = 0; p < kRtLoads; ++p) {
            const int row = 8 * kRtLoads * wave + 8 * p + (lane >> 3);    // 0..191
            const int chunk = (lane & 7) ^ ((row >> 1) & 7);
            const uint16_t* src = (row < kRtTok) ? x + (size_t)min(t0 + row, T - 1) * H
                                                 : wr + (size_t)min(e0 + row - kRtTok, E - 1) * H;
            __builtin_amdgcn_global_load_lds(src + st * kRtStageK + 8 * chunk,
                                             (lds_void_r*)(lds + (8 * kRtLoads * wave + 8 * p) * kRtRowBytes), 16, 0, 0);
        }
    };
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[j][q] = 0.0f;

    auto stage = [&](auto setc, int st) {
        constexpr int SET = decltype(setc)::value;
        // stage st landed in every wave; the buffer of stage st-1 is free
        __builtin_amdgcn_s_waitcnt(rt_vmcnt(kRtLoads));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        load_stage(std::integral_constant<int, (SET + 2) % 3>{}, min(st + 2, nstage - 1));
        const uint8_t* lds = buf(setc);
#pragma unroll
        for (int s = 0; s < kRtStageK / 16; ++s) {
            const v8bf xa = *(const v8bf*)(lds + rt_swz(32 * wm + r, 2 * s + g));
            v8bf wa[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) wa[j] = *(const v8bf*)(lds + rt_swz(kRtTok + 64 * wn + 32 * j + r, 2 * s + g));
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[j], xa, acc[j], 0, 0, 0);
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    load_stage(I0{}, 0);
    load_stage(I1{}, min(1, nstage - 1));
    int st = 0;
    for (; st + 3 <= nstage; st += 3) {
        stage(I0{}, st);
        stage(I1{}, st + 1);
        stage(I2{}, st + 2);
    }
    if (st < nstage) stage(I0{}, st);
    if (st + 1 < nstage) stage(I1{}, st + 1);
    __builtin_amdgcn_s_waitcnt(rt_vmcnt(0));
}

// Workgroup id -> tile: workgroups on XCD x (id mod 8) take the token blocks
// x, x + 8, x + 16, ... (tpx of them) for expert block 0, then the same token
// blocks for expert block 1, and so on.  The workgroups an XCD runs at one time
// then share one or two expert blocks of W_r in its L2 (with every expert block
// in flight at once, 384 x 6144 bf16 = 4.5 MiB does not fit one XCD's 4 MB)
// and read the same token blocks of x.  Ids past the tiles exit at once.
__global__ void __launch_bounds__(256) router_logits_tiled_kernel(const uint16_t* __restrict__ x,
                                                                   const uint16_t* __restrict__ wr,
                                                                   float* __restrict__ logits, int T, int H, int E,
                                                                   int tpx) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 5, r = lane & 31;
    const int wm = wave & 1, wn = wave >> 1;
    const int local = (int)(blockIdx.x >> 3);
    const int eb = local / tpx, tb = (local - eb * tpx) * 8 + (int)(blockIdx.x & 7);
    const int e0 = eb * kRtExp, t0 = tb * kRtTok;
    if (e0 >= E || t0 >= T) return;
    v16f_r acc[2];
    router_tiled_kloop(x, wr, T, H, E, t0, e0, acc, rt_buf0, rt_buf1, rt_buf2);
    // acc[j]: token t0 + 32wm + r, experts e0 + 64wn + 32j + 8q + 4g + (0..3)
    const int t = t0 + 32 * wm + r;
    if (t >= T) return;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = e0 + 64 * wn + 32 * j + 8 * q + 4 * g;
            float* o = logits + (size_t)t * E + e;
            const v4f v = {acc[j][4 * q], acc[j][4 * q + 1], acc[j][4 * q + 2], acc[j][4 * q + 3]};
            if (e + 3 < E && (E & 3) == 0) {
                *(v4f*)o = v;
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (e + u < E) o[u] = v[u];
            }
        }
    }
}

hipError_t launch_router_quant(const uint16_t* x, const uint16_t* w_router, float* logits, int64_t T, int H, int E,
                               uint8_t* xq, void* xs, int f32_scales, hipStream_t stream) {
    if (T > kDecodeRouterMaxT) return hipErrorInvalidValue;
    const int gx = (E + 15) / 16, gy = (int)((T + 15) / 16);
    const int gq = (int)((T + gx - 1) / gx);   // token rows to quantise, gx per block row
    dim3 grid(gx, gy + gq);
    if (f32_scales)
        hipLaunchKernelGGL(router_quant_kernel<true>, grid, dim3(256), 0, stream, x, w_router, logits, (int)T, H, E,
                           gy, xq, xs);
    else
        hipLaunchKernelGGL(router_quant_kernel<false>, grid, dim3(256), 0, stream, x, w_router, logits, (int)T, H, E,
                           gy, xq, xs);
    return hipGetLastError();
}

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* w_router, float* logits,
                                int64_t T, int H, int E, hipStream_t stream) {
    if (T <= kDecodeRouterMaxT) {
        // decode shapes: 16 tokens x 16 experts per workgroup, K split over 4 waves
        dim3 grid((E + 15) / 16, (unsigned)((T + 15) / 16));
        hipLaunchKernelGGL((router_logits_kernel<1, 4>), grid, dim3(256), 0, stream, x, w_router, logits,
                           (int)T, H, E);
    } else {
        // prefill shapes: LDS-tiled, 64 tokens x 128 experts per workgroup, an
        // XCD's workgroups grouped by expert block (router_logits_tiled_kernel)
        const int nbe = (E + kRtExp - 1) / kRtExp;
        const int tpx = (int)(((T + kRtTok - 1) / kRtTok + 7) / 8);   // token blocks per XCD
        hipLaunchKernelGGL(router_logits_tiled_kernel, dim3((unsigned)(nbe * tpx * 8)), dim3(256), 0, stream, x,
                           w_router, logits, (int)T, H, E, tpx);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Selection-bias load balancing, one step (the rule of
// moe_update_selection_bias): an expert below the mean load N / E gets
// +step, one above it -step; E * n_e against N in 64-bit integers, so the
// sign is exact; the new bias is one fp32 addition.  One thread per expert.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) bias_update_kernel(const int32_t* __restrict__ offsets, int E, float step,
                                                          float* __restrict__ bias) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= E) return;
    const int64_t n = (int64_t)offsets[e + 1] - offsets[e];
    const int64_t N = (int64_t)offsets[E] - offsets[0];
    const int64_t d = N - (int64_t)E * n;
    const float delta = d > 0 ? step : (d < 0 ? -step : 0.0f);
    bias[e] = bias[e] + delta;
}

hipError_t launch_bias_update(const int32_t* offsets, int E, float step, float* bias, hipStream_t stream) {
    hipLaunchKernelGGL(bias_update_kernel, dim3((E + 255) / 256), dim3(256), 0, stream, offsets, E, step, bias);
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

// Largest value over the wave, returned wave-uniform: DPP shifts by 1, 2, 4
// and 8 lanes leave each 16-lane row's maximum in its lane 15, two row
// broadcasts (row 0 into row 1 and row 2 into row 3, then lane 31 into rows 2
// and 3) carry the maxima to lane 63, and a readlane returns it.  DPP moves
// stay in the VALU; a shuffle goes through LDS and costs far more latency.
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t v, uint32_t t) { return t > v ? t : v; }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = dpp_max_step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x111, 0xf, 0xf, false));   // row_shr:1
    v = dpp_max_step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x112, 0xf, 0xf, false));   // row_shr:2
    v = dpp_max_step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x114, 0xf, 0xf, false));   // row_shr:4
    v = dpp_max_step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x118, 0xf, 0xf, false));   // row_shr:8
    v = dpp_max_step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xa, 0xf, false));   // row_bcast:15
    v = dpp_max_step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xc, 0xf, false));   // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// The same pattern for a float maximum and a float sum (lanes without a DPP
// source add 0).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float old, float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_max_f32(float v) {
    v = fmaxf(v, dpp_f<0x111, 0xf>(v, v));
    v = fmaxf(v, dpp_f<0x112, 0xf>(v, v));
    v = fmaxf(v, dpp_f<0x114, 0xf>(v, v));
    v = fmaxf(v, dpp_f<0x118, 0xf>(v, v));
    v = fmaxf(v, dpp_f<0x142, 0xa>(v, v));
    v = fmaxf(v, dpp_f<0x143, 0xc>(v, v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_sum_f32(float v) {
    v += dpp_f<0x111, 0xf>(0.0f, v);
    v += dpp_f<0x112, 0xf>(0.0f, v);
    v += dpp_f<0x114, 0xf>(0.0f, v);
    v += dpp_f<0x118, 0xf>(0.0f, v);
    v += dpp_f<0x142, 0xa>(0.0f, v);
    v += dpp_f<0x143, 0xc>(0.0f, v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// SIG: sigmoid scoring (teardown "How Big Is Each Expert?": sigmoid expert
// scores and a per-expert load-balancing bias):
// key = fp32(sigmoid(L) + b), weights = sigmoid of the selected logits over
// their sum.  Otherwise softmax scoring as above.
template <int EJ, bool SIG>
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
            // the score replaces the logit: sigmoid evaluated in float64 and
            // rounded once to float32, so that two implementations of it agree
            // on the float32 score (and with it on the selection) unless the
            // float64 value lies within an ulp or two of a float32 midpoint
            if constexpr (SIG) l = (float)(1.0 / (1.0 + exp(-(double)l)));
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
        // the largest ordered key, then among the lanes holding it the
        // largest ~id (the lowest expert id)
        const uint32_t hi = wave_max_u32((uint32_t)(best >> 32));
        const uint32_t lo = wave_max_u32((uint32_t)(best >> 32) == hi ? (uint32_t)best : 0u);
        const int e = (int)(~lo);
        const int owner = e & 63, slot = e >> 6;
        float lsel = 0.0f;
        if (lane == owner) {
#pragma unroll
            for (int q = 0; q < EJ; ++q)
                if (q == slot) { key[q] = 0; lsel = lv[q]; }
        }
        lsel = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lsel), owner));
        if (lane == j) { sel = lsel; sid = e; }
    }

    // softmax over the k selected logits held by lanes 0..k-1, or the
    // selected sigmoid scores over their sum
    float z;
    if constexpr (SIG) {
        z = lane < k ? sel : 0.0f;
    } else {
        const float m = wave_max_f32(lane < k ? sel : -__builtin_inff());
        z = lane < k ? expf(sel - m) : 0.0f;
    }
    const float s = wave_sum_f32(z);
    if (lane < k) {
        ids[(size_t)t * k + lane] = sid;
        w[(size_t)t * k + lane] = z / s;
    }
}

template <bool SIG>
static hipError_t launch_topk_score(const float* logits, const float* bias, int32_t* ids, float* w, int64_t T,
                                    int E, int k, hipStream_t stream) {
    dim3 grid((unsigned)((T + 3) / 4)), block(256);
    const int ej = (E + 63) / 64;
#define MOE_TOPK_CASE(n) \
    case n: hipLaunchKernelGGL((topk_kernel<n, SIG>), grid, block, 0, stream, logits, bias, ids, w, (int)T, E, k); break;
    switch (ej) {
        MOE_TOPK_CASE(1) MOE_TOPK_CASE(2) MOE_TOPK_CASE(3) MOE_TOPK_CASE(4)
        MOE_TOPK_CASE(5) MOE_TOPK_CASE(6) MOE_TOPK_CASE(7) MOE_TOPK_CASE(8)
        default: return hipErrorInvalidValue;
    }
#undef MOE_TOPK_CASE
    return hipGetLastError();
}

hipError_t launch_topk(const float* logits, const float* bias, int32_t* ids, float* w, int64_t T, int E,
                       int k, int sigmoid, hipStream_t stream) {
    return sigmoid ? launch_topk_score<true>(logits, bias, ids, w, T, E, k, stream)
                   : launch_topk_score<false>(logits, bias, ids, w, T, E, k, stream);
}

}  // namespace moe
