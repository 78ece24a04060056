// Microbenchmarks that measure the two ceilings the layer's kernels are held
// against on the running MI355X (include/moe_micro.h):
//   * HBM: a plain stream of 16-byte reads (or writes) over a buffer much
//     larger than the caches, in the two access patterns the kernels use
//     (grid-stride, and one contiguous chunk per workgroup);
//   * matrix cores: back-to-back block-scaled MFMAs on register operands
//     (FP4 x FP8 as the expert GEMMs issue them, and the other operand
//     formats for comparison), with the shader clock counted over the run.
// They compute nothing of the layer.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_micro.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// ---- HBM ------------------------------------------------------------------

// Four 16-byte loads in flight per lane per iteration; NT = false: ordinary
// cached loads (as the GEMMs' weight loads), true: non-temporal loads (as the
// combine's).  The XOR of everything read is stored per thread so that no
// load is dead.
template <bool NT>
__device__ __forceinline__ v4u ld16(const v4u* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <bool NT>
__global__ void __launch_bounds__(256) read_grid_stride_kernel(const v4u* __restrict__ buf, size_t n16,
                                                               uint32_t* __restrict__ out) {
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t x = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const v4u a = ld16<NT>(buf + i), b = ld16<NT>(buf + i + stride);
        const v4u c = ld16<NT>(buf + i + 2 * stride), d = ld16<NT>(buf + i + 3 * stride);
        x ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const v4u a = ld16<NT>(buf + i);
        x ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = x;
}

template <bool NT>
__global__ void __launch_bounds__(256) read_chunk_kernel(const v4u* __restrict__ buf, size_t n16,
                                                         uint32_t* __restrict__ out) {
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t lo = (size_t)blockIdx.x * per, hi = lo + per < n16 ? lo + per : n16;
    uint32_t x = 0;
    size_t i = lo + threadIdx.x;
    for (; i + 3 * 256 < hi; i += 4 * 256) {
        const v4u a = ld16<NT>(buf + i), b = ld16<NT>(buf + i + 256);
        const v4u c = ld16<NT>(buf + i + 512), d = ld16<NT>(buf + i + 768);
        x ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < hi; i += 256) {
        const v4u a = ld16<NT>(buf + i);
        x ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = x;
}

// The read pattern of the streaming expert GEMMs over packed weights: each
// workgroup owns a region of 16 groups (one 16-row group of weight rows
// each) of gbytes, gstride bytes apart (gstride >= gbytes; the region is
// 16 gstride); wave w reads groups 4w .. 4w+3, each in 1 KB blocks (lane l at
// 16 l), two blocks per group per stage and two stages in flight: 16 loads of
// 16 bytes per lane outstanding, as in the GEMMs.  skew 1: wave w walks its
// stages starting at w nstage / 4 (wrapping), skew 2: at (blockIdx mod 8)
// nstage / 8, skew 0: all from stage 0.
template <bool NT>
__global__ void __launch_bounds__(256) read_groups_kernel(const uint8_t* __restrict__ buf, size_t gbytes,
                                                          size_t gstride, int skew, uint32_t* __restrict__ out) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint8_t* base = buf + (size_t)blockIdx.x * 16 * gstride + (size_t)(4 * wave) * gstride + 16 * lane;
    const int nstage = (int)(gbytes / 2048);
    const int st0 = skew == 1 ? wave * nstage / 4 : skew == 2 ? (int)(blockIdx.x & 7) * nstage / 8 : 0;
    uint32_t x = 0;
    v4u a[2][8];
    auto issue = [&](int b, int st) __attribute__((always_inline)) {
        int sp = st + st0;
        sp = sp >= nstage ? sp - nstage : sp;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            a[b][q] = ld16<NT>((const v4u*)(base + (size_t)(q >> 1) * gstride + (size_t)sp * 2048 + 1024 * (q & 1)));
    };
    auto use = [&](int b) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 8; ++q) x ^= a[b][q].x ^ a[b][q].y ^ a[b][q].z ^ a[b][q].w;
    };
    issue(0, 0);
    issue(1, nstage > 1 ? 1 : 0);
    for (int st = 0; st < nstage; st += 2) {
        use(0);
        issue(0, st + 2 < nstage ? st + 2 : nstage - 1);
        use(1);
        issue(1, st + 3 < nstage ? st + 3 : nstage - 1);
    }
    use(0);
    use(1);
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = x;
}

__global__ void __launch_bounds__(256) write_grid_stride_kernel(v4u* __restrict__ buf, size_t n16, uint32_t v) {
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
        buf[i] = v4u{v, v ^ 1u, v ^ 2u, (uint32_t)i};
}

// ---- matrix cores -----------------------------------------------------------

// ACC independent accumulators per wave, `iters` rounds of ACC MFMAs each.
// FA / FB: operand formats of the block-scaled MFMA (0 e4m3, 1 e5m2, 2 e2m3,
// 3 e3m2, 4 e2m1), unit scales.  The block's shader-clock and constant-clock
// (100 MHz) spans are written by thread 0 of workgroup 0.
constexpr int kAcc = 8;

template <int FA, int FB>
__global__ void __launch_bounds__(256) mfma32_kernel(int iters, float* __restrict__ out,
                                                     unsigned long long* __restrict__ clk) {
    const int lane = threadIdx.x & 63;
    v8i a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = 0x22222222 + lane * 0x01010101 + i;   // small nonzero codes in every format
        b[i] = 0x31313131 + lane + i * 0x00010001;
    }
    v16f acc[kAcc];
#pragma unroll
    for (int j = 0; j < kAcc; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
    const unsigned long long c0 = clock64(), t0 = wall_clock64();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kAcc; ++j)
            acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], FA, FB, 0, 127, 0, 127);
    }
    const unsigned long long c1 = clock64(), t1 = wall_clock64();
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kAcc; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        clk[0] = c1 - c0;
        clk[1] = t1 - t0;
    }
}

template <int FA, int FB>
__global__ void __launch_bounds__(256) mfma16_kernel(int iters, float* __restrict__ out,
                                                     unsigned long long* __restrict__ clk) {
    const int lane = threadIdx.x & 63;
    v8i a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = 0x22222222 + lane * 0x01010101 + i;
        b[i] = 0x31313131 + lane + i * 0x00010001;
    }
    v4f acc[2 * kAcc];
#pragma unroll
    for (int j = 0; j < 2 * kAcc; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
    const unsigned long long c0 = clock64(), t0 = wall_clock64();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 2 * kAcc; ++j)
            acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[j], FA, FB, 0, 127, 0, 127);
    }
    const unsigned long long c1 = clock64(), t1 = wall_clock64();
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 2 * kAcc; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        clk[0] = c1 - c0;
        clk[1] = t1 - t0;
    }
}

template <int FA, int FB>
hipError_t launch_mfma(int shape, int iters, int grid, float* out, unsigned long long* clk, hipStream_t s) {
    if (shape == 32)
        hipLaunchKernelGGL((mfma32_kernel<FA, FB>), dim3(grid), dim3(256), 0, s, iters, out, clk);
    else
        hipLaunchKernelGGL((mfma16_kernel<FA, FB>), dim3(grid), dim3(256), 0, s, iters, out, clk);
    return hipGetLastError();
}

}  // namespace

extern "C" {

int moe_micro_hbm_read(const void* buf, size_t bytes, uint32_t* out, int grid, int pattern, hipStream_t stream) {
    if (!buf || !out || grid <= 0 || bytes < 16 || (bytes & 15) || pattern < 0 || pattern > 3) return 1;
    const v4u* b = (const v4u*)buf;
    switch (pattern) {
        case 0: hipLaunchKernelGGL(read_grid_stride_kernel<false>, dim3(grid), dim3(256), 0, stream, b, bytes / 16, out); break;
        case 1: hipLaunchKernelGGL(read_chunk_kernel<false>, dim3(grid), dim3(256), 0, stream, b, bytes / 16, out); break;
        case 2: hipLaunchKernelGGL(read_grid_stride_kernel<true>, dim3(grid), dim3(256), 0, stream, b, bytes / 16, out); break;
        default: hipLaunchKernelGGL(read_chunk_kernel<true>, dim3(grid), dim3(256), 0, stream, b, bytes / 16, out); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

int moe_micro_hbm_read_groups(const void* buf, size_t bytes, size_t group_bytes, size_t group_stride, int skew,
                              uint32_t* out, int nontemporal, hipStream_t stream) {
    // a multiple of 4 KiB: an even number of 2 KiB stages (the read loop takes two at a time)
    if (!buf || !out || group_bytes < 4096 || (group_bytes & 4095) || group_stride < group_bytes ||
        (group_stride & 15) || skew < 0 || skew > 2)
        return 1;
    const size_t region = 16 * group_stride;
    if (bytes < region) return 1;
    const size_t grid = bytes / region;
    if (grid > (size_t)1 << 20) return 1;
    if (nontemporal)
        hipLaunchKernelGGL(read_groups_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream, (const uint8_t*)buf,
                           group_bytes, group_stride, skew, out);
    else
        hipLaunchKernelGGL(read_groups_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream, (const uint8_t*)buf,
                           group_bytes, group_stride, skew, out);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

int moe_micro_hbm_write(void* buf, size_t bytes, int grid, hipStream_t stream) {
    if (!buf || grid <= 0 || bytes < 16 || (bytes & 15)) return 1;
    hipLaunchKernelGGL(write_grid_stride_kernel, dim3(grid), dim3(256), 0, stream, (v4u*)buf, bytes / 16, 7u);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

int moe_micro_mfma(int fmt_a, int fmt_b, int shape, int iters, int grid, float* out, unsigned long long* clocks,
                   hipStream_t stream) {
    if (!out || !clocks || grid <= 0 || iters <= 0 || (shape != 16 && shape != 32)) return 1;
    hipError_t e;
    if (fmt_a == 4 && fmt_b == 0) e = launch_mfma<4, 0>(shape, iters, grid, out, clocks, stream);
    else if (fmt_a == 0 && fmt_b == 0) e = launch_mfma<0, 0>(shape, iters, grid, out, clocks, stream);
    else if (fmt_a == 4 && fmt_b == 4) e = launch_mfma<4, 4>(shape, iters, grid, out, clocks, stream);
    else return 2;
    return e == hipSuccess ? 0 : 4;
}

}  // extern "C"
