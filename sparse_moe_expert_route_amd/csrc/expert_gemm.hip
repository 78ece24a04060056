// Grouped expert GEMMs on the gfx950 block-scaled MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4), A = MXFP4 weights, B = FP8 activations.
//
// Experts are gate/up/down projections around a 2,048-wide middle (teardown,
// "How Big Is Each Expert?"), stored as MXFP4 ("Why Are the V2.6 Files Half
// the Size of V2.5?") and computed in FP8 e4m3 (vLLM recipe, "Overview").
// MXFP4 runs natively on CDNA 4 (vLLM recipe, "AMD (MI355X, TP4)"), so the
// e2m1 codes and their e8m0 scales go to the MFMA as stored.
//
// Operand layout of the 16x16x128 instruction (lane l, g = l/16, r = l%16):
//   FP4 operand: 16 bytes = 32 consecutive k, k = 32g + i, element 2i in the
//                low nibble (the MXFP4 storage order);
//   FP8 operand: bytes 0..15 -> k = 16g + i, bytes 16..31 -> k = 64 + 16g + i;
//   scale VGPR : byte op_sel of lane l scales row r, k in [32g, 32g+32);
//   result     : lane l holds D[4g + i][r], i = 0..3.
//
// Streaming structure (weight-bandwidth-bound shapes): a workgroup owns one
// m-tile of 16 rows of one expert and a block of weight rows; every weight
// byte is read exactly once per m-tile, directly into registers, never
// through LDS.  To make each lane's weight reads contiguous, K is walked in
// super-steps of S*128: within a super-step, MFMA s pairs logical k-block b
// (32 wide) with physical block S*b + s.  A lane then reads 16*S contiguous
// weight bytes and S consecutive scale bytes (one dword for S = 4, selected
// by op_sel = s), and the activation pieces are gathered to match.
#include "moe_internal.h"

namespace moe {

template <int S>
struct Stage {
    uint4 w[4][S];      // weight codes, 4 row-tiles
    uint32_t ws[4];     // weight scales (S bytes used)
    uint4 xa[S], xb[S]; // activation halves
    uint32_t xs;        // activation scale byte
};

template <int S>
__device__ __forceinline__ uint32_t load_scale_bytes(const uint8_t* p) {
    if constexpr (S == 4) return *(const uint32_t*)p;
    else if constexpr (S == 2) return *(const uint16_t*)p;
    else return *p;
}

template <int S, int s>
__device__ __forceinline__ void mfma_step(const Stage<S>& st, v4f (&acc)[4]) {
    v8i b;
    b[0] = st.xa[s].x; b[1] = st.xa[s].y; b[2] = st.xa[s].z; b[3] = st.xa[s].w;
    b[4] = st.xb[s].x; b[5] = st.xb[s].y; b[6] = st.xb[s].z; b[7] = st.xb[s].w;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v8i a;
        a[0] = st.w[j][s].x; a[1] = st.w[j][s].y; a[2] = st.w[j][s].z; a[3] = st.w[j][s].w;
        a[4] = 0; a[5] = 0; a[6] = 0; a[7] = 0;
        acc[j] = mfma_w4a8<s>(a, b, acc[j], (int)st.ws[j], (int)st.xs);
    }
}

template <int S>
__device__ __forceinline__ void compute_stage(const Stage<S>& st, v4f (&acc)[4]) {
    mfma_step<S, 0>(st, acc);
    if constexpr (S > 1) mfma_step<S, 1>(st, acc);
    if constexpr (S > 2) { mfma_step<S, 2>(st, acc); mfma_step<S, 3>(st, acc); }
}

template <int MODE, int S>
__global__ void __launch_bounds__(256, 2) expert_gemm_stream_kernel(GemmArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, r = lane & 15;

    // ---- m-tile -> expert (largest e with tile_start[e] <= tile) ----
    const int tile = blockIdx.y;
    if (tile >= a.tile_start[a.E]) return;
    int lo = 0, hi = a.E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.tile_start[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int row0 = a.offsets[e] + (tile - a.tile_start[e]) * kRowsPerTile;
    const int nrows = min(kRowsPerTile, a.offsets[e + 1] - row0);

    const int K = (MODE == kGemm2) ? a.I : a.H;
    const int wrows = (MODE == kGemm2) ? a.H : 2 * a.I;   // weight rows per expert
    int wrow[4];
    if constexpr (MODE == kGemm2) {
        const int n0 = blockIdx.x * 256 + wave * 64;
        if (n0 >= a.H) return;   // whole wave past the last output feature (no barriers in this mode)
#pragma unroll
        for (int j = 0; j < 4; ++j) wrow[j] = n0 + 16 * j;
    } else {
        const int f0 = blockIdx.x * 128 + wave * 32;
        wrow[0] = f0; wrow[1] = f0 + 16; wrow[2] = a.I + f0; wrow[3] = a.I + f0 + 16;
    }

    const size_t wstride = (size_t)K / 2, sstride = (size_t)K / 32;
    const uint8_t* wp[4];
    const uint8_t* sp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const size_t row = (size_t)e * wrows + wrow[j] + r;
        wp[j] = a.w + row * wstride + g * 16 * S;
        sp[j] = a.w_scale + row * sstride + g * S;
    }
    const int arow = row0 + min(r, nrows - 1);
    const uint8_t* xp = a.act + (size_t)arow * K;
    const int xoff_a = 32 * (S * (g >> 1)) + 16 * (g & 1);
    const int xoff_b = 32 * (S * (2 + (g >> 1))) + 16 * (g & 1);
    const uint8_t* xsp = a.act_scale + (size_t)arow * (K / kFp8Block) + (S * g) / 4;

    auto load = [&](Stage<S>& st, int kk) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int s = 0; s < S; ++s) st.w[j][s] = *(const uint4*)(wp[j] + kk / 2 + 16 * s);
            st.ws[j] = load_scale_bytes<S>(sp[j] + kk / 32);
        }
#pragma unroll
        for (int s = 0; s < S; ++s) {
            st.xa[s] = *(const uint4*)(xp + kk + xoff_a + 32 * s);
            st.xb[s] = *(const uint4*)(xp + kk + xoff_b + 32 * s);
        }
        st.xs = xsp[kk / kFp8Block];
    };

    v4f acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};

    constexpr int KS = 128 * S;
    const int nsteps = K / KS;
    Stage<S> s0, s1;
    load(s0, 0);
    for (int i = 0; i < nsteps; i += 2) {
        if (i + 1 < nsteps) load(s1, (i + 1) * KS);
        compute_stage<S>(s0, acc);
        if (i + 1 < nsteps) {
            if (i + 2 < nsteps) load(s0, (i + 2) * KS);
            compute_stage<S>(s1, acc);
        }
    }

    // ---- epilogues ----
    const int orow = row0 + r;
    const bool rvalid = r < nrows;
    if constexpr (MODE == kGemm2) {
        if (rvalid) {
            float* o = (float*)a.out + (size_t)orow * a.H + wrow[0] + 4 * g;
#pragma unroll
            for (int j = 0; j < 4; ++j) *(v4f*)(o + 16 * j) = acc[j];
        }
    } else if constexpr (MODE == kGemm1Preact) {
        if (rvalid) {
            float* o = (float*)a.out + (size_t)orow * (2 * a.I);
#pragma unroll
            for (int j = 0; j < 4; ++j) *(v4f*)(o + wrow[j] + 4 * g) = acc[j];
        }
    } else {
        // SwiGLU: h = silu(gate) * up, then FP8 over the workgroup's 128 features
        float h[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float g0 = acc[0][i], g1 = acc[1][i];
            h[i] = g0 / (1.0f + __expf(-g0)) * acc[2][i];
            h[4 + i] = g1 / (1.0f + __expf(-g1)) * acc[3][i];
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(h[i]));
        amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        __shared__ float red[4][16];
        if (g == 0) red[wave][r] = amax;
        __syncthreads();
        amax = fmaxf(fmaxf(red[0][r], red[1][r]), fmaxf(red[2][r], red[3][r]));
        const int ex = fp8_block_exponent(amax);
        if (rvalid) {
            uint8_t* q = (uint8_t*)a.out + (size_t)orow * a.I + wrow[0] + 4 * g;
            *(uint32_t*)q = pack_fp8x4(__builtin_amdgcn_ldexpf(h[0], -ex), __builtin_amdgcn_ldexpf(h[1], -ex),
                                       __builtin_amdgcn_ldexpf(h[2], -ex), __builtin_amdgcn_ldexpf(h[3], -ex));
            *(uint32_t*)(q + 16) = pack_fp8x4(__builtin_amdgcn_ldexpf(h[4], -ex), __builtin_amdgcn_ldexpf(h[5], -ex),
                                              __builtin_amdgcn_ldexpf(h[6], -ex), __builtin_amdgcn_ldexpf(h[7], -ex));
            if (wave == 0 && g == 0)
                a.out_scale[(size_t)orow * (a.I / kFp8Block) + blockIdx.x] = (uint8_t)(ex + 127);
        }
    }
}

template <int MODE>
static hipError_t launch_mode(const GemmArgs& a, int K, hipStream_t stream) {
    // grid.y: upper bound on m-tiles (sum over experts of ceil(n_e / 16));
    // workgroups past the real tile count exit at once.
    const int64_t tiles = (a.N + kRowsPerTile - 1) / kRowsPerTile + a.E;
    const int gx = (MODE == kGemm2) ? (a.H + 255) / 256 : a.I / 128;
    dim3 grid(gx, (unsigned)tiles), block(256);
    if (K % 512 == 0)
        hipLaunchKernelGGL((expert_gemm_stream_kernel<MODE, 4>), grid, block, 0, stream, a);
    else if (K % 256 == 0)
        hipLaunchKernelGGL((expert_gemm_stream_kernel<MODE, 2>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((expert_gemm_stream_kernel<MODE, 1>), grid, block, 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_expert_gemm(GemmMode mode, const GemmArgs& a, hipStream_t stream) {
    switch (mode) {
        case kGemm1Swiglu: return launch_mode<kGemm1Swiglu>(a, a.H, stream);
        case kGemm1Preact: return launch_mode<kGemm1Preact>(a, a.H, stream);
        case kGemm2: return launch_mode<kGemm2>(a, a.I, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace moe
