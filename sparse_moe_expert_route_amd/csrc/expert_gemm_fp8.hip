// Grouped expert GEMMs for FP8 block-scaled experts: e4m3 weight codes with
// one float32 scale per 128 x 128 block (the earlier, V2.5 expert format in
// the teardown's "Why Are the V2.6 Files Half the Size of V2.5?" table;
// computed block-wise in e4m3 at 128 x 128 granularity, vLLM recipe
// "Overview"), times FP8 activations with one float32 scale per row per 128
// channels.
//
// The block-scaled MFMA only takes power-of-two (e8m0) scales, and a float32
// scale is not one.  So each 128-deep K block is multiplied with unit scales
// into a fresh accumulator (v_mfma_scale_f32_16x16x128_f8f6f4, both operands
// e4m3), and the running sum gains that partial times the product of the two
// float32 scales of the block: four FMAs per lane per MFMA.
//
// Operand layout of the 16x16x128 instruction for e4m3 x e4m3 (lane l,
// g = l/16, r = l%16): each operand's bytes 0..15 are k = 16g + i and bytes
// 16..31 are k = 64 + 16g + i; the result lane holds D[4g + i][r].  A (16
// weight rows) and B (16 activation rows) use the same layout.
//
// Streaming structure, for shapes with few rows per expert: a workgroup owns
// one m-tile of 16 rows of one expert and a block of weight rows (gate/up:
// 128 features = 128 gate rows and the 128 matching up rows, which is one
// 128-channel block of h, so the block maximum for the FP8 requantisation of
// h is a workgroup reduction; down: 256 output features).  Every weight byte
// is read once per m-tile, straight into registers.  Each 16-row weight tile
// lies inside one 128-row scale block, so its scale is wave-uniform and comes
// through the scalar cache.
#include "moe_internal.h"

namespace moe {

namespace {

template <int S>
struct StageF8 {
    uint4 w[4][S][2];   // weight codes: row-tile j, step s, bytes 0..15 / 16..31 of the lane
    v8i x[S];           // activation operand of each step
    float xs[S];        // activation scale of the lane's row for each step's K block
    float ws[2][S];     // weight block scales (gate/up: gate and up rows; down: one row block)
};

struct PtrsF8 {
    const uint8_t* w[4];    // this lane's first weight byte of each row-tile
    const float* ws[2];     // first scale of each weight row block (wave-uniform)
    const uint8_t* x;       // this lane's first activation byte
    const float* xs;        // first activation scale of the lane's row
};

__device__ __forceinline__ v4f mfma_f8f8(v8i a, v8i b) {
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    // format 0 = e4m3 for both operands; scale byte 127 = 2^0
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 127, 0, 127);
}

typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
// NT: a non-temporal load (the weights are read once per m-tile)
template <bool NT>
__device__ __forceinline__ uint4 load_weight16(const uint8_t* p) {
    if constexpr (NT) {
        const v4u32 v = __builtin_nontemporal_load((const v4u32*)p);
        return make_uint4(v.x, v.y, v.z, v.w);
    } else {
        return *(const uint4*)p;
    }
}

template <int S, bool PK, bool NT>
__device__ __forceinline__ StageF8<S> load_stage(const PtrsF8& P, int kk, int K) {
    StageF8<S> st;
    const int kb = kk / kFp8Block;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            // packed: one 2 KB block per 16 rows x 128 columns, lane l's bytes
            // 0..15 at 16 l and 16..31 at 1024 + 16 l; canonical: the row's
            // bytes 16g and 64 + 16g of the K block
            if constexpr (PK) {
                st.w[j][s][0] = load_weight16<NT>(P.w[j] + 2048 * (kb + s));
                st.w[j][s][1] = load_weight16<NT>(P.w[j] + 2048 * (kb + s) + 1024);
            } else {
                st.w[j][s][0] = load_weight16<NT>(P.w[j] + kk + 128 * s);
                st.w[j][s][1] = load_weight16<NT>(P.w[j] + kk + 128 * s + 64);
            }
        }
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const uint4 lo = *(const uint4*)(P.x + kk + 128 * s);
        const uint4 hi = *(const uint4*)(P.x + kk + 128 * s + 64);
        st.x[s] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    if constexpr (S == 2) {
        const float2 v = *(const float2*)(P.xs + kb);
        st.xs[0] = v.x; st.xs[1] = v.y;
    } else {
        st.xs[0] = P.xs[kb];
    }
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int s = 0; s < S; ++s) st.ws[b][s] = P.ws[b][kb + s];
    (void)K;
    return st;
}

template <int MODE, int S>
__device__ __forceinline__ void compute_stage(const StageF8<S>& st, v4f (&acc)[4]) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint4 lo = st.w[j][s][0], hi = st.w[j][s][1];
            const v8i a = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            const v4f part = mfma_f8f8(a, st.x[s]);
            // gate/up: tiles 0, 1 are gate rows, 2, 3 the up rows
            const float c = st.ws[(MODE != kGemm2 && j >= 2) ? 1 : 0][s] * st.xs[s];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[j][i] = __builtin_fmaf(part[i], c, acc[j][i]);
        }
    }
}

}  // namespace

template <int MODE, int S, bool PK, bool NT>
__global__ void __launch_bounds__(256, 2) expert_gemm_fp8_stream_kernel(GemmArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, r = lane & 15;

    // ---- m-tile: expert, first row, rows ----
    // workgroup 0 reports whether the offsets are valid (error word 1)
    if (a.err && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 64) {
        const uint32_t bad = offsets_error(a.offsets, a.E, a.N);
        if (threadIdx.x == 0) *a.err = bad;
    }
    const int4 ti = find_stream_tile(a.offsets, a.E, (int)a.N, blockIdx.y);
    if (ti.x < 0) return;   // past the last m-tile
    const int e = ti.x, row0 = ti.y, nrows = ti.z;

    const int K = (MODE == kGemm2) ? a.I : a.H;
    const int wrows = (MODE == kGemm2) ? a.H : 2 * a.I;   // weight rows per expert
    const int KB = K / kFp8Block;
    int wrow[4];
    bool live = true;   // down: false for a wave past the last output feature
    if constexpr (MODE == kGemm2) {
        int n0 = blockIdx.x * 256 + wave * 64;
        live = n0 < a.H;
        if (!live) n0 = a.H - 64;   // keeps its loads in bounds; it stores nothing
#pragma unroll
        for (int j = 0; j < 4; ++j) wrow[j] = n0 + 16 * j;
    } else {
        const int f0 = blockIdx.x * 128 + wave * 32;
        wrow[0] = f0; wrow[1] = f0 + 16; wrow[2] = a.I + f0; wrow[3] = a.I + f0 + 16;
    }

    PtrsF8 P;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const size_t row = (size_t)e * wrows + wrow[j] + r;
        if constexpr (PK) P.w[j] = a.w + (row - r) * K + 16 * lane;
        else P.w[j] = a.w + row * K + 16 * g;
    }
    const float* wsc = (const float*)a.w_scale;
    const size_t sblk0 = (size_t)e * (wrows / kFp8Block);
    P.ws[0] = wsc + (sblk0 + wrow[0] / kFp8Block) * KB;
    P.ws[1] = wsc + (sblk0 + wrow[(MODE == kGemm2) ? 0 : 2] / kFp8Block) * KB;
    int arow = row0 + min(r, nrows - 1);
    if (a.act_rows) arow = a.act_rows[arow];
    P.x = a.act + (size_t)arow * K + 16 * g;
    P.xs = (const float*)a.act_scale + (size_t)arow * KB;

    v4f acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};

    // two register stages in a copy-free ping-pong: while one stage is
    // multiplied the other one's loads are in flight.  Loads past the end
    // re-read the last stage (an L2 hit) so that every load is unconditional.
    // Wave w walks the stages starting at stage w * nstage / 4, wrapping
    // around, so that the four waves' loads of the workgroup's weight-row
    // groups (16 K bytes apart) do not fall on the same HBM channels at once;
    // only the order of each wave's fp32 additions changes.
    constexpr int KS = 128 * S;
    const int nstage = K / KS;
    const int st0 = __builtin_amdgcn_readfirstlane(wave * nstage / 4);
    auto koff = [&](int i) __attribute__((always_inline)) {
        int q = min(i, nstage - 1) + st0;
        q = q >= nstage ? q - nstage : q;
        return q * KS;
    };
    StageF8<S> s0 = load_stage<S, PK, NT>(P, koff(0), K);
    StageF8<S> s1 = load_stage<S, PK, NT>(P, koff(1), K);
    int i = 0;
    for (; i + 2 <= nstage; i += 2) {
        compute_stage<MODE, S>(s0, acc);
        __builtin_amdgcn_sched_barrier(0);
        s0 = load_stage<S, PK, NT>(P, koff(i + 2), K);
        __builtin_amdgcn_sched_barrier(0);
        compute_stage<MODE, S>(s1, acc);
        __builtin_amdgcn_sched_barrier(0);
        s1 = load_stage<S, PK, NT>(P, koff(i + 3), K);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (i < nstage) compute_stage<MODE, S>(s0, acc);   // odd number of stages: the last one is in s0

    // ---- epilogues ----
    const int orow = row0 + r;
    const bool rvalid = r < nrows;
    if constexpr (MODE == kGemm2) {
        if (live && rvalid) {
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
        // SwiGLU h = silu(gate) * up, then FP8 with a float32 scale over the
        // workgroup's 128 features: s = amax / 448, codes of h / s
        float h[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float g0 = acc[0][i], g1 = acc[1][i];
            h[i] = silu_f32(g0) * acc[2][i];
            h[4 + i] = silu_f32(g1) * acc[3][i];
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
        const float sc = fp8_f32_scale(amax);
        const float d = amax > 0.0f ? sc : 1.0f;
        if (rvalid) {
            float q[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = fp8_f32_quotient(h[i], d);
            uint8_t* o = (uint8_t*)a.out + (size_t)orow * a.I + wrow[0] + 4 * g;
            *(uint32_t*)o = pack_fp8x4(q[0], q[1], q[2], q[3]);
            *(uint32_t*)(o + 16) = pack_fp8x4(q[4], q[5], q[6], q[7]);
            if (wave == 0 && g == 0) ((float*)a.out_scale)[(size_t)orow * (a.I / kFp8Block) + blockIdx.x] = sc;
        }
    }
}

template <int MODE, bool PK, bool NT>
static hipError_t launch_fp8_mode(const GemmArgs& a, int K, hipStream_t stream) {
    // grid.y: upper bound on m-tiles (sum over experts of ceil(n_e / 16));
    // workgroups past the real tile count exit at once.
    const int tiles = max_tiles(a.N, a.E, kRowsPerTile);
    const int gx = (MODE == kGemm2) ? (a.H + 255) / 256 : a.I / 128;
    dim3 grid(gx, (unsigned)tiles), block(256);
    if (K % 256 == 0)
        hipLaunchKernelGGL((expert_gemm_fp8_stream_kernel<MODE, 2, PK, NT>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((expert_gemm_fp8_stream_kernel<MODE, 1, PK, NT>), grid, block, 0, stream, a);
    return hipGetLastError();
}

template <int MODE>
static hipError_t launch_fp8_mode(const GemmArgs& a, int K, hipStream_t stream) {
    const bool nt = K >= 6144;   // non-temporal weight loads for long weight-row groups
    if (a.packed) return nt ? launch_fp8_mode<MODE, true, true>(a, K, stream) : launch_fp8_mode<MODE, true, false>(a, K, stream);
    return nt ? launch_fp8_mode<MODE, false, true>(a, K, stream) : launch_fp8_mode<MODE, false, false>(a, K, stream);
}

hipError_t launch_expert_gemm_fp8(GemmMode mode, const GemmArgs& a, hipStream_t stream) {
    switch (mode) {
        case kGemm1Swiglu: return launch_fp8_mode<kGemm1Swiglu>(a, a.H, stream);
        case kGemm1Preact: return launch_fp8_mode<kGemm1Preact>(a, a.H, stream);
        case kGemm2: return launch_fp8_mode<kGemm2>(a, a.I, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace moe
