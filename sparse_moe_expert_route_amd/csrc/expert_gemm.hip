// Grouped expert GEMMs on the gfx950 block-scaled MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4), A = MXFP4 weights, B = FP8 activations.
//
// Experts are gate, up and down matrices with an intermediate width of 2,048
// (teardown, "How Big Is Each Expert?"), stored as MXFP4 ("Why Are the V2.6 Files Half
// the Size of V2.5?") and computed in FP8 e4m3 (vLLM recipe, "Overview").
// CDNA 4 executes MXFP4 directly (vLLM recipe, "AMD (MI355X, TP4)"), so the
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
// through LDS.  K is walked 128 per MFMA, S MFMAs per pipeline stage: one load
// instruction then covers 64 contiguous bytes of each of 16 weight rows (4
// lanes per row).  Each wave starts its stages a quarter of K after the wave
// before it and wraps around (see the K loop).  Lane (g, r) needs the scale of 32-block
// 4s + g at step s: it loads the row's 4S scale bytes of the stage and shifts
// byte g of word s to the bottom (op_sel 0).  The activation scale of step s is
// the row's scale byte of that 128-channel block.
#include "moe_internal.h"

namespace moe {

template <int S>
struct Stage {
    uint4 w[4][S];      // weight codes, 4 row-tiles x S steps
    uint32_t ws[4][S];  // weight scale words (byte g of word s used at step s)
    v8i x[S];           // activation operand of each step (both 16-byte halves)
    uint32_t xs[S];     // activation scale byte of each step
};

template <int S>
__device__ __forceinline__ void load_scale_words(const uint8_t* p, uint32_t (&w)[S]) {
    if constexpr (S == 4) {
        const uint4 v = *(const uint4*)p;
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (S == 2) {
        const uint2 v = *(const uint2*)p;
        w[0] = v.x; w[1] = v.y;
    } else {
        w[0] = *(const uint32_t*)p;
    }
}

struct Ptrs {
    const uint8_t* w[4];   // this lane's first weight byte of each row-tile
    const uint8_t* s[4];   // first scale byte of each weight row (packed: its first scale dword)
    const uint8_t* x;      // this lane's first activation byte
    const uint8_t* xs;     // first activation scale byte of the row
    uint32_t ls[4];        // LDS byte offset of each weight row's scales (scales staged in LDS)
    uint32_t lx;           // LDS byte offset of the activation row's scales
};

// Scales staged in LDS: the workgroup's 256 weight rows (K/32 bytes each),
// then its 16 activation rows (K/128 bytes each), unpadded, filled by direct
// global->LDS loads.  Weight scales in the layout they have in memory: row
// by row (canonical) or as the 16 packed 16-row groups one after another
// (packed: the 4 bytes of row r for 128 columns c at 64 c + 4 r of its group).
extern __shared__ __attribute__((aligned(16))) uint8_t stream_smem[];
__host__ __device__ constexpr int stream_lds_bytes(int K) { return 256 * (K / 32) + 16 * (K / 128); }

// s_waitcnt immediate that waits until at most n vector-memory loads are
// outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and
// lgkmcnt left at their maxima)
__host__ __device__ constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// global loads of one pipeline stage (S steps of 128 K) at K offset kk:
// 4*S weight loads and 2*S activation loads of 16 bytes per lane.  NT:
// non-temporal weight loads (the weights are read once per m-tile).
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
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
__device__ __forceinline__ void load_stage_mem(const Ptrs& P, int kk, Stage<S>& st) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            // canonical: 64 bytes of the row per step; packed: one 1 KB block
            // (16 rows x 64 bytes) per step, lane l at 16 l
            if constexpr (PK) st.w[j][s] = load_weight16<NT>(P.w[j] + 8 * kk + 1024 * s);
            else st.w[j][s] = load_weight16<NT>(P.w[j] + kk / 2 + 64 * s);
        }
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const uint4 lo = *(const uint4*)(P.x + kk + 128 * s);
        const uint4 hi = *(const uint4*)(P.x + kk + 128 * s + 64);
        st.x[s] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
}
constexpr int kStageLoads = 6 * 2;   // load_stage_mem<2, *>

// scales of the stage from LDS (two-step stages)
template <int S, bool PK>
__device__ __forceinline__ void load_stage_lds(const Ptrs& P, int kk, Stage<S>& st) {
    static_assert(S == 2, "LDS-staged scales use two-step stages");
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (PK) {
            // the two 128-column steps of the stage, 64 bytes apart
            st.ws[j][0] = *(const uint32_t*)(stream_smem + P.ls[j] + kk / 2);
            st.ws[j][1] = *(const uint32_t*)(stream_smem + P.ls[j] + kk / 2 + 64);
        } else {
            const uint2 v = *(const uint2*)(stream_smem + P.ls[j] + kk / 32);   // 8 scale bytes of the stage
            st.ws[j][0] = v.x; st.ws[j][1] = v.y;
        }
    }
    // both steps' activation scale bytes in one 16-bit read; the MFMA picks byte s
    st.xs[0] = *(const uint16_t*)(stream_smem + P.lx + kk / kFp8Block);
}

// scales of the stage from global memory
template <int S, bool PK>
__device__ __forceinline__ void load_stage_gscales(const Ptrs& P, int kk, Stage<S>& st) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (PK) {
#pragma unroll
            for (int s = 0; s < S; ++s) st.ws[j][s] = *(const uint32_t*)(P.s[j] + (kk / 128 + s) * 64);
        } else {
            load_scale_words<S>(P.s[j] + kk / 32, st.ws[j]);
        }
    }
    // separate byte loads (a relaxed atomic load is never merged with its
    // neighbour, which would need VALU extraction and an early wait)
#pragma unroll
    for (int s = 0; s < S; ++s) st.xs[s] = __atomic_load_n(P.xs + kk / kFp8Block + s, __ATOMIC_RELAXED);
}

template <int S, bool SL, bool PK, bool NT>
__device__ __forceinline__ Stage<S> load_stage(const Ptrs& P, int kk) {
    Stage<S> st;
    load_stage_mem<S, PK, NT>(P, kk, st);
    if constexpr (SL) load_stage_lds<S, PK>(P, kk, st);
    else load_stage_gscales<S, PK>(P, kk, st);
    return st;
}

template <int S, bool SL, int s>
__device__ __forceinline__ void mfma_step(const Stage<S>& st, v4f (&acc)[4], int gshift) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint4 w = st.w[j][s];
        const v8i a = {(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
        if constexpr (SL)
            acc[j] = mfma_w4a8<0, s>(a, st.x[s], acc[j], (int)(st.ws[j][s] >> gshift), (int)st.xs[0]);
        else
            acc[j] = mfma_w4a8<0, 0>(a, st.x[s], acc[j], (int)(st.ws[j][s] >> gshift), (int)st.xs[s]);
    }
}

template <int S, bool SL>
__device__ __forceinline__ void compute_stage(const Stage<S>& st, v4f (&acc)[4], int gshift) {
    mfma_step<S, SL, 0>(st, acc, gshift);
    if constexpr (S > 1) mfma_step<S, SL, 1>(st, acc, gshift);
    if constexpr (S > 2) { mfma_step<S, SL, 2>(st, acc, gshift); mfma_step<S, SL, 3>(st, acc, gshift); }
}

typedef __attribute__((address_space(3))) void lds_void;

// Start the copy of the workgroup's scales into LDS: weight rows in the order
// of the waves' row-tiles (GEMM-1: 128 gate rows then the 128 matching up
// rows; GEMM-2: 256 consecutive output rows), 16 bytes per lane, then the
// activation rows of the m-tile (clamped to its last real row), 4 bytes per
// lane.  Direct global->LDS loads: lane l of a load lands at base + size * l.
// The caller waits on the load counter and barriers before reading.
// Needs K % 512 == 0 and stream_lds_bytes(K) <= 64 KB (at most 15 weight and
// 4 activation loads per wave).
template <int MODE, bool PK>
__device__ __forceinline__ void stage_scales_issue(const GemmArgs& a, int e, int K, int row0, int nrows) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int SB = K / 32, n16 = SB / 16;                   // 16-byte pieces per weight row
    const int wrows = (MODE == kGemm2) ? a.H : 2 * a.I;
    const uint8_t* base = a.w_scale + (size_t)e * wrows * SB;
    for (int q = 0; q < n16; ++q) {
        const int m = 4 * q + wave;                         // 1 KB piece of the LDS image
        if constexpr (PK) {
            // image group G (K/2 bytes) is memory group gq, contiguous
            const int o = 1024 * m + 16 * lane, G = o / (K / 2), off = o - G * (K / 2);
            int gq;
            if constexpr (MODE == kGemm2) gq = min((int)blockIdx.x * 16 + G, wrows / 16 - 1);   // past H: never read
            else gq = (G < 8 ? 0 : a.I / 16 - 8) + blockIdx.x * 8 + G;
            __builtin_amdgcn_global_load_lds(base + (size_t)gq * (K / 2) + off, (lds_void*)(stream_smem + 1024 * m), 16, 0, 0);
        } else {
            const int i = 64 * m + lane, R = i / n16, c = i - R * n16;
            int grow;
            if constexpr (MODE == kGemm2) grow = min((int)blockIdx.x * 256 + R, wrows - 1);   // rows past H: never read
            else grow = (R < 128 ? 0 : a.I - 128) + blockIdx.x * 128 + R;
            __builtin_amdgcn_global_load_lds(base + (size_t)grow * SB + 16 * c, (lds_void*)(stream_smem + 1024 * m), 16, 0, 0);
        }
    }
    const int XB = K / kFp8Block, n4 = XB / 4;              // dwords per activation row, 16 rows
    const int i = 64 * wave + lane;                         // 64 dwords per load, 16 * n4 in all
    if (i < 16 * n4) {
        const int rr = i / n4, c = i - rr * n4;
        int srow = row0 + min(rr, nrows - 1);
        if (a.act_rows) srow = a.act_rows[srow];
        const uint8_t* src = a.act_scale + (size_t)srow * XB + 4 * c;
        __builtin_amdgcn_global_load_lds(src, (lds_void*)(stream_smem + 256 * SB + 256 * wave), 4, 0, 0);
    }
}

template <int MODE, int S, bool SL, bool PK, bool NT>
__global__ void __launch_bounds__(256, 2) expert_gemm_stream_kernel(GemmArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
    int wrow[4];
    bool live = true;   // GEMM-2: false for a wave past the last output feature
    if constexpr (MODE == kGemm2) {
        int n0 = blockIdx.x * 256 + wave * 64;
        live = n0 < a.H;
        if (!live) n0 = a.H - 64;   // keeps its loads in bounds until it leaves after the barrier
#pragma unroll
        for (int j = 0; j < 4; ++j) wrow[j] = n0 + 16 * j;
    } else {
        const int f0 = blockIdx.x * 128 + wave * 32;
        wrow[0] = f0; wrow[1] = f0 + 16; wrow[2] = a.I + f0; wrow[3] = a.I + f0 + 16;
    }

    const size_t wstride = (size_t)K / 2, sstride = (size_t)K / 32;
    Ptrs P;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const size_t row = (size_t)e * wrows + wrow[j] + r;
        // packed: the row's 16-row group, lane l's 16 bytes at 16 l of each block
        if constexpr (PK) P.w[j] = a.w + (row - r) * wstride + 16 * lane;
        else P.w[j] = a.w + row * wstride + 16 * g;
        // packed scales: the row's group at (row - r) K/32, row r's dword at 4 r of each step
        if constexpr (PK) P.s[j] = a.w_scale + (row - r) * sstride + 4 * r;
        else P.s[j] = a.w_scale + row * sstride;
    }
    const int gshift = 8 * g;
    int arow = row0 + min(r, nrows - 1);
    if (a.act_rows) arow = a.act_rows[arow];
    P.x = a.act + (size_t)arow * K + 16 * g;
    P.xs = a.act_scale + (size_t)arow * (K / kFp8Block);
    if constexpr (SL) {
        // LDS row of tile j: the wave's 64 rows in the order the scales are staged
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int lrow = (MODE == kGemm2) ? 64 * wave + 16 * j : (j >> 1) * 128 + 32 * wave + 16 * (j & 1);
            if constexpr (PK) P.ls[j] = (uint32_t)((lrow / 16) * (K / 2) + 4 * r);
            else P.ls[j] = (uint32_t)((lrow + r) * (K / 32));
        }
        P.lx = (uint32_t)(256 * (K / 32) + r * (K / kFp8Block));
    }

    v4f acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};

    // software pipeline over two register stages, ping-pong without copies:
    // while one stage is multiplied the other one's loads are in flight, and
    // each wait covers only the stage about to be consumed.  Loads past the
    // end re-read the last stage (an L2 hit) so that every load is unconditional.
    // The scheduling barriers keep each phase's instructions in place, so the
    // in-order load counter lets every wait cover exactly one stage.
    //
    // Wave w walks the K stages starting at stage w * nstage / 4, wrapping
    // around.  The 16 weight-row groups of a workgroup lie K/2 * 16 bytes apart
    // (16 or 32 KiB for K = 2048 or 4096); read in step, the four waves' loads
    // fall on the same few HBM channels, and staggered they spread (in the
    // packed-weight read pattern of the microbenchmark: 5.35 -> 6.05 TB/s at
    // 32 KiB, 5.56 -> 6.10 at 16 KiB).  Each wave sums its own rows, so only the
    // order of its fp32 additions changes.
    constexpr int KS = 128 * S;
    const int nstage = K / KS;
    const int st0 = __builtin_amdgcn_readfirstlane(wave * nstage / 4);
    // K offset of the wave's i-th stage (past the last: the last again)
    auto koff = [&](int i) __attribute__((always_inline)) {
        int q = min(i, nstage - 1) + st0;
        q = q >= nstage ? q - nstage : q;
        return q * KS;
    };
    Stage<S> s0, s1;
    if constexpr (SL) {
        // the scale copy overlaps the first two stages' weight and activation
        // loads: wait for the copy alone (the load counter retires in order;
        // the two stages issue kStageLoads loads each), then barrier
        stage_scales_issue<MODE, PK>(a, e, K, row0, nrows);
        __builtin_amdgcn_sched_barrier(0);
        load_stage_mem<S, PK, NT>(P, koff(0), s0);
        load_stage_mem<S, PK, NT>(P, koff(1), s1);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * kStageLoads));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (!live) return;
        load_stage_lds<S, PK>(P, koff(0), s0);
        load_stage_lds<S, PK>(P, koff(1), s1);
    } else {
        s0 = load_stage<S, SL, PK, NT>(P, koff(0));
        s1 = load_stage<S, SL, PK, NT>(P, koff(1));
    }
    int i = 0;
    for (; i + 2 <= nstage; i += 2) {
        compute_stage<S, SL>(s0, acc, gshift);
        __builtin_amdgcn_sched_barrier(0);
        s0 = load_stage<S, SL, PK, NT>(P, koff(i + 2));
        __builtin_amdgcn_sched_barrier(0);
        compute_stage<S, SL>(s1, acc, gshift);
        __builtin_amdgcn_sched_barrier(0);
        s1 = load_stage<S, SL, PK, NT>(P, koff(i + 3));
        __builtin_amdgcn_sched_barrier(0);
    }
    if (i < nstage) compute_stage<S, SL>(s0, acc, gshift);   // odd number of stages: the last one is in s0

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

template <int MODE, bool PK, bool NT>
static hipError_t launch_mode(const GemmArgs& a, int K, hipStream_t stream) {
    // grid.y: upper bound on m-tiles (sum over experts of ceil(n_e / 16));
    // workgroups past the real tile count exit at once.
    const int tiles = max_tiles(a.N, a.E, kRowsPerTile);
    const int gx = (MODE == kGemm2) ? (a.H + 255) / 256 : a.I / 128;
    dim3 grid(gx, (unsigned)tiles), block(256);
    // stages of 256 K (two MFMA steps), two stages in flight per wave: about
    // 16 KB of weights in flight per wave, over 100 KB per CU.
    // Scales are staged in LDS once per workgroup where they fit: per-stage
    // scale loads would cost as many memory requests as the weights.
    if (K % 512 == 0 && stream_lds_bytes(K) <= 65536)
        hipLaunchKernelGGL((expert_gemm_stream_kernel<MODE, 2, true, PK, NT>), grid, block, stream_lds_bytes(K), stream, a);
    else if (K % 256 == 0)
        hipLaunchKernelGGL((expert_gemm_stream_kernel<MODE, 2, false, PK, NT>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((expert_gemm_stream_kernel<MODE, 1, false, PK, NT>), grid, block, 0, stream, a);
    return hipGetLastError();
}

template <int MODE>
static hipError_t launch_mode(const GemmArgs& a, int K, hipStream_t stream) {
    // Non-temporal weight loads where each weight-row group is long (K >= 6144:
    // 48 KiB per 16-row group and more).  In the microbenchmark of the packed
    // read pattern (staggered waves) they read 6.39 against 6.03 TB/s at 48 KiB
    // groups, the same at 32 KiB and less at 16 KiB (5.82 against 6.10).
    const bool nt = K >= 6144;
    if (a.packed) return nt ? launch_mode<MODE, true, true>(a, K, stream) : launch_mode<MODE, true, false>(a, K, stream);
    return nt ? launch_mode<MODE, false, true>(a, K, stream) : launch_mode<MODE, false, false>(a, K, stream);
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
