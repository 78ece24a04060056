// Grouped expert GEMMs for shapes with many rows per expert (prefill):
// LDS-tiled, on the 32x32x64 block-scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4), A = MXFP4 weights, B = FP8 activations.
//
// Same computation as the streaming kernel (expert_gemm.hip): experts are
// gate/up/down projections around a 2,048-wide middle (teardown, "How Big Is
// Each Expert?"), stored as MXFP4 and computed in FP8 e4m3 (vLLM recipe,
// "Overview"); e2m1 codes and e8m0 scales go to the MFMA as stored.
//
// Operand layout of the 32x32x64 instruction (lane l, g = l/32, r = l%32):
//   FP4 operand: 16 bytes = k 32g .. 32g+31 (low nibble first);
//   FP8 operand: bytes 0..15 -> k = 16g + i, bytes 16..31 -> k = 32 + 16g + i;
//   scale byte op_sel of lane l scales row r, k in [32g, 32g+32);
//   result: acc[i] of lane l is D[8*(i/4) + 4g + (i%4)][r].
// K is walked in stages of 256 = 4 MFMA steps; step s pairs logical 32-block
// b with physical block 4b + s, so each lane's weight bytes for a stage are 64
// contiguous bytes and its 4 weight scales one dword (op_sel = s).
//
// Work decomposition: an item is (m-tile of 128 rows of one expert, n-block).
// A workgroup of 4 waves computes 128 rows x (128 h-features = 256 W13 rows)
// for the gate/up GEMM, or 128 rows x 256 output features for the down GEMM.
// The activation tile is staged through LDS by direct global->LDS loads
// (global_load_lds_dwordx4: no staging registers), double-buffered, with the
// 16-byte chunk c of row p stored at chunk slot c ^ (p mod 16) so that the 32
// rows read by one MFMA operand fetch hit distinct banks; every wave streams
// its own weight rows straight into registers.  The grid is persistent: workgroups on one XCD
// (block id mod 8) take a contiguous 1/8 of the item list.  Items are grouped
// by expert; an expert's m-tiles go in chunks of four, each chunk ordered
// n-block major, m-tile minor: the m-tiles that read the same block of weight
// rows run side by side on one L2 (weights come from HBM about once per
// chunk), and the chunk's activations stay in L2 across its n-blocks.
#include "moe_internal.h"

#include <type_traits>

namespace moe {

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kTileRows = 128;            // m-tile rows
constexpr int kStageK = 256;              // K per LDS stage (bytes of an FP8 row)
constexpr int kMChunk = 4;                // m-tiles of one expert scheduled together

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane, global -> LDS at lds_base + 16 * lane (lds_base wave-uniform)
__device__ __forceinline__ void dma16(const void* g, void* lds_base) {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_base, 16, 0, 0);
}
// 2 bytes per lane, global -> LDS: the LDS slot of each lane is a dword
// (lds_base + 4 * lane, upper half zero)
__device__ __forceinline__ void dma2(const void* g, void* lds_base) {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_base, 2, 0, 0);
}
__device__ __forceinline__ int swz(int row, int chunk) { return row * kStageK + ((chunk ^ (row & 15)) << 4); }

template <int OPSEL_A>
__device__ __forceinline__ v16f mfma32_w4a8(v8i a, v8i b, v16f c, int scale_a, int scale_b) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 0, OPSEL_A, scale_a, 0, scale_b);
}

// Activation stage ring in LDS: three buffers, declared as separate objects
// so that the compiler's wait tracking for direct global->LDS loads can tell
// a buffer being filled from the one being read.
__shared__ __attribute__((aligned(16))) uint8_t tl_act0[kTileRows * kStageK];
__shared__ __attribute__((aligned(16))) uint8_t tl_act1[kTileRows * kStageK];
__shared__ __attribute__((aligned(16))) uint8_t tl_act2[kTileRows * kStageK];
// activation scales: 2 bytes per row in dword slots; wave w's 32 rows at
// slots 64w .. 64w+31 (its lanes 32..63 write a copy above them)
__shared__ __attribute__((aligned(16))) uint32_t tl_scl0[2 * kTileRows];
__shared__ __attribute__((aligned(16))) uint32_t tl_scl1[2 * kTileRows];
__shared__ __attribute__((aligned(16))) uint32_t tl_scl2[2 * kTileRows];

// s_waitcnt immediate: at most n vector-memory operations outstanding (gfx9
// encoding, vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt at their maxima)
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// vector-memory operations one stage issues per wave: 8 activation pieces,
// 1 activation-scale piece, 8 weight loads, 2 weight-scale loads
constexpr int kStageLoads = 19;

// Workgroup barrier that waits on nothing: the callers first wait for their
// own direct-to-LDS loads with an explicit vmcnt.  The empty asm statements
// keep the compiler from moving memory accesses across it (a release fence
// would also wait for every direct-to-LDS load in flight).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

struct WStage {
    uint4 w[2][4];    // 2 weight tiles x 4 steps of 16 bytes
    uint32_t ws[2];   // 4 scale bytes per tile
};

// Per-item state of the stage loop.
struct TileCtx {
    const uint8_t* act;        // FP8 activations [N][K]
    const uint8_t* act_scale;  // [N][K/128]
    const uint8_t* wp0;        // this lane's weight bytes, tile 0 (k = 0)
    const uint8_t* wp1;        // tile 1
    const uint8_t* sp0;        // this lane's weight scale bytes, tile 0
    const uint8_t* sp1;        // tile 1
    int K, nstage, row0, nrows;
};

// The K loop of one item.  The three activation buffers come in as restrict
// pointers: the compiler then tags every LDS access with the buffer it
// touches, and its wait tracking for direct global->LDS loads (which would
// otherwise make each LDS read wait for every such load in flight) lets a
// buffer be read while the others are being filled.
__device__ __forceinline__ void tile_kloop(const TileCtx& c, v16f (&acc)[4][2],
                                           uint8_t* __restrict__ act0, uint8_t* __restrict__ act1,
                                           uint8_t* __restrict__ act2, uint32_t* __restrict__ scl0,
                                           uint32_t* __restrict__ scl1, uint32_t* __restrict__ scl2) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, r = lane & 31;
    const int K = c.K, nstage = c.nstage, row0 = c.row0, nrows = c.nrows;
    const uint8_t* wp0 = c.wp0; const uint8_t* wp1 = c.wp1;
    const uint8_t* sp0 = c.sp0; const uint8_t* sp1 = c.sp1;
    auto abuf = [&](auto bc) -> uint8_t* {
        constexpr int B = decltype(bc)::value;
        if constexpr (B == 0) return act0; else if constexpr (B == 1) return act1; else return act2;
    };
    auto sbuf = [&](auto bc) -> uint32_t* {
        constexpr int B = decltype(bc)::value;
        if constexpr (B == 0) return scl0; else if constexpr (B == 1) return scl1; else return scl2;
    };
    auto load_w = [&](WStage& ws, int st) {
        const int kb = st * (kStageK / 2);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            ws.w[0][s] = *(const uint4*)(wp0 + kb + 16 * s);
            ws.w[1][s] = *(const uint4*)(wp1 + kb + 16 * s);
        }
        ws.ws[0] = *(const uint32_t*)(sp0 + st * (kStageK / 32));
        ws.ws[1] = *(const uint32_t*)(sp1 + st * (kStageK / 32));
    };

    // activation stage: 128 rows x 256 bytes.  Wave w moves rows 32w .. 32w+31,
    // four rows (64 lanes x 16 bytes) per instruction; lane i of an instruction
    // fills chunk slot i%16 of row 4p + i/16 with the global chunk that the
    // swizzle maps there.  Every wave also moves the two scale bytes of its
    // rows (twice: all 64 lanes), so that every wave issues kStageLoads loads.
    auto dma_act = [&](auto bufc, int st) {
        const int k0 = st * kStageK;
        uint8_t* lds = abuf(bufc);
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int row = 32 * wave + 4 * p + (lane >> 4);
            const int chunk = (lane & 15) ^ (row & 15);
            const int rr = row0 + min(row, nrows - 1);
            dma16(c.act + (size_t)rr * K + k0 + 16 * chunk, lds + (32 * wave + 4 * p) * kStageK);
        }
        {
            const int rr = row0 + min(32 * wave + (lane & 31), nrows - 1);
            dma2(c.act_scale + (size_t)rr * (K / kFp8Block) + k0 / kFp8Block, sbuf(bufc) + 64 * wave);
        }
    };

#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[j][t][i] = 0.0f;

    // Three-deep pipeline: stage st+2's activations (into LDS) and weights
    // (into a third register set) are issued while stage st is multiplied,
    // so each load has two stages of MFMA work to land.  Buffer and
    // register set of stage st are st mod 3; the stage loop is unrolled by
    // three so that every set is a fixed set of registers.
    WStage w0, w1, w2;
    auto stage = [&](auto setc, int st, const WStage& wc, WStage& wn) {
        constexpr int SET = decltype(setc)::value;
        constexpr int NXT = (SET + 2) % 3;
        // stage st landed (only stage st+1's loads may still be in flight),
        // in every wave: then its buffer may be read, and the buffer of
        // stage st-1, which stage st+2 refills, is no longer read.  Near
        // the end the prefetch re-reads the last stage into a free buffer,
        // so the body has no branch and the load count never changes.
        __builtin_amdgcn_s_waitcnt(vmcnt_only(kStageLoads));
        lds_barrier();
        dma_act(std::integral_constant<int, NXT>{}, min(st + 2, nstage - 1));
        load_w(wn, min(st + 2, nstage - 1));
        __builtin_amdgcn_sched_barrier(0);
        const uint8_t* lds = abuf(setc);
        int bs[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) bs[j] = (sbuf(setc)[64 * j + r] >> (8 * g)) & 0xFF;
        // B operands one MFMA step ahead of their use
        v8i B[2][4];
        auto read_b = [&](v8i (&Bd)[4], int s) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 32 * j + r;
                const uint4 lo4 = *(const uint4*)(lds + swz(row, 2 * s + g));
                const uint4 hi4 = *(const uint4*)(lds + swz(row, 8 + 2 * s + g));
                Bd[j][0] = lo4.x; Bd[j][1] = lo4.y; Bd[j][2] = lo4.z; Bd[j][3] = lo4.w;
                Bd[j][4] = hi4.x; Bd[j][5] = hi4.y; Bd[j][6] = hi4.z; Bd[j][7] = hi4.w;
            }
        };
        read_b(B[0], 0);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < 3) read_b(B[(s + 1) & 1], s + 1);
            v8i A0, A1;
            A0[0] = wc.w[0][s].x; A0[1] = wc.w[0][s].y; A0[2] = wc.w[0][s].z; A0[3] = wc.w[0][s].w;
            A1[0] = wc.w[1][s].x; A1[1] = wc.w[1][s].y; A1[2] = wc.w[1][s].z; A1[3] = wc.w[1][s].w;
            A0[4] = A0[5] = A0[6] = A0[7] = 0;
            A1[4] = A1[5] = A1[6] = A1[7] = 0;
            const v8i (&Bc)[4] = B[s & 1];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                switch (s) {
                    case 0:
                        acc[j][0] = mfma32_w4a8<0>(A0, Bc[j], acc[j][0], (int)wc.ws[0], bs[j]);
                        acc[j][1] = mfma32_w4a8<0>(A1, Bc[j], acc[j][1], (int)wc.ws[1], bs[j]);
                        break;
                    case 1:
                        acc[j][0] = mfma32_w4a8<1>(A0, Bc[j], acc[j][0], (int)wc.ws[0], bs[j]);
                        acc[j][1] = mfma32_w4a8<1>(A1, Bc[j], acc[j][1], (int)wc.ws[1], bs[j]);
                        break;
                    case 2:
                        acc[j][0] = mfma32_w4a8<2>(A0, Bc[j], acc[j][0], (int)wc.ws[0], bs[j]);
                        acc[j][1] = mfma32_w4a8<2>(A1, Bc[j], acc[j][1], (int)wc.ws[1], bs[j]);
                        break;
                    default:
                        acc[j][0] = mfma32_w4a8<3>(A0, Bc[j], acc[j][0], (int)wc.ws[0], bs[j]);
                        acc[j][1] = mfma32_w4a8<3>(A1, Bc[j], acc[j][1], (int)wc.ws[1], bs[j]);
                        break;
                }
            }
            // keep each step's LDS reads next to the step before their use
            // (hoisting them all would need every B operand of the stage live)
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    dma_act(I0{}, 0);
    load_w(w0, 0);
    dma_act(I1{}, min(1, nstage - 1));
    load_w(w1, min(1, nstage - 1));
    int st = 0;
    for (; st + 3 <= nstage; st += 3) {
        stage(I0{}, st, w0, w2);
        stage(I1{}, st + 1, w1, w0);
        stage(I2{}, st + 2, w2, w1);
    }
    if (st < nstage) stage(I0{}, st, w0, w2);
    if (st + 1 < nstage) stage(I1{}, st + 1, w1, w0);
    // the tail prefetches have landed and every wave is done reading the
    // ring before the next item refills it
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    lds_barrier();

}

template <int MODE>
__global__ void __launch_bounds__(256, 1) expert_gemm_tiled_kernel(GemmArgs a) {
    __shared__ float red[4][kTileRows];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, r = lane & 31;

    const int K = (MODE == kGemm2) ? a.I : a.H;
    const int wrows = (MODE == kGemm2) ? a.H : 2 * a.I;
    const int NB = (MODE == kGemm2) ? (a.H + 255) / 256 : a.I / 128;
    const int nstage = K / kStageK;

    const int ntiles = a.tile_start[a.E];
    const int total = ntiles * NB;
    const int xcd = blockIdx.x & 7, per_xcd = gridDim.x >> 3;
    const int beg = (int)(((long long)total * xcd) >> 3);
    const int end = (int)(((long long)total * (xcd + 1)) >> 3);

    for (int item = beg + (int)(blockIdx.x >> 3); item < end; item += per_xcd) {
        // items of expert e: [NB * tile_start[e], NB * tile_start[e+1]).  Its
        // m-tiles go in chunks of kMChunk; within a chunk the order is n-block
        // major, m-tile minor, so the m-tiles that share a block of weight rows
        // run together, while a chunk's activations stay in L2 across n-blocks.
        const int e = a.tile_info[item / NB].x;
        const int t0 = a.tile_start[e], nt = a.tile_start[e + 1] - t0;
        const int local = item - NB * t0;
        const int full = nt / kMChunk;                              // full chunks
        const int chunk = min(local / (kMChunk * NB), full);
        const int cs = (chunk < full) ? kMChunk : nt - kMChunk * full;  // tiles in this chunk
        const int within = local - kMChunk * NB * chunk;
        const int nblk = within / cs;
        const int4 ti = a.tile_info[t0 + kMChunk * chunk + (within - nblk * cs)];
        const int row0 = ti.y, nrows = ti.z;

        // weight rows of this wave: two 32-row tiles
        int wrow0, wrow1;
        bool wave_valid = true;
        if constexpr (MODE == kGemm2) {
            wrow0 = nblk * 256 + wave * 64;
            wrow1 = wrow0 + 32;
            wave_valid = wrow0 < a.H;
            if (!wave_valid) { wrow0 = 0; wrow1 = 32; }   // loads stay in bounds; results dropped
        } else {
            wrow0 = nblk * 128 + wave * 32;    // gate
            wrow1 = a.I + wrow0;               // up
        }
        const size_t wstride = (size_t)K / 2, sstride = (size_t)K / 32;
        const uint8_t* wp0 = a.w + ((size_t)e * wrows + wrow0 + r) * wstride + 64 * g;
        const uint8_t* wp1 = a.w + ((size_t)e * wrows + wrow1 + r) * wstride + 64 * g;
        const uint8_t* sp0 = a.w_scale + ((size_t)e * wrows + wrow0 + r) * sstride + 4 * g;
        const uint8_t* sp1 = a.w_scale + ((size_t)e * wrows + wrow1 + r) * sstride + 4 * g;

        TileCtx c;
        c.act = a.act; c.act_scale = a.act_scale;
        c.wp0 = wp0; c.wp1 = wp1; c.sp0 = sp0; c.sp1 = sp1;
        c.K = K; c.nstage = nstage; c.row0 = row0; c.nrows = nrows;
        v16f acc[4][2];
        tile_kloop(c, acc, tl_act0, tl_act1, tl_act2, tl_scl0, tl_scl1, tl_scl2);

        // ---- epilogues: lane holds tokens 32j + r, features 8*(i/4) + 4g + (i%4) of each tile ----
        if constexpr (MODE == kGemm2) {
            if (wave_valid) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int rr = 32 * j + r;
                    if (rr >= nrows) continue;
                    float* o = (float*)a.out + (size_t)(row0 + rr) * a.H;
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const int n = (t == 0 ? wrow0 : wrow1) + 4 * g;
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            *(v4f*)(o + n + 8 * q) = v4f{acc[j][t][4 * q], acc[j][t][4 * q + 1],
                                                         acc[j][t][4 * q + 2], acc[j][t][4 * q + 3]};
                    }
                }
            }
        } else if constexpr (MODE == kGemm1Preact) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int rr = 32 * j + r;
                if (rr >= nrows) continue;
                float* o = (float*)a.out + (size_t)(row0 + rr) * (2 * a.I);
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int n = (t == 0 ? wrow0 : wrow1) + 4 * g;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *(v4f*)(o + n + 8 * q) = v4f{acc[j][t][4 * q], acc[j][t][4 * q + 1],
                                                     acc[j][t][4 * q + 2], acc[j][t][4 * q + 3]};
                }
            }
        } else {
            // SwiGLU, then FP8 over the workgroup's 128 features per row
            float amax[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float m = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float gv = acc[j][0][i];
                    const float h = gv / (1.0f + __expf(-gv)) * acc[j][1][i];
                    acc[j][0][i] = h;
                    m = fmaxf(m, fabsf(h));
                }
                m = fmaxf(m, __shfl_xor(m, 32, 64));
                amax[j] = m;
            }
            if (g == 0) {
#pragma unroll
                for (int j = 0; j < 4; ++j) red[wave][32 * j + r] = amax[j];
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int rr = 32 * j + r;
                const float m = fmaxf(fmaxf(red[0][rr], red[1][rr]), fmaxf(red[2][rr], red[3][rr]));
                const int ex = fp8_block_exponent(m);
                if (rr < nrows) {
                    uint8_t* q = (uint8_t*)a.out + (size_t)(row0 + rr) * a.I + wrow0 + 4 * g;
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq)
                        *(uint32_t*)(q + 8 * qq) = pack_fp8x4(__builtin_amdgcn_ldexpf(acc[j][0][4 * qq], -ex),
                                                              __builtin_amdgcn_ldexpf(acc[j][0][4 * qq + 1], -ex),
                                                              __builtin_amdgcn_ldexpf(acc[j][0][4 * qq + 2], -ex),
                                                              __builtin_amdgcn_ldexpf(acc[j][0][4 * qq + 3], -ex));
                    if (wave == 0 && g == 0)
                        a.out_scale[(size_t)(row0 + rr) * (a.I / kFp8Block) + nblk] = (uint8_t)(ex + 127);
                }
            }
            __syncthreads();   // red is reused by the next item
        }
    }
}

static int persistent_grid() {
    static int cached = 0;
    if (!cached) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cached = cus & ~7;   // one workgroup per CU, a multiple of the 8 XCDs
    }
    return cached;
}

bool tiled_gemm_supported(int H, int I) {
    return H % kStageK == 0 && I % kStageK == 0;
}

hipError_t launch_expert_gemm_tiled(GemmMode mode, const GemmArgs& a, hipStream_t stream) {
    dim3 grid(persistent_grid()), block(256);
    switch (mode) {
        case kGemm1Swiglu: hipLaunchKernelGGL((expert_gemm_tiled_kernel<kGemm1Swiglu>), grid, block, 0, stream, a); break;
        case kGemm1Preact: hipLaunchKernelGGL((expert_gemm_tiled_kernel<kGemm1Preact>), grid, block, 0, stream, a); break;
        case kGemm2: hipLaunchKernelGGL((expert_gemm_tiled_kernel<kGemm2>), grid, block, 0, stream, a); break;
    }
    return hipGetLastError();
}

}  // namespace moe
