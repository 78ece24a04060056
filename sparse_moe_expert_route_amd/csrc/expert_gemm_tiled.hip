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
// (block id mod 8) take a contiguous 1/8 of the item list, n-block fastest,
// so items sharing an m-tile (activations) or an expert (weights) run
// together on the same L2.
#include "moe_internal.h"

namespace moe {

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kTileRows = 128;            // m-tile rows
constexpr int kStageK = 256;              // K per LDS stage (bytes of an FP8 row)

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

struct WStage {
    uint4 w[2][4];    // 2 weight tiles x 4 steps of 16 bytes
    uint32_t ws[2];   // 4 scale bytes per tile
};

template <int MODE>
__global__ void __launch_bounds__(256, 1) expert_gemm_tiled_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t act_lds[2][kTileRows * kStageK];
    __shared__ __attribute__((aligned(16))) uint32_t act_scale_lds[2][kTileRows];   // 2 scale bytes per row
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
        const int tile = item / NB, nblk = item - tile * NB;
        const int4 ti = a.tile_info[tile];
        const int e = ti.x, row0 = ti.y, nrows = ti.z;

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
        // swizzle maps there.  Waves 0 and 1 also move the rows' two scale bytes.
        auto dma_act = [&](int st, int buf) {
            const int k0 = st * kStageK;
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const int row = 32 * wave + 4 * p + (lane >> 4);
                const int chunk = (lane & 15) ^ (row & 15);
                const int rr = row0 + min(row, nrows - 1);
                dma16(a.act + (size_t)rr * K + k0 + 16 * chunk, &act_lds[buf][(32 * wave + 4 * p) * kStageK]);
            }
            if (wave < 2) {
                const int rr = row0 + min(64 * wave + lane, nrows - 1);
                dma2(a.act_scale + (size_t)rr * (K / kFp8Block) + k0 / kFp8Block, &act_scale_lds[buf][64 * wave]);
            }
        };

        v16f acc[4][2];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[j][t][i] = 0.0f;

        WStage wcur, wnext;
        dma_act(0, 0);
        load_w(wcur, 0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        for (int st = 0; st < nstage; ++st) {
            const int buf = st & 1;
            const bool more = st + 1 < nstage;
            // operands of this stage from LDS first, so the next stage's LDS writes
            // are issued after every read of this buffer pair
            const uint8_t* lds = act_lds[buf];
            v8i B[4][4];
            int bs[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 32 * j + r;
                bs[j] = (act_scale_lds[buf][row] >> (8 * g)) & 0xFF;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const uint4 lo4 = *(const uint4*)(lds + swz(row, 2 * s + g));
                    const uint4 hi4 = *(const uint4*)(lds + swz(row, 8 + 2 * s + g));
                    B[j][s][0] = lo4.x; B[j][s][1] = lo4.y; B[j][s][2] = lo4.z; B[j][s][3] = lo4.w;
                    B[j][s][4] = hi4.x; B[j][s][5] = hi4.y; B[j][s][6] = hi4.z; B[j][s][7] = hi4.w;
                }
            }
            if (more) {
                dma_act(st + 1, buf ^ 1);
                load_w(wnext, st + 1);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                v8i A0, A1;
                A0[0] = wcur.w[0][s].x; A0[1] = wcur.w[0][s].y; A0[2] = wcur.w[0][s].z; A0[3] = wcur.w[0][s].w;
                A1[0] = wcur.w[1][s].x; A1[1] = wcur.w[1][s].y; A1[2] = wcur.w[1][s].z; A1[3] = wcur.w[1][s].w;
                A0[4] = A0[5] = A0[6] = A0[7] = 0;
                A1[4] = A1[5] = A1[6] = A1[7] = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    switch (s) {
                        case 0:
                            acc[j][0] = mfma32_w4a8<0>(A0, B[j][s], acc[j][0], (int)wcur.ws[0], bs[j]);
                            acc[j][1] = mfma32_w4a8<0>(A1, B[j][s], acc[j][1], (int)wcur.ws[1], bs[j]);
                            break;
                        case 1:
                            acc[j][0] = mfma32_w4a8<1>(A0, B[j][s], acc[j][0], (int)wcur.ws[0], bs[j]);
                            acc[j][1] = mfma32_w4a8<1>(A1, B[j][s], acc[j][1], (int)wcur.ws[1], bs[j]);
                            break;
                        case 2:
                            acc[j][0] = mfma32_w4a8<2>(A0, B[j][s], acc[j][0], (int)wcur.ws[0], bs[j]);
                            acc[j][1] = mfma32_w4a8<2>(A1, B[j][s], acc[j][1], (int)wcur.ws[1], bs[j]);
                            break;
                        default:
                            acc[j][0] = mfma32_w4a8<3>(A0, B[j][s], acc[j][0], (int)wcur.ws[0], bs[j]);
                            acc[j][1] = mfma32_w4a8<3>(A1, B[j][s], acc[j][1], (int)wcur.ws[1], bs[j]);
                            break;
                    }
                }
            }
            if (more) wcur = wnext;
            __builtin_amdgcn_s_waitcnt(0);   // this wave's LDS writes for the next stage have landed
            __syncthreads();
        }

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
