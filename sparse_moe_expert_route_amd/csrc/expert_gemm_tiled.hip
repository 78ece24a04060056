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
// contiguous bytes of its row and its 4 weight scales one dword (op_sel = s).
//
// Work decomposition: an item is (m-tile of 128 rows of one expert, n-block).
// A workgroup of 8 waves (two per SIMD) computes 128 rows x (128 h-features =
// 256 W13 rows) for the gate/up GEMM, or 128 rows x 256 output features for
// the down GEMM; each wave owns one 32-row weight tile and all 128 rows.
// The activation tile is staged through LDS by direct global->LDS loads
// (global_load_lds_dwordx4: no staging registers) in a three-buffer ring, with
// the 16-byte chunk c of row p stored at chunk slot c ^ (p mod 16) so that the
// 32 rows read by one MFMA operand fetch hit distinct banks; every wave
// streams its own weight rows straight into registers.  The item's weight and
// activation scales are copied to LDS once, at its start.
//
// Weight layouts: canonical (row-major codes) or the 16-row packed layout
// written by moe_prepack_weights, in which one load instruction of a wave
// covers whole 128-byte lines (a third of the address-unit time of the
// row-strided canonical loads).
//
// The grid is persistent: workgroups on one XCD (block id mod 8) take a
// contiguous 1/8 of the item list.  Items are grouped by expert; an expert's
// m-tiles go in chunks of four, each chunk ordered n-block major, m-tile
// minor: the m-tiles that read the same block of weight rows run side by
// side on one L2 (weights come from HBM about once per chunk), and the
// chunk's activations stay in L2 across its n-blocks.
#include "moe_internal.h"

#include <type_traits>

namespace moe {

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kTileRows = 128;            // m-tile rows
constexpr int kStageK = 256;              // K per LDS stage (bytes of an FP8 row)
constexpr int kMChunk = 4;                // m-tiles of one expert scheduled together
constexpr int kWaves = 8;                 // waves per workgroup, two per SIMD
constexpr int kMaxK = 6144;               // largest K the LDS scale copies hold

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane, global -> LDS at lds_base + 16 * lane (lds_base wave-uniform)
__device__ __forceinline__ void dma16(const void* g, void* lds_base) {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_base, 16, 0, 0);
}
// 4 bytes per lane, global -> LDS at lds_base + 4 * lane
__device__ __forceinline__ void dma4(const void* g, void* lds_base) {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_base, 4, 0, 0);
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
// the item's weight scales: 256 rows x K/32 bytes, the 16-byte chunks of row
// R rotated by R (chunk c at slot (c + R) mod K/512), so that the 32 rows of
// a wave read different banks
__shared__ __attribute__((aligned(16))) uint8_t tl_wsc[256 * (kMaxK / 32)];
// the item's activation scales: 128 rows x K/128 bytes, row-major
__shared__ __attribute__((aligned(16))) uint8_t tl_xsc[kTileRows * (kMaxK / 128)];

// s_waitcnt immediate: at most n vector-memory operations outstanding (gfx9
// encoding, vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt at their maxima)
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// vector-memory operations one stage issues per wave: 4 activation pieces and
// 4 weight loads
constexpr int kStageLoads = 8;

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
    uint4 w[4];     // the wave's 32-row weight tile, 4 steps of 16 bytes
};

// Per-item state of the stage loop.
struct TileCtx {
    const uint8_t* act;        // FP8 activations [N][K]
    const uint8_t* act_scale;  // [N][K/128]
    const int32_t* act_rows;   // activation row of each expert-ordered row, or null (identity)
    const uint8_t* wp;         // this lane's weight bytes at k = 0
    const uint8_t* wscale;     // the expert's weight scales [rows][K/32]
    int wstage, wstep;         // byte strides of wp per stage and per step
    int K, nstage, row0, nrows;
    int nblk, I, H;
};

// The K loop of one item.  The LDS buffers come in as restrict pointers: the
// compiler then tags every LDS access with the buffer it touches, and its
// wait tracking for direct global->LDS loads (which would otherwise make each
// LDS read wait for every such load in flight) lets a buffer be read while
// the others are being filled.
template <int MODE, int PF_STEP>
__device__ __forceinline__ void tile_kloop(const TileCtx& c, v16f (&acc)[4],
                                           uint8_t* __restrict__ act0, uint8_t* __restrict__ act1,
                                           uint8_t* __restrict__ act2, uint8_t* __restrict__ wsc,
                                           uint8_t* __restrict__ xsc) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, r = lane & 31;
    const int K = c.K, nstage = c.nstage, row0 = c.row0, nrows = c.nrows;
    const uint8_t* wp = c.wp;
    const int SB = K / 32, n16 = K / 512, XB = K / kFp8Block;
    auto abuf = [&](auto bc) -> uint8_t* {
        constexpr int B = decltype(bc)::value;
        if constexpr (B == 0) return act0; else if constexpr (B == 1) return act1; else return act2;
    };

    // ---- the item's scales into LDS (waited for with the first stage) ----
    // weight scales: 256 rows of n16 16-byte chunks, 64 chunks per load
    for (int m = wave; m < 4 * n16; m += kWaves) {
        const int i = 64 * m + lane, R = i / n16, slot = i - R * n16;
        const int ch = (slot + n16 - R % n16) % n16;    // the chunk stored at this slot
        int grow;                                       // the weight row of LDS row R
        if constexpr (MODE == kGemm2) {
            grow = min(c.nblk * 256 + R, c.H - 1);
        } else {
            const int w = R >> 5, rr = R & 31;
            grow = (rr < 16 ? 0 : c.I - 16) + c.nblk * 128 + 16 * w + rr;
        }
        dma16(c.wscale + (size_t)grow * SB + 16 * ch, wsc + 1024 * m);
    }
    // activation scales: 128 rows x XB bytes, 64 dwords per load
    for (int m = wave; m < XB / 2; m += kWaves) {
        const int i = 64 * m + lane, row = i / (XB / 4), col = i - row * (XB / 4);
        int srow = row0 + min(row, nrows - 1);
        if (c.act_rows) srow = c.act_rows[srow];
        dma4(c.act_scale + (size_t)srow * XB + 4 * col, xsc + 256 * m);
    }
    const int R = 32 * wave + r;                        // this lane's LDS weight-scale row
    const int rmod = R % n16;

    // the wave's weight tile for stage st: 16 bytes per lane per step
    auto load_w = [&](WStage& ws, int st) {
#pragma unroll
        for (int s = 0; s < 4; ++s) ws.w[s] = *(const uint4*)(wp + st * c.wstage + s * c.wstep);
    };

    // activation row of each of this lane's four stage pieces (fixed for the item)
    int arow[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        arow[p] = row0 + min(16 * wave + 4 * p + (lane >> 4), nrows - 1);
        if (c.act_rows) arow[p] = c.act_rows[arow[p]];
    }

    // activation stage: 128 rows x 256 bytes.  Wave w moves rows 16w .. 16w+15,
    // four rows (64 lanes x 16 bytes) per instruction; lane i of an instruction
    // fills chunk slot i%16 of row 4p + i/16 with the global chunk that the
    // swizzle maps there.
    auto dma_act = [&](auto bufc, int st) {
        uint8_t* lds = abuf(bufc);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int row = 16 * wave + 4 * p + (lane >> 4);
            const int chunk = (lane & 15) ^ (row & 15);
            dma16(c.act + (size_t)arow[p] * K + st * kStageK + 16 * chunk, lds + (16 * wave + 4 * p) * kStageK);
        }
    };

#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][i] = 0.0f;

    // Three-deep pipeline: stage st+2's activations (into LDS) and weights
    // (into a third register set) are issued while stage st is multiplied,
    // so each load has two stages of MFMA work to land.  Buffer and
    // register set of stage st are st mod 3; the stage loop is unrolled by
    // three so that every set is a fixed set of registers.  Two waves share
    // each SIMD and issue their prefetch at different steps (PF_STEP): while
    // one waits to issue its loads, the other's MFMAs run.
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
        const int sp = min(st + 2, nstage - 1);
        auto prefetch = [&]() {
            dma_act(std::integral_constant<int, NXT>{}, sp);
            load_w(wn, sp);
            __builtin_amdgcn_sched_barrier(0);
        };
        if constexpr (PF_STEP == 0) prefetch();
        const uint8_t* lds = abuf(setc);
        // scales of the stage: 4 weight-scale bytes of this lane's row
        // (byte s for step s), one activation-scale byte per row tile
        int slot = (st >> 1) + rmod;
        if (slot >= n16) slot -= n16;
        const int wsv = *(const int*)(wsc + R * SB + 16 * slot + 8 * (st & 1) + 4 * g);
        int bs[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) bs[j] = xsc[(32 * j + r) * XB + 2 * st + g];
        v8i B[4];
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
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s == PF_STEP && s > 0) prefetch();
            // B operands of one MFMA step (the other wave on the SIMD covers
            // the LDS latency)
            read_b(B, s);
            v8i A;
            A[0] = wc.w[s].x; A[1] = wc.w[s].y; A[2] = wc.w[s].z; A[3] = wc.w[s].w;
            A[4] = A[5] = A[6] = A[7] = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                switch (s) {
                    case 0: acc[j] = mfma32_w4a8<0>(A, B[j], acc[j], wsv, bs[j]); break;
                    case 1: acc[j] = mfma32_w4a8<1>(A, B[j], acc[j], wsv, bs[j]); break;
                    case 2: acc[j] = mfma32_w4a8<2>(A, B[j], acc[j], wsv, bs[j]); break;
                    default: acc[j] = mfma32_w4a8<3>(A, B[j], acc[j], wsv, bs[j]); break;
                }
            }
            // keep each step's LDS reads next to their use (hoisting them
            // all would need every B operand of the stage live)
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
    // ring and the scale copies before the next item refills them
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    lds_barrier();
}

template <int MODE, bool PACKED>
__global__ void __launch_bounds__(64 * kWaves, 1) expert_gemm_tiled_kernel(GemmArgs a) {
    __shared__ float red[kWaves][kTileRows];

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

        // weight rows of this wave: one 32-row tile.  Gate/up: rows 0..15 of
        // the tile are gate features f0 .. f0+15 and rows 16..31 the up rows
        // of the same features, so each lane ends up holding matching gate
        // and up values (accumulator elements i and i + 8).
        int wrow;
        bool wave_valid = true;
        const int f0 = nblk * 128 + 16 * wave;
        if constexpr (MODE == kGemm2) {
            const int n0 = nblk * 256 + 32 * wave;
            wave_valid = n0 < a.H;
            wrow = (wave_valid ? n0 : 0) + r;   // loads stay in bounds; results dropped
        } else {
            wrow = (r < 16) ? f0 + r : a.I + f0 + (r - 16);
        }
        TileCtx c;
        c.act = a.act; c.act_scale = a.act_scale; c.act_rows = a.act_rows;
        const size_t erow = (size_t)e * wrows + wrow;
        if constexpr (PACKED) {
            // 16-row group of the row, K/128 blocks of 1 KB: lane (g, r) takes
            // its 16 bytes of step s of stage st from block 2st + g, at
            // 16 * (16s + r mod 16)
            c.wp = a.w + (erow - (r & 15)) * ((size_t)K / 2) + 1024 * g + 16 * (r & 15);
            c.wstage = 2048; c.wstep = 256;
        } else {
            c.wp = a.w + erow * ((size_t)K / 2) + 64 * g;
            c.wstage = kStageK / 2; c.wstep = 16;
        }
        c.wscale = a.w_scale + (size_t)e * wrows * (K / 32);
        c.K = K; c.nstage = nstage; c.row0 = row0; c.nrows = nrows;
        c.nblk = nblk; c.I = a.I; c.H = a.H;
        v16f acc[4];
        // the two waves of a SIMD (w and w + 4) issue their prefetch half a
        // stage apart, so that one multiplies while the other waits on the
        // load queue
        if (wave < 4) tile_kloop<MODE, 0>(c, acc, tl_act0, tl_act1, tl_act2, tl_wsc, tl_xsc);
        else tile_kloop<MODE, 2>(c, acc, tl_act0, tl_act1, tl_act2, tl_wsc, tl_xsc);

        // ---- epilogues: lane holds tokens 32j + r and tile rows 8*(i/4) + 4g + (i%4) ----
        if constexpr (MODE == kGemm2) {
            if (wave_valid) {
                const int n0 = nblk * 256 + 32 * wave + 4 * g;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int rr = 32 * j + r;
                    if (rr >= nrows) continue;
                    float* o = (float*)a.out + (size_t)(row0 + rr) * a.H + n0;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *(v4f*)(o + 8 * q) = v4f{acc[j][4 * q], acc[j][4 * q + 1], acc[j][4 * q + 2], acc[j][4 * q + 3]};
                }
            }
        } else if constexpr (MODE == kGemm1Preact) {
            // tile row 8q + 4g + i: q = 0, 1 gate features f0 + 8q + 4g + i, q = 2, 3 up
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int rr = 32 * j + r;
                if (rr >= nrows) continue;
                float* o = (float*)a.out + (size_t)(row0 + rr) * (2 * a.I);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = (q < 2 ? f0 : a.I + f0) + 8 * (q & 1) + 4 * g;
                    *(v4f*)(o + n) = v4f{acc[j][4 * q], acc[j][4 * q + 1], acc[j][4 * q + 2], acc[j][4 * q + 3]};
                }
            }
        } else {
            // SwiGLU on matching gate (element i) and up (element i + 8) values,
            // then FP8 over the workgroup's 128 features of each row
            float amax[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float m = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float gv = acc[j][i];
                    const float h = gv / (1.0f + __expf(-gv)) * acc[j][i + 8];
                    acc[j][i] = h;
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
                float m = red[0][rr];
#pragma unroll
                for (int w = 1; w < kWaves; ++w) m = fmaxf(m, red[w][rr]);
                const int ex = fp8_block_exponent(m);
                if (rr < nrows) {
                    uint8_t* q = (uint8_t*)a.out + (size_t)(row0 + rr) * a.I + f0 + 4 * g;
#pragma unroll
                    for (int qq = 0; qq < 2; ++qq)
                        *(uint32_t*)(q + 8 * qq) = pack_fp8x4(__builtin_amdgcn_ldexpf(acc[j][4 * qq], -ex),
                                                              __builtin_amdgcn_ldexpf(acc[j][4 * qq + 1], -ex),
                                                              __builtin_amdgcn_ldexpf(acc[j][4 * qq + 2], -ex),
                                                              __builtin_amdgcn_ldexpf(acc[j][4 * qq + 3], -ex));
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
    return H % 512 == 0 && I % 512 == 0 && H <= kMaxK && I <= kMaxK;
}

template <int MODE>
static void launch_tiled_mode(const GemmArgs& a, hipStream_t stream) {
    dim3 grid(persistent_grid()), block(64 * kWaves);
    if (a.packed) hipLaunchKernelGGL((expert_gemm_tiled_kernel<MODE, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((expert_gemm_tiled_kernel<MODE, false>), grid, block, 0, stream, a);
}

hipError_t launch_expert_gemm_tiled(GemmMode mode, const GemmArgs& a, hipStream_t stream) {
    switch (mode) {
        case kGemm1Swiglu: launch_tiled_mode<kGemm1Swiglu>(a, stream); break;
        case kGemm1Preact: launch_tiled_mode<kGemm1Preact>(a, stream); break;
        case kGemm2: launch_tiled_mode<kGemm2>(a, stream); break;
    }
    return hipGetLastError();
}

}  // namespace moe
