// Grouped expert GEMMs for FP8 block-scaled experts (e4m3 weights, one
// float32 scale per 128 x 128 block; teardown "Why Are the V2.6 Files Half
// the Size of V2.5?", V2.5 column) on shapes with many rows per expert
// (prefill): LDS-tiled, on the 32x32x64 MFMA with e4m3 on both sides.
//
// As in the streaming variant (expert_gemm_fp8.hip), the scale operand of
// the MFMA only takes powers of two, so each 128-deep K block is multiplied
// with unit scales into a fresh accumulator (two 64-deep MFMAs) and added to
// the running sum times the product of its weight block scale and the
// token's activation scale.
//
// Operand layout of the 32x32x64 instruction for e4m3 (lane l, g = l/32,
// r = l%32): bytes 0..15 -> k = 16g + i, bytes 16..31 -> k = 32 + 16g + i;
// the result lane holds acc[i] = D[8(i/4) + 4g + (i%4)][r].  A = 32 weight
// rows, B = 32 tokens.  K runs in natural order: step s of a 256-deep stage
// covers k = 64s .. 64s + 63, so steps 0-1 and 2-3 are the stage's two
// 128-deep scale blocks.
//
// Work decomposition: an item is (m-tile of 128 tokens of one expert, 256
// weight rows): 128 features of the gate/up GEMM (their gate and up rows,
// one 128-channel block of h) or 256 output features of the down GEMM.  A
// workgroup has 8 waves, two per SIMD; each wave owns one 32-row weight tile
// (gate/up: 16 gate rows and the 16 matching up rows) and multiplies it with
// the 4 token tiles of the m-tile.
//
// Pipeline: activations of a stage (128 rows x 256 bytes, plus the rows'
// two float32 scales) go global -> registers -> LDS into one of two buffers;
// the global loads of stage st+1 are in flight while stage st is multiplied,
// and each wave's weight codes for stage st+1 (32 rows x 256 bytes, straight
// into registers) as well.  One barrier per stage.  The 16-byte chunk c of
// activation row p sits at chunk slot c ^ (p mod 16), so the 32 rows of one
// operand fetch hit distinct banks.  Weight block scales are wave-uniform and
// come through the scalar cache.
//
// The grid is persistent (one workgroup per CU); workgroups on one XCD take a
// contiguous 1/8 of the items, which go expert by expert in chunks of four
// m-tiles, n-block major within a chunk, so the m-tiles that read one block
// of weight rows run side by side on one L2.
#include "moe_internal.h"

namespace moe {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kF8TileRows = 128;               // tokens per m-tile
constexpr int kF8StageK = 256;                 // K (bytes of an e4m3 row) per stage
constexpr int kF8Waves = 8;
constexpr int kF8ItemRows = 32 * kF8Waves;     // weight rows per item
constexpr int kF8MChunk = 4;                   // m-tiles of one expert scheduled together
constexpr int kF8TT = kF8TileRows / 32;        // token tiles per m-tile
constexpr int kF8ActLoads = kF8TileRows * kF8StageK / 16 / (64 * kF8Waves);   // 16-byte loads per lane per stage
constexpr int kF8MaxKB = kF8TiledMaxK / 128;    // 128-deep K blocks the LDS weight-scale copy holds

// One LDS block, scales first: every operand read of the K loop then sits
// below 64 KB, in reach of the 16-bit immediate offset of a DS instruction
// (one base register per lane instead of one per operand).
struct F8Lds {
    float xsc[2][kF8TileRows * 2];                 // activation scales of the two stage buffers
    uint8_t act[2][kF8TileRows * kF8StageK];       // the two activation stage buffers
    float red[kF8Waves * kF8TileRows];             // per-row maxima of the SwiGLU epilogue
    float wsc[kF8Waves][2][kF8MaxKB];              // each wave's weight block scales for the item (gate, up)
};
__shared__ __attribute__((aligned(16))) F8Lds f8_lds;

__device__ __forceinline__ int f8_swz(int row, int chunk) { return row * kF8StageK + ((chunk ^ (row & 15)) << 4); }

typedef int v4i __attribute__((ext_vector_type(4)));
// two 16-byte halves -> one 32-byte MFMA operand (a concatenation the
// register allocator can satisfy by placing the halves side by side)
__device__ __forceinline__ v8i cat8(v4i lo, v4i hi) { return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7); }

__device__ __forceinline__ v16f mfma32_f8f8(v8i a, v8i b, v16f c) {
    // format 0 = e4m3 for both operands; scale byte 127 = 2^0
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

struct F8Item {
    int e, row0, nrows, nblk;
};

// read-only data that every lane of a wave reads alike (constant address space)
typedef const __attribute__((address_space(4))) int* cint_p;
__device__ __forceinline__ int4 load_uniform4(const int4* p) {
    const cint_p q = (cint_p)p;
    return make_int4(q[0], q[1], q[2], q[3]);
}

__device__ __forceinline__ F8Item f8_item_at(const GemmArgs& a, int item, int NB) {
    // items of expert e: [NB * t0, NB * (t0 + nt)) with t0 its first tile in
    // the plan and nt = ceil(n_e / 128) its tiles; its m-tiles in chunks of
    // kF8MChunk, n-block major, m-tile minor within a chunk
    // (the plan and the offsets are read-only here and alike in every lane:
    // scalar loads, which do not queue behind the wave's vector loads)
    const cint_p offs = (cint_p)a.offsets;
    const int4 head = load_uniform4(a.tile_info + item / NB);
    const int e = head.x, t0 = head.w;
    const int nt = (offs[e + 1] - offs[e] + kF8TileRows - 1) / kF8TileRows;
    const int local = item - NB * t0;
    const int full = nt / kF8MChunk;
    const int chunk = min(local / (kF8MChunk * NB), full);
    const int cs = (chunk < full) ? kF8MChunk : nt - kF8MChunk * full;
    const int within = local - kF8MChunk * NB * chunk;
    const int nblk = within / cs;
    const int4 ti = load_uniform4(a.tile_info + t0 + kF8MChunk * chunk + (within - nblk * cs));
    return F8Item{e, ti.y, ti.z, nblk};
}

}  // namespace

template <int MODE, bool PACKED, bool GATHER>
__global__ void __launch_bounds__(64 * kF8Waves, 1) expert_gemm_fp8_tiled_kernel(GemmArgs a) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, r = lane & 31;

    const int K = (MODE == kGemm2) ? a.I : a.H;
    const int wrows = (MODE == kGemm2) ? a.H : 2 * a.I;
    const int KB = K / kFp8Block;
    const int NB = (MODE == kGemm2) ? a.H / kF8ItemRows : a.I / (kF8ItemRows / 2);
    const int nstage = K / kF8StageK;

    const int ntiles = a.tile_start[a.E];
    const int total = ntiles * NB;
    const int xcd = blockIdx.x & 7, per_xcd = gridDim.x >> 3;
    const int end = (int)(((long long)total * (xcd + 1)) >> 3);
    int item = (int)(((long long)total * xcd) >> 3) + (int)(blockIdx.x >> 3);

    // ---- per-lane geometry ----
    // weight row of this lane within the item's 256 rows (gate/up: 16 gate
    // rows of features 16w..16w+15, then their up rows; down: 32 rows)
    const int lrow_in = (MODE == kGemm2) ? 32 * wave + r : 16 * wave + (r & 15);   // feature / row offset in the item
    // activation stage loads: thread tid moves chunks q = tid + 512 p (row q/16, chunk q%16)
    int srow[kF8ActLoads], schunk[kF8ActLoads];
#pragma unroll
    for (int p = 0; p < kF8ActLoads; ++p) {
        const int q = tid + 64 * kF8Waves * p;
        srow[p] = q >> 4;
        schunk[p] = q & 15;
    }
    // LDS operand reads: byte offset of row r, and of the swizzled chunk slots
    // 8b + 2m + g (m = 0..3: steps 2b and 2b+1, bytes 0..15 and 16..31)
    const int lane_row = r * kF8StageK;
    int slot[2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int m = 0; m < 4; ++m) slot[b][m] = ((8 * b + 2 * m + g) ^ (r & 15)) << 4;
    // scale loads: threads 0..255 copy float (row tid/2, block tid%2) of the stage
    const int xs_row = (tid >> 1) & (kF8TileRows - 1), xs_blk = tid & 1;
    const float* wsc = (const float*)a.w_scale;
    const float* asc = (const float*)a.act_scale;

    for (; item < end; item += per_xcd) {
        const F8Item it = f8_item_at(a, item, NB);
        const int row0 = it.row0, nrows = it.nrows;
        // activation rows of this thread's stage loads and scale copy
        uint32_t aoff[kF8ActLoads];   // byte offset of the thread's chunk in its activation row (< 2 GiB)
#pragma unroll
        for (int p = 0; p < kF8ActLoads; ++p) {
            const int rr = row0 + min(srow[p], nrows - 1);
            const int arow = GATHER ? a.act_rows[rr] : rr;
            aoff[p] = (uint32_t)arow * (uint32_t)K + 16 * schunk[p];
        }
        int xrow = row0 + min(xs_row, nrows - 1);
        if (GATHER) xrow = a.act_rows[xrow];

        // weight rows: gate/up lanes r < 16 read gate feature f, r >= 16 its up row
        const size_t ebase = (size_t)it.e * wrows;
        size_t wrow;
        if constexpr (MODE == kGemm2) wrow = ebase + (size_t)it.nblk * kF8ItemRows + lrow_in;
        else wrow = ebase + (r < 16 ? 0 : a.I) + (size_t)it.nblk * (kF8ItemRows / 2) + lrow_in;
        // packed: 16-row group, 2 KB block per 128 columns, lane bytes of
        // piece p of row r' at (16 p + r') * 16; canonical: row-major
        const uint8_t* wl = PACKED ? a.w + (wrow - (wrow & 15)) * K + 256 * g + 16 * (wrow & 15)
                                   : a.w + wrow * K + 16 * g;
        // wave-uniform weight block scale rows (per 128-deep K block)
        const float* sw0;
        const float* sw1;
        if constexpr (MODE == kGemm2) {
            sw0 = wsc + ((size_t)it.e * (wrows / kFp8Block) + (it.nblk * kF8ItemRows + 32 * wave) / kFp8Block) * KB;
            sw1 = sw0;
        } else {
            sw0 = wsc + ((size_t)it.e * (wrows / kFp8Block) + it.nblk) * KB;                       // gate rows
            sw1 = wsc + ((size_t)it.e * (wrows / kFp8Block) + a.I / kFp8Block + it.nblk) * KB;   // up rows
        }

        // weight codes of the current stage [step][half]: the two steps of a
        // 128-deep block are refilled with the next stage's as soon as the
        // block's MFMAs are issued (past the last stage: the last stage again)
        v4i wreg[4][2];
        auto load_w = [&](int st, int blk) __attribute__((always_inline)) {
#pragma unroll
            for (int s = 2 * blk; s < 2 * blk + 2; ++s) {
                if constexpr (PACKED) {
                    const uint8_t* b = wl + (size_t)(2 * st + (s >> 1)) * 2048 + 1024 * (s & 1);
                    wreg[s][0] = *(const v4i*)b;
                    wreg[s][1] = *(const v4i*)(b + 512);
                } else {
                    const uint8_t* b = wl + st * kF8StageK + 64 * s;
                    wreg[s][0] = *(const v4i*)b;
                    wreg[s][1] = *(const v4i*)(b + 32);
                }
            }
        };
        // this thread's share of an activation stage and of its scales
        v4i areg[kF8ActLoads];
        float xreg;
        auto load_act = [&](int st) __attribute__((always_inline)) {
#pragma unroll
            for (int p = 0; p < kF8ActLoads; ++p) {
                const uint8_t* base = a.act + st * kF8StageK;   // wave-uniform
                areg[p] = *(const v4i*)(base + aoff[p]);
            }
            xreg = asc[(size_t)xrow * KB + 2 * st + xs_blk];
        };
        auto store_act = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
            for (int p = 0; p < kF8ActLoads; ++p) *(v4i*)(&f8_lds.act[buf][f8_swz(srow[p], schunk[p])]) = areg[p];
            // threads tid and tid + 256 hold the same scale: a duplicate store of one
            // value keeps the stage free of branches
            f8_lds.xsc[buf][tid & (2 * kF8TileRows - 1)] = xreg;
        };

        v16f acc[kF8TT];
#pragma unroll
        for (int j = 0; j < kF8TT; ++j)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[j][i] = 0.0f;

        // One stage: for each of its two 128-deep blocks b and token tiles j,
        // two MFMAs into a fresh partial, then acc += partial * (weight scale x
        // token scale).  Two partials alternate between the token tiles: the
        // MFMAs of tile j run on the matrix core while the vector ALU scales
        // and adds the partial of tile j - 1 (half of it after each MFMA).  The
        // LDS operands of the next (block, tile) pair are read while the
        // current pair is multiplied, so their latency is not waited out before
        // each MFMA.  The scheduling barriers fix that order and keep the
        // compiler from hoisting every LDS read (which costs registers the
        // weights need).
        auto compute = [&](int st, int buf) __attribute__((always_inline)) {
            const uint8_t* lds = f8_lds.act[buf];
            const float* xsl = f8_lds.xsc[buf];
            const int wnext = min(st + 1, nstage - 1);
            // steps 2b and 2b+1 of row 32j + r: chunks 4s + g and 4s + 2 + g
            // (the row's swizzle depends on r only: 32j adds a constant), and
            // the row's activation scale of block b
            v8i Bn0, Bn1;
            float sxn;
            auto read_ops = [&](int b, int j) __attribute__((always_inline)) {
                const uint8_t* rowp = lds + (32 * j) * kF8StageK + lane_row;
                Bn0 = cat8(*(const v4i*)(rowp + slot[b][0]), *(const v4i*)(rowp + slot[b][1]));
                Bn1 = cat8(*(const v4i*)(rowp + slot[b][2]), *(const v4i*)(rowp + slot[b][3]));
                sxn = xsl[2 * (32 * j + r) + b];
            };
            read_ops(0, 0);
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                // (from LDS: a global load here would make the in-order load
                // counter wait for the activation prefetch as well)
                const float wg = f8_lds.wsc[wave][0][2 * st + b], wu = f8_lds.wsc[wave][1][2 * st + b];
                const v8i A0 = cat8(wreg[2 * b][0], wreg[2 * b][1]);
                const v8i A1 = cat8(wreg[2 * b + 1][0], wreg[2 * b + 1][1]);
                v16f part[2];
                float cg[2], cu[2];
                // elements 8h .. 8h + 7 of tile j's partial (h = 0: gate rows, 1: up rows)
                auto rescale = [&](int j, int h) __attribute__((always_inline)) {
#pragma unroll
                    for (int i = 8 * h; i < 8 * h + 8; ++i)
                        acc[j][i] = __builtin_fmaf(part[j & 1][i], h == 0 ? cg[j & 1] : cu[j & 1], acc[j][i]);
                };
#pragma unroll
                for (int j = 0; j < kF8TT; ++j) {
                    // The older wave of a SIMD would otherwise take every MFMA
                    // issue slot until it stalls; a priority that falls through
                    // the stage lets the wave that is behind issue first, which
                    // keeps the two waves of a SIMD apart
                    switch ((kF8TT * b + j) >> 1) {
                        case 0: __builtin_amdgcn_s_setprio(3); break;
                        case 1: __builtin_amdgcn_s_setprio(2); break;
                        case 2: __builtin_amdgcn_s_setprio(1); break;
                        default: __builtin_amdgcn_s_setprio(0); break;
                    }
                    const v8i B0 = Bn0, B1 = Bn1;
                    const float sx = sxn;
                    part[j & 1] = mfma32_f8f8(A0, B0, v16f{});
                    __builtin_amdgcn_sched_barrier(0);
                    if (j + 1 < kF8TT) read_ops(b, j + 1);
                    else if (b == 0) read_ops(1, 0);
                    if (j > 0) rescale(j - 1, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    part[j & 1] = mfma32_f8f8(A1, B1, part[j & 1]);
                    __builtin_amdgcn_sched_barrier(0);
                    if (j > 0) rescale(j - 1, 1);
                    cg[j & 1] = wg * sx;
                    cu[j & 1] = wu * sx;
                    if (j == kF8TT - 1) load_w(wnext, b);   // block b's weights are no longer needed
                    __builtin_amdgcn_sched_barrier(0);
                }
                rescale(kF8TT - 1, 0);
                rescale(kF8TT - 1, 1);
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        // ---- pipeline over the item's stages: weights one stage ahead in
        // registers, activations one stage ahead in registers, two LDS buffers ----
        load_w(0, 0);
        load_w(0, 1);
        load_act(0);
        // the wave's weight block scales for the whole item (lanes past KB repeat the last)
        const float sg = sw0[min(lane, KB - 1)], su = sw1[min(lane, KB - 1)];
        __syncthreads();                       // every wave is done with the previous item's LDS
        f8_lds.wsc[wave][0][min(lane, KB - 1)] = sg;
        f8_lds.wsc[wave][1][min(lane, KB - 1)] = su;
        store_act(0);
        load_act(min(1, nstage - 1));
        __syncthreads();
        // The loop body has no branches: a branch would let the compiler sink
        // the MFMAs below the barrier and keep every LDS operand live.  Past
        // the last stage the loads repeat the last stage and the store fills the
        // idle buffer, which nobody reads.
        for (int st = 0; st < nstage; st += 2) {   // nstage is even (K % 512 == 0)
            compute(st, 0);
            store_act(1);                      // stage st + 1 into the other buffer
            __syncthreads();
            load_act(min(st + 2, nstage - 1));
            compute(st + 1, 1);
            store_act(0);
            __syncthreads();
            load_act(min(st + 3, nstage - 1));
        }

        // ---- epilogues: lane holds tokens 32j + r and tile rows 8(i/4) + 4g + (i%4) ----
        if constexpr (MODE == kGemm2) {
#pragma unroll
            for (int j = 0; j < kF8TT; ++j) {
                const int rr = 32 * j + r;
                if (rr < nrows) {
                    float* o = (float*)a.out + (size_t)(row0 + rr) * a.H + it.nblk * kF8ItemRows + 32 * wave + 4 * g;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *(v4f*)(o + 8 * q) = v4f{acc[j][4 * q], acc[j][4 * q + 1], acc[j][4 * q + 2], acc[j][4 * q + 3]};
                }
            }
        } else if constexpr (MODE == kGemm1Preact) {
#pragma unroll
            for (int j = 0; j < kF8TT; ++j) {
                const int rr = 32 * j + r;
                if (rr < nrows) {
                    float* o = (float*)a.out + (size_t)(row0 + rr) * (2 * a.I);
                    const int f = it.nblk * (kF8ItemRows / 2) + 16 * wave;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int n = (q < 2 ? f : a.I + f) + 8 * (q & 1) + 4 * g;
                        *(v4f*)(o + n) = v4f{acc[j][4 * q], acc[j][4 * q + 1], acc[j][4 * q + 2], acc[j][4 * q + 3]};
                    }
                }
            }
        } else {
            // SwiGLU on matching gate (element i) and up (element i + 8) values,
            // then FP8 with a float32 scale over the item's 128 features
            float amax[kF8TT];
#pragma unroll
            for (int j = 0; j < kF8TT; ++j) {
                float m = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float gv = acc[j][i];
                    const float h = silu_f32(gv) * acc[j][i + 8];
                    acc[j][i] = h;
                    m = fmaxf(m, fabsf(h));
                }
                amax[j] = fmaxf(m, __shfl_xor(m, 32, 64));
            }
            if (g == 0) {
#pragma unroll
                for (int j = 0; j < kF8TT; ++j) f8_lds.red[wave * kF8TileRows + 32 * j + r] = amax[j];
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < kF8TT; ++j) {
                const int rr = 32 * j + r;
                float m = f8_lds.red[rr];
#pragma unroll
                for (int w = 1; w < kF8Waves; ++w) m = fmaxf(m, f8_lds.red[w * kF8TileRows + rr]);
                const float sc = fp8_f32_scale(m);
                const float d = m > 0.0f ? sc : 1.0f;
                if (rr < nrows) {
                    // features 16 wave + 4g + (0..3) and 16 wave + 8 + 4g + (0..3)
                    uint8_t* q = (uint8_t*)a.out + (size_t)(row0 + rr) * a.I + it.nblk * (kF8ItemRows / 2) + 16 * wave + 4 * g;
                    *(uint32_t*)q = pack_fp8x4(fp8_f32_quotient(acc[j][0], d), fp8_f32_quotient(acc[j][1], d),
                                               fp8_f32_quotient(acc[j][2], d), fp8_f32_quotient(acc[j][3], d));
                    *(uint32_t*)(q + 8) = pack_fp8x4(fp8_f32_quotient(acc[j][4], d), fp8_f32_quotient(acc[j][5], d),
                                                     fp8_f32_quotient(acc[j][6], d), fp8_f32_quotient(acc[j][7], d));
                    if (wave == 0 && g == 0) ((float*)a.out_scale)[(size_t)(row0 + rr) * (a.I / kFp8Block) + it.nblk] = sc;
                }
            }
        }
    }
}


static int f8_persistent_grid() {
    static int cached = 0;
    if (!cached) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cached = cus & ~7;   // one workgroup per CU, a multiple of the 8 XCDs
    }
    return cached;
}

template <int MODE, bool PACKED, bool GATHER>
static void launch_f8_tiled(const GemmArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((expert_gemm_fp8_tiled_kernel<MODE, PACKED, GATHER>), dim3(f8_persistent_grid()),
                       dim3(64 * kF8Waves), 0, stream, a);
}

template <int MODE>
static void launch_f8_tiled_mode(const GemmArgs& a, hipStream_t stream) {
    constexpr bool kCanGather = MODE != kGemm2;   // the down GEMM reads h in expert order
    if (kCanGather && a.act_rows) {
        if (a.packed) launch_f8_tiled<MODE, true, kCanGather>(a, stream);
        else launch_f8_tiled<MODE, false, kCanGather>(a, stream);
    } else {
        if (a.packed) launch_f8_tiled<MODE, true, false>(a, stream);
        else launch_f8_tiled<MODE, false, false>(a, stream);
    }
}

hipError_t launch_expert_gemm_fp8_tiled(GemmMode mode, const GemmArgs& a, hipStream_t stream) {
    switch (mode) {
        case kGemm1Swiglu: launch_f8_tiled_mode<kGemm1Swiglu>(a, stream); break;
        case kGemm1Preact: launch_f8_tiled_mode<kGemm1Preact>(a, stream); break;
        case kGemm2: launch_f8_tiled_mode<kGemm2>(a, stream); break;
    }
    return hipGetLastError();
}

}  // namespace moe
