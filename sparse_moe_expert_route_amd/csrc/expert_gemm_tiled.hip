// Grouped expert GEMMs for shapes with many rows per expert (prefill):
// LDS-tiled, on the 32x32x64 block-scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4), A = MXFP4 weights, B = FP8 activations
// (the other way round in the down GEMM of items of four or more stages).
//
// Same computation as the streaming kernel (expert_gemm.hip): experts are
// gate, up and down matrices with an intermediate width of 2,048 (teardown,
// "How Big Is Each Expert?"), stored as MXFP4 and computed in FP8 e4m3 (vLLM recipe,
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
// Work decomposition: an item is (m-tile of 128 rows of one expert, block of
// 512 weight rows): 256 features (gate and up rows) of the gate/up GEMM, or
// 512 output features of the down GEMM.  A workgroup has 8 waves, two per
// SIMD; each wave owns 2 weight tiles of 32 rows (in registers, loaded
// straight from memory) and multiplies them with the 4 token tiles of the
// m-tile (from LDS), so every activation operand read from LDS feeds two
// MFMAs.  The 128 accumulators of a wave are 2 x 4 32x32 tiles.
//
// Pipeline: the activation tile of a stage (128 rows x 256 bytes) is staged
// by direct global->LDS loads (no staging registers) into a ring of four
// buffers, three stages ahead, with the 16-byte chunk c of row p stored at
// chunk slot c ^ (p mod 16) so that the 32 rows read by one operand fetch hit
// distinct banks; weight codes and scales go one stage ahead into a second
// register set.  The loads of a stage are spread over the MFMAs of its first
// two steps.  The pipeline runs across items: the last stages of an item
// already fetch the first stages of the workgroup's next item.
//
// Weight layouts: canonical (row-major codes and scales) or the packed layout
// written by moe_prepack_weights, in which one load instruction of a wave
// covers whole 128-byte lines (codes: 8 lines per load instead of 32; scales:
// the 4 bytes of a lane for one stage sit next to those of the other lanes).
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
constexpr int kStageK = 256;              // K per stage (bytes of an FP8 row)
constexpr int kMChunk = 4;                // m-tiles of one expert scheduled together
constexpr int kWaves = 8;                 // waves per workgroup, two per SIMD
constexpr int kWT = 2;                    // 32-row weight tiles per wave
constexpr int kTT = kTileRows / 32;       // 32-row token tiles per m-tile
constexpr int kItemRows = 32 * kWT * kWaves;   // weight rows per item (512)
constexpr int kMaxK = kTiledMaxK;         // largest K the LDS scale copies hold
constexpr int kActDma = kTileRows * kStageK / 1024 / kWaves;   // 1 KB activation loads per wave per stage
constexpr int kWaveRows = kTileRows / kWaves;   // activation rows each wave stages
constexpr int kBlkWaves = kFp8Block / (16 * kWT);   // waves holding one 128-feature block (gate/up)

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane, global -> LDS at lds_base + 16 * lane (lds_base wave-uniform)
__device__ __forceinline__ void dma16(const void* g, void* lds_base) {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_base, 16, 0, 0);
}
// 4 bytes per lane, global -> LDS at lds_base + 4 * lane
__device__ __forceinline__ void dma4(const void* g, void* lds_base) {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_base, 4, 0, 0);
}
// The activation scale bytes of one stage for the four token tiles: bytes at
// LDS offsets addr, addr + 128, addr + 256 and addr + 384, read in one asm
// block that waits for its own reads.  The compiler's wait tracking for the
// direct global->LDS loads cannot tell this copy from the activation ring
// being filled, and before an ordinary read of it would wait for every load
// in flight; the copy is complete and visible here through the stage's own
// wait and barrier.
__device__ __forceinline__ void lds_scale_bytes(uint32_t addr, uint32_t (&b)[4]) {
    asm volatile(
        "ds_read_u8 %0, %4\n\t"
        "ds_read_u8 %1, %4 offset:128\n\t"
        "ds_read_u8 %2, %4 offset:256\n\t"
        "ds_read_u8 %3, %4 offset:384\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3])
        : "v"(addr));
}
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * kStageK + ((chunk ^ (row & 15)) << 4); }

template <int OPSEL_A>
__device__ __forceinline__ v16f mfma32_w4a8(v8i a, v8i b, v16f c, int scale_a, int scale_b) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 0, OPSEL_A, scale_a, 0, scale_b);
}
// The same product with the operands in the other order (FP8 activations as
// A, MXFP4 weights as B; the register contents of both are unchanged): the
// accumulators then hold D transposed, acc[i] of lane l being token
// 8*(i/4) + 4g + (i%4) of the token tile and feature r of the weight tile.
template <int OPSEL_B>
__device__ __forceinline__ v16f mfma32_a8w4(v8i act, v8i w, v16f c, int scale_act, int scale_w) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(act, w, c, 0, 4, 0, scale_act, OPSEL_B, scale_w);
}

// Activation stage ring in LDS: four buffers, declared as separate objects
// so that the compiler's wait tracking for direct global->LDS loads can tell
// a buffer being filled from the one being read.
__shared__ __attribute__((aligned(16))) uint8_t tl_act0[kTileRows * kStageK];
__shared__ __attribute__((aligned(16))) uint8_t tl_act1[kTileRows * kStageK];
__shared__ __attribute__((aligned(16))) uint8_t tl_act2[kTileRows * kStageK];
__shared__ __attribute__((aligned(16))) uint8_t tl_act3[kTileRows * kStageK];
// activation scales of the current and the next item: 128 rows x K/128
// bytes each, dword-column major (dword c of row p at byte 4 * (128 c + p)),
// so that one 4-byte load per lane covers a dword column of 64 rows
constexpr int kXscBytes = kTileRows * (kMaxK / kFp8Block);
// 4-byte loads per wave that copy one item's activation scales (at most)
constexpr int kXscLoads = (kMaxK / kFp8Block / 2 + kWaves - 1) / kWaves;
__shared__ __attribute__((aligned(16))) uint8_t tl_xsc[2 * kXscBytes];
// per-row maxima of the SwiGLU epilogue
__shared__ float tl_red[kWaves * kTileRows];

// s_waitcnt immediate: at most n vector-memory operations outstanding (gfx9
// encoding, vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt at their maxima)
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Weight codes and scales are read with buffer loads: a wave-uniform
// resource per item (base address in scalar registers), a 32-bit lane offset
// that stays fixed for the whole kernel, and the stage offset as the scalar
// offset, so that the loads cost no per-load address registers.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit elements (gfx9 family)
constexpr int kNonTemporal = 2;           // cache-policy bit of a buffer store: non-temporal
__device__ __forceinline__ rsrc_t make_rsrc(const uint8_t* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, 0x7fffffff, kRsrcWord3);
}
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t bload4(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// Workgroup barrier that waits on nothing: the callers first wait for their
// own direct-to-LDS loads with an explicit vmcnt.  The empty asm statements
// keep the compiler from moving memory accesses across it (a release fence
// would also wait for every direct-to-LDS load in flight).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// vector-memory operations a stage issues per wave, in this order: 4 weight
// scale dwords, 4 weight loads per step, the activation loads
constexpr int kStageOps = kWT + 4 * kWT + kActDma;
// waits before the steps of a stage: the step's weights have landed when at
// most the operations issued after them are outstanding (one stage ahead: the
// later steps' weights, the activation loads, and the next stage's scales and
// weights issued by earlier steps of this stage)
constexpr int kWaitStep0 = 3 * kWT + kActDma;
constexpr int kWaitStepN = 2 * kWT + kActDma + kWT + kWT;
static_assert(kWaitStepN == 3 * kWT + kActDma + kWT, "step wait");

// A work item (wave-uniform); ntt = 32-row token tiles that hold rows.
struct Item {
    int e, row0, nrows, nblk, ntt;
};

// Activation rows of one item that this lane loads (with the gather fused,
// looked up through act_rows).
struct Rows {
    int arow[kActDma];     // row of each of the lane's stage loads
    int xrow;              // row whose scale dwords the lane copies
};

// read-only data that every lane of a wave reads alike (constant address space)
typedef const __attribute__((address_space(4))) int* cint_p;
__device__ __forceinline__ int4 load_uniform4(const int4* p) {
    const cint_p q = (cint_p)p;
    return make_int4(q[0], q[1], q[2], q[3]);
}

__device__ __forceinline__ Item item_at(const GemmArgs& a, int item, int NB) {
    // items of expert e: [NB * t0, NB * (t0 + nt)) with t0 its first tile in
    // the plan and nt = ceil(n_e / 128) its tiles.  Its m-tiles go in chunks of
    // kMChunk; within a chunk the order is n-block major, m-tile minor.  The
    // item multiplies the expert's token-tile class: its tiles' height / 32.
    // The plan and the offsets do not change during the kernel and every lane
    // reads the same entries, so they come through scalar loads, which neither
    // wait behind the wave's vector loads in flight nor count against them.
    const cint_p offs = (cint_p)a.offsets;
    const int4 head = load_uniform4(a.tile_info + item / NB);
    const int e = head.x, t0 = head.w;
    const int ne = offs[e + 1] - offs[e];
    const int nt = (ne + kTileRows - 1) / kTileRows;
    const int local = item - NB * t0;
    const int full = nt / kMChunk;
    const int chunk = min(local / (kMChunk * NB), full);
    const int cs = (chunk < full) ? kMChunk : nt - kMChunk * full;
    const int within = local - kMChunk * NB * chunk;
    const int nblk = within / cs;
    const int4 ti = load_uniform4(a.tile_info + t0 + kMChunk * chunk + (within - nblk * cs));
    // every lane computes the same item: keep it in scalar registers
    return Item{__builtin_amdgcn_readfirstlane(e), __builtin_amdgcn_readfirstlane(ti.y),
                __builtin_amdgcn_readfirstlane(ti.z), __builtin_amdgcn_readfirstlane(nblk),
                __builtin_amdgcn_readfirstlane(tile_height(ne, nt) >> 5)};
}

// The persistent loop of one workgroup.  The LDS buffers are separate
// objects: the compiler's wait tracking for direct global->LDS loads tells
// accesses to different objects apart, so a ring buffer can be read while the
// others are being filled (the scale copy, one object of two halves, is read
// in asm for that reason).
template <int MODE, bool PACKED, bool GATHER, int DA, bool PAIR>
__device__ __forceinline__ void tiled_gemm(const GemmArgs& a, uint8_t* __restrict__ act0, uint8_t* __restrict__ act1,
                                           uint8_t* __restrict__ act2, uint8_t* __restrict__ act3,
                                           uint8_t* __restrict__ xsc, float* __restrict__ red) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, r = lane & 31;
    // Down GEMM, items of four or more stages: the operands go to the MFMA the
    // other way round (same register contents, bit-identical results) so that
    // the fp32 rows leave as whole lines straight from the accumulators (Pro
    // skewed prefill 1.71 -> 1.67 ms against rows staged through an LDS
    // tile).  Two-stage items (K = 512, the tensor-parallel shares) keep the
    // weight-major order and store 32-byte pieces: the token-major epilogue
    // spills about 110 registers there and took 1.16 -> 1.79 ms.
    constexpr bool TOKEN_MAJOR = MODE == kGemm2 && !PAIR;

    const int K = (MODE == kGemm2) ? a.I : a.H;
    const int wrows = (MODE == kGemm2) ? a.H : 2 * a.I;
    const int NB = (MODE == kGemm2) ? a.H / kItemRows : a.I / (kItemRows / 2);
    const int nstage = K / kStageK;
    const int XB = K / kFp8Block;

    const int ntiles = a.tile_start[a.E];
    const int total = ntiles * NB;
    const int xcd = blockIdx.x & 7, per_xcd = gridDim.x >> 3;
    const int end = (int)(((long long)total * (xcd + 1)) >> 3);
    int item = (int)(((long long)total * xcd) >> 3) + (int)(blockIdx.x >> 3);
    if (item >= end) return;

    // ---- per-lane geometry ----
    // Weight row of this lane in weight tile 0, relative to the item's first
    // row; tile t adds TROWS * t.  Gate/up: rows 0..15 of a tile are gate
    // features and rows 16..31 the up rows of the same features, so each lane
    // ends up holding matching gate and up values (accumulator elements i and
    // i + 8).  Down: 32 consecutive output features per tile.
    constexpr int TROWS = (MODE == kGemm2) ? 32 : 16;
    const int lrow = (MODE == kGemm2) ? 32 * kWT * wave + r : ((r < 16) ? 0 : a.I) + 16 * kWT * wave + (r & 15);
    const int rows_per_blk = (MODE == kGemm2) ? kItemRows : kItemRows / 2;
    // packed codes: 16-row group q, 128-column step c at (q K/128 + c) KB, row
    // r's 16 bytes of step piece p at 16 (16 p + r); packed scales: group q,
    // step c at 64 (q K/128 + c), row r's 4 bytes at 4 r
    const int wlane = PACKED ? (lrow >> 4) * (8 * K) + 1024 * g + 16 * (r & 15) : lrow * (K / 2) + 64 * g;
    const int slane = PACKED ? (lrow >> 4) * (K / 2) + 64 * g + 4 * (r & 15) : lrow * (K / 32) + 4 * g;
    constexpr int WST = PACKED ? 2048 : kStageK / 2;   // code bytes per stage
    constexpr int WSS = PACKED ? 256 : 16;             // code bytes per step
    constexpr int SST = PACKED ? 128 : 8;              // scale bytes per stage
    const int WTS = TROWS * (K / 2), STS = TROWS * (K / 32);   // per weight tile
    // lane offsets of each weight tile's codes and scales within an item
    uint32_t wl[kWT], sl[kWT];
#pragma unroll
    for (int t = 0; t < kWT; ++t) {
        wl[t] = wlane + t * WTS;
        sl[t] = slane + t * STS;
    }
    // swizzled chunk of this lane's activation loads (piece p and p + 4 alike)
    int coff[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) coff[p] = 16 * ((lane & 15) ^ ((4 * p + (lane >> 4)) & 15));

    // first weight row of an item (in the expert-major weight matrix)
    auto wrow0 = [&](const Item& it) -> size_t { return (size_t)it.e * wrows + (size_t)it.nblk * rows_per_blk; };
    // expert-ordered rows of the lane's stage loads and scale copies
    auto arow_of = [&](const Item& it, int p) { return it.row0 + min(kWaveRows * wave + 4 * p + (lane >> 4), it.nrows - 1); };
    auto xrow_of = [&](const Item& it) { return it.row0 + min(64 * (wave & 1) + lane, it.nrows - 1); };
    // activation rows of an item (fused gather: expert-ordered row ->
    // activation row through act_rows)
    auto lookup_rows = [&](const Item& it, Rows& rw) {
#pragma unroll
        for (int p = 0; p < kActDma; ++p) rw.arow[p] = GATHER ? a.act_rows[arow_of(it, p)] : arow_of(it, p);
        rw.xrow = GATHER ? a.act_rows[xrow_of(it)] : xrow_of(it);
    };
    // activation scales of an item: dword column c of rows 64 h .. 64 h + 63
    // per load (h = wave & 1), loads m = wave, wave + kWaves, ... of XB / 2.  A
    // fixed count, the surplus repeating the last load: the stage bodies stay
    // free of branches (a branch lets the compiler sink the previous stage's
    // MFMAs past the barrier).
    auto dma_xsc = [&](int xrow, uint8_t* dst) {
#pragma unroll
        for (int i = 0; i < kXscLoads; ++i) {
            // past the wave's last load: the last load of the same row half
            const int m = min(wave + kWaves * i, XB / 2 - 1 - ((XB / 2 - 1 - wave) & 1));
            dma4(a.act_scale + 4 * (m >> 1) + (uint32_t)(xrow * XB), dst + 256 * m);
        }
    };
    auto abuf = [&](auto bc) -> uint8_t* {
        constexpr int B = decltype(bc)::value;
        if constexpr (B == 0) return act0;
        else if constexpr (B == 1) return act1;
        else if constexpr (B == 2) return act2;
        else return act3;
    };
    // activation stage st of pieces p0 .. p0+np-1: wave w moves rows 32w ..
    // 32w+31, four rows (64 lanes x 16 bytes) per load; lane i of a load
    // fills chunk slot i%16 of row 4p + i/16 with the chunk the swizzle maps
    // there
    auto dma_act = [&](auto bc, const int (&arow)[kActDma], int st, int p0, int np) {
        uint8_t* lds = abuf(bc);
        const uint8_t* base = a.act + st * kStageK;   // wave-uniform; the lane part fits 32 bits
#pragma unroll
        for (int p = p0; p < p0 + np; ++p)
            dma16(base + (uint32_t)(arow[p] * K + coff[p & 3]), lds + (kWaveRows * wave + 4 * p) * kStageK);
    };

    v16f acc[kWT][kTT];
#pragma unroll
    for (int t = 0; t < kWT; ++t)
#pragma unroll
        for (int j = 0; j < kTT; ++j)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[t][j][i] = 0.0f;

    // weight codes of the current stage [step][weight tile]: step s is
    // refilled with the next stage's codes right after its MFMAs are issued;
    // weight scales of the current and the next stage (byte s for step s)
    uint4 wreg[4][kWT];
    uint32_t wsc[2][kWT];
    Item icur = item_at(a, item, NB);
    int nitem = item + per_xcd;
    bool has_next = nitem < end;
    Item inxt = has_next ? item_at(a, nitem, NB) : icur;
    Rows cur, nxt;
    lookup_rows(icur, cur);
    int xpar = 0;   // which half of tl_xsc holds the current item's scales

    // ---- prologue: scales and the first stages of the first item ----
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    {
        int arow[kActDma];
#pragma unroll
        for (int p = 0; p < kActDma; ++p) arow[p] = cur.arow[p];
        dma_xsc(cur.xrow, xsc);
        dma_act(I0{}, arow, 0, 0, kActDma);
        if constexpr (DA == 3) dma_act(I1{}, arow, 1, 0, kActDma);
        const rsrc_t rs = make_rsrc(a.w_scale + wrow0(icur) * (K / 32));
        const rsrc_t rw = make_rsrc(a.w + wrow0(icur) * (K / 2));
#pragma unroll
        for (int t = 0; t < kWT; ++t) wsc[0][t] = bload4(rs, sl[t], 0);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int t = 0; t < kWT; ++t) wreg[s][t] = bload16(rw, wl[t], s * WSS);
        if constexpr (DA == 3) dma_act(I2{}, arow, 2, 0, kActDma);
        else dma_act(I1{}, arow, 1, 0, kActDma);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));

    // One stage.  KIND 1: the item's first stage (everything it needs has
    // landed; starts the row lookups of the next item); KIND 2: its second
    // (starts the copy of the next item's activation scales).  SET: which
    // weight-scale set the stage reads.
    auto stage = [&](auto bufc, auto setc, auto kindc, auto nttc, int st) {
        constexpr int BUF = decltype(bufc)::value;
        constexpr int SET = decltype(setc)::value;
        constexpr int KIND = decltype(kindc)::value;
        constexpr int NTT = decltype(nttc)::value;   // token tiles multiplied (the rest hold no rows)
        constexpr int NBUF = (BUF + DA) % 4;
        // this stage's activations, scales and first weights have landed in
        // every wave, and every wave is done with the buffer the prefetch
        // below refills
        __builtin_amdgcn_s_waitcnt(vmcnt_only(kWaitStep0));
        lds_barrier();
        const uint8_t* lds = abuf(bufc);
        const uint8_t* xs = xsc + xpar * kXscBytes;
        // activation scale byte of each token tile (128-channel block 2st + g)
        const int xb = 2 * st + g;
        v8i B[NTT];
        auto read_b = [&](int j, int s) {
            const int row = 32 * j + r;
            const uint4 lo4 = *(const uint4*)(lds + swz(row, 2 * s + g));
            const uint4 hi4 = *(const uint4*)(lds + swz(row, 8 + 2 * s + g));
            B[j][0] = lo4.x; B[j][1] = lo4.y; B[j][2] = lo4.z; B[j][3] = lo4.w;
            B[j][4] = hi4.x; B[j][5] = hi4.y; B[j][6] = hi4.z; B[j][7] = hi4.w;
        };
#pragma unroll
        for (int j = 0; j < NTT; ++j) read_b(j, 0);
        int bs[NTT];
        {
            uint32_t b4[kTT];
            lds_scale_bytes(lds_offset(xs) + 4 * ((xb >> 2) * kTileRows + r) + (xb & 3), b4);
#pragma unroll
            for (int j = 0; j < NTT; ++j) bs[j] = (int)b4[j];
        }
        if constexpr (KIND == 1) lookup_rows(inxt, nxt);
        if constexpr (KIND == 2) dma_xsc(nxt.xrow, xsc + (xpar ^ 1) * kXscBytes);
        // prefetch targets: weights of the next stage, activations DA stages
        // ahead (past the item's end: the next item's first stages)
        const bool wcur = st + 1 < nstage;
        const size_t wr = wcur ? wrow0(icur) : wrow0(inxt);
        const int wst = wcur ? st + 1 : 0;
        const rsrc_t rw = make_rsrc(a.w + wr * (K / 2));
        const rsrc_t rs = make_rsrc(a.w_scale + wr * (K / 32));
        const bool acur = st + DA < nstage;
        const int ast = acur ? st + DA : st + DA - nstage;
        int arow[kActDma];
#pragma unroll
        for (int p = 0; p < kActDma; ++p) arow[p] = acur ? cur.arow[p] : nxt.arow[p];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            // The older wave of a SIMD would otherwise take every MFMA issue
            // slot until it stalls, leaving the younger one to finish the
            // stage alone; a priority that falls with the step keeps the two
            // waves of a SIMD within a step of each other.
            switch (s) {
                case 0: __builtin_amdgcn_s_setprio(3); break;
                case 1: __builtin_amdgcn_s_setprio(2); break;
                case 2: __builtin_amdgcn_s_setprio(1); break;
                default: __builtin_amdgcn_s_setprio(0); break;
            }
            // step s's weights have landed
            if (s > 0) {
                __builtin_amdgcn_s_waitcnt(vmcnt_only(kWaitStepN));
                asm volatile("s_nop 0");
                __builtin_amdgcn_sched_barrier(0);
            }
            auto mfmas = [&](int j) {
#pragma unroll
                for (int t = 0; t < kWT; ++t) {
                    const uint4 w = wreg[s][t];
                    const v8i A = {(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
                    const int sa = (int)wsc[SET][t];
                    if constexpr (TOKEN_MAJOR) {
                        // token-major accumulators for the down GEMM's fp32 stores
                        switch (s) {
                            case 0: acc[t][j] = mfma32_a8w4<0>(B[j], A, acc[t][j], bs[j], sa); break;
                            case 1: acc[t][j] = mfma32_a8w4<1>(B[j], A, acc[t][j], bs[j], sa); break;
                            case 2: acc[t][j] = mfma32_a8w4<2>(B[j], A, acc[t][j], bs[j], sa); break;
                            default: acc[t][j] = mfma32_a8w4<3>(B[j], A, acc[t][j], bs[j], sa); break;
                        }
                    } else {
                        switch (s) {
                            case 0: acc[t][j] = mfma32_w4a8<0>(A, B[j], acc[t][j], sa, bs[j]); break;
                            case 1: acc[t][j] = mfma32_w4a8<1>(A, B[j], acc[t][j], sa, bs[j]); break;
                            case 2: acc[t][j] = mfma32_w4a8<2>(A, B[j], acc[t][j], sa, bs[j]); break;
                            default: acc[t][j] = mfma32_w4a8<3>(A, B[j], acc[t][j], sa, bs[j]); break;
                        }
                    }
                }
                if (s < 3) read_b(j, s + 1);
            };
            mfmas(0);
            if (s == 0) {
#pragma unroll
                for (int t = 0; t < kWT; ++t) wsc[SET ^ 1][t] = bload4(rs, sl[t], wst * SST);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 1; j < NTT; ++j) {
                mfmas(j);
                __builtin_amdgcn_sched_barrier(0);
            }
            // step s is done with its weights: refill them with the next stage's
#pragma unroll
            for (int t = 0; t < kWT; ++t) wreg[s][t] = bload16(rw, wl[t], wst * WST + s * WSS);
            if (s == 3) dma_act(std::integral_constant<int, NBUF>{}, arow, ast, 0, kActDma);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // The stages of one item; B0 = ring buffer of its first stage (0, or 2
    // when the stage count is 2 mod 4 and the item is odd); NTT = its token
    // tiles.
    auto run_item = [&](auto b0c, auto nttc) {
        constexpr int B0 = decltype(b0c)::value;
        using S0 = std::integral_constant<int, 0>;
        using S1 = std::integral_constant<int, 1>;
        using KN = std::integral_constant<int, 0>;
        stage(std::integral_constant<int, B0>{}, S0{}, std::integral_constant<int, 1>{}, nttc, 0);
        stage(std::integral_constant<int, (B0 + 1) % 4>{}, S1{}, std::integral_constant<int, 2>{}, nttc, 1);
        int st = 2;
        for (; st + 4 <= nstage; st += 4) {
            stage(std::integral_constant<int, (B0 + 2) % 4>{}, S0{}, KN{}, nttc, st);
            stage(std::integral_constant<int, (B0 + 3) % 4>{}, S1{}, KN{}, nttc, st + 1);
            stage(std::integral_constant<int, B0>{}, S0{}, KN{}, nttc, st + 2);
            stage(std::integral_constant<int, (B0 + 1) % 4>{}, S1{}, KN{}, nttc, st + 3);
        }
        if (st < nstage) {
            stage(std::integral_constant<int, (B0 + 2) % 4>{}, S0{}, KN{}, nttc, st);
            stage(std::integral_constant<int, (B0 + 3) % 4>{}, S1{}, KN{}, nttc, st + 1);
        }
    };

    // Epilogue of the current item (NTT token tiles), then move on to the
    // next; false past the workgroup's last item.
    auto finish_item = [&](auto nttc) -> bool {
        constexpr int NTT = decltype(nttc)::value;
        // ---- epilogue: lane holds tokens 32j + r and tile rows 8*(i/4) + 4g + (i%4) ----
        const int row0 = icur.row0, nrows = icur.nrows, nblk = icur.nblk;
        if constexpr (TOKEN_MAJOR) {
            // token-major accumulators (mfma32_a8w4): lane (g, r) holds feature
            // r of weight tile t for token rows 8*(i/4) + 4g + (i%4) of token
            // tile j, so one dword store over the wave writes two whole
            // 128-byte lines (rows p and p + 4) straight from the registers.
            // Written once and not read again by this kernel: the stores
            // bypass the caches.  Buffer stores: the item's base in the
            // resource, the lane's byte offset in one register, the row's in
            // the scalar offset.  The row stride and the lane offset pass
            // through an empty asm statement, so the 64 row offsets are derived
            // here rather than kept live across the item loop.
            const rsrc_t ro = make_rsrc((const uint8_t*)a.out +
                                        4 * ((size_t)row0 * a.H + nblk * kItemRows + 32 * kWT * wave));
            int hb = 4 * a.H;
            uint32_t vo = 4 * (4 * g * a.H + r);
            asm volatile("" : "+s"(hb), "+v"(vo));
#pragma unroll
            for (int j = 0; j < NTT; ++j) {
                if (32 * j >= nrows) break;   // token tiles past the item's rows hold nothing
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int p = 32 * j + 8 * (i >> 2) + (i & 3);   // row of lanes 0..31; lanes 32..63: p + 4
                    if (p + 4 * g < nrows) {
#pragma unroll
                        for (int t = 0; t < kWT; ++t) {
                            // copied out first: this compiler's bit cast of a vector element
                            // expression reads element 0 whatever the index
                            const float v = acc[t][j][i];
                            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), ro, vo + 128 * t,
                                                                  p * hb, kNonTemporal);
                        }
                    }
                }
            }
        } else if constexpr (MODE == kGemm2) {
            // fp32 rows stored straight from the accumulators: lane (g, r)
            // writes 16 bytes of row r per (tile, quarter), 32 rows per store
#pragma unroll
            for (int j = 0; j < NTT; ++j) {
                if (r >= nrows - 32 * j) continue;
                float* ob = (float*)a.out + ((size_t)(row0 + 32 * j) * a.H + nblk * kItemRows + 32 * kWT * wave);
                const uint32_t lo = (uint32_t)(r * a.H + 4 * g);
#pragma unroll
                for (int t = 0; t < kWT; ++t)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *(v4f*)(ob + (lo + 32 * t + 8 * q)) =
                            v4f{acc[t][j][4 * q], acc[t][j][4 * q + 1], acc[t][j][4 * q + 2], acc[t][j][4 * q + 3]};
            }
        } else if constexpr (MODE == kGemm1Preact) {
            // tile row 8q + 4g + i: q = 0, 1 gate features f + 8q + 4g + i, q = 2, 3 up
#pragma unroll
            for (int j = 0; j < NTT; ++j) {
                if (r >= nrows - 32 * j) continue;
                float* o = (float*)a.out + (size_t)(row0 + 32 * j) * (2 * a.I) + (uint32_t)(r * 2 * a.I);
#pragma unroll
                for (int t = 0; t < kWT; ++t) {
                    const int f = nblk * (kItemRows / 2) + 16 * kWT * wave + 16 * t;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int n = (q < 2 ? f : a.I + f) + 8 * (q & 1) + 4 * g;
                        *(v4f*)(o + n) = v4f{acc[t][j][4 * q], acc[t][j][4 * q + 1], acc[t][j][4 * q + 2],
                                             acc[t][j][4 * q + 3]};
                    }
                }
            }
        } else {
            // SwiGLU on matching gate (element i) and up (element i + 8)
            // values, then FP8 over 128 features: waves 2b and 2b + 1 hold
            // the features of block b of the item
            float amax[NTT];
#pragma unroll
            for (int j = 0; j < NTT; ++j) {
                float m = 0.0f;
#pragma unroll
                for (int t = 0; t < kWT; ++t)
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float gv = acc[t][j][i];
                        const float h = silu_f32(gv) * acc[t][j][i + 8];
                        acc[t][j][i] = h;
                        m = fmaxf(m, fabsf(h));
                    }
                m = fmaxf(m, __shfl_xor(m, 32, 64));
                amax[j] = m;
            }
            if (g == 0) {
#pragma unroll
                for (int j = 0; j < NTT; ++j) red[wave * kTileRows + 32 * j + r] = amax[j];
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < NTT; ++j) {
                const int rr = 32 * j + r;
                const int w0 = wave - wave % kBlkWaves;
                float m = red[w0 * kTileRows + rr];
#pragma unroll
                for (int w = 1; w < kBlkWaves; ++w) m = fmaxf(m, red[(w0 + w) * kTileRows + rr]);
                const int ex = fp8_block_exponent(m);
                // dword d = 4t + 2qq + g of the row's 32 features: lane g holds
                // d = g, g + 2, g + 4, g + 6; one swap with lane l ^ 32 leaves
                // lane g with d = 4g .. 4g + 3, 16 contiguous bytes
                uint32_t dw[kWT][2];
#pragma unroll
                for (int t = 0; t < kWT; ++t)
#pragma unroll
                    for (int qq = 0; qq < 2; ++qq)
                        dw[t][qq] = pack_fp8x4(
                            __builtin_amdgcn_ldexpf(acc[t][j][4 * qq], -ex), __builtin_amdgcn_ldexpf(acc[t][j][4 * qq + 1], -ex),
                            __builtin_amdgcn_ldexpf(acc[t][j][4 * qq + 2], -ex), __builtin_amdgcn_ldexpf(acc[t][j][4 * qq + 3], -ex));
                const uint32_t x0 = g ? dw[0][0] : dw[1][0], x1 = g ? dw[0][1] : dw[1][1];
                const uint32_t y0 = __shfl_xor(x0, 32, 64), y1 = __shfl_xor(x1, 32, 64);
                const uint4 v = g ? uint4{y0, dw[1][0], y1, dw[1][1]} : uint4{dw[0][0], y0, dw[0][1], y1};
                if (r < nrows - 32 * j) {
                    uint8_t* qb = (uint8_t*)a.out + ((size_t)(row0 + 32 * j) * a.I + nblk * (kItemRows / 2) + 16 * kWT * wave);
                    *(uint4*)(qb + (uint32_t)(r * a.I + 16 * g)) = v;
                    if (wave % kBlkWaves == 0 && g == 0)
                        a.out_scale[(size_t)(row0 + rr) * (a.I / kFp8Block) + 2 * nblk + wave / kBlkWaves] = (uint8_t)(ex + 127);
                }
            }
        }
        // stores and the next item's first loads are complete (stores may
        // finish out of order with loads, so no partial count is safe here)
        __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
        if (!has_next) return false;
#pragma unroll
        for (int t = 0; t < kWT; ++t)
#pragma unroll
            for (int j = 0; j < kTT; ++j)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[t][j][i] = 0.0f;
        item = nitem;
        icur = inxt;
        cur = nxt;
        xpar ^= 1;
        nitem = item + per_xcd;
        has_next = nitem < end;
        inxt = has_next ? item_at(a, nitem, NB) : icur;
        return true;
    };

    // With a stage count of 2 mod 4 consecutive items start at ring buffers 0
    // and 2, so items go in pairs; the ring position of every stage stays a
    // compile-time constant either way.  Those kernels run every item on all
    // four token tiles.  The others run each item on its expert's token-tile
    // class, a compile-time constant in one loop per class: the plan lists the
    // classes in the order 4, 3, 2, 1, so a workgroup goes through the loops
    // once, in that order, and the items that share a weight block (the
    // m-tiles of one expert, all of one class) run the same stage bodies.
    using T4 = std::integral_constant<int, 4>;
    if constexpr (PAIR) {
        for (;;) {
            run_item(I0{}, T4{});
            if (!finish_item(T4{})) break;
            run_item(I2{}, T4{});
            if (!finish_item(T4{})) break;
        }
    } else {
        bool more = true;
        auto run_class = [&](auto nttc) {
            while (more && icur.ntt == decltype(nttc)::value) {
                run_item(I0{}, nttc);
                more = finish_item(nttc);
            }
        };
        run_class(T4{});
        run_class(std::integral_constant<int, 3>{});
        run_class(std::integral_constant<int, 2>{});
        run_class(std::integral_constant<int, 1>{});
    }
}

template <int MODE, bool PACKED, bool GATHER, int DA, bool PAIR>
__global__ void __launch_bounds__(64 * kWaves, 1) expert_gemm_tiled_kernel(GemmArgs a) {
    tiled_gemm<MODE, PACKED, GATHER, DA, PAIR>(a, tl_act0, tl_act1, tl_act2, tl_act3, tl_xsc, tl_red);
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


template <int MODE, bool PACKED, bool GATHER>
static void launch_tiled_variant(const GemmArgs& a, hipStream_t stream) {
    dim3 grid(persistent_grid()), block(64 * kWaves);
    const int K = (MODE == kGemm2) ? a.I : a.H;
    // three stages of activations in flight need at least four stages per item
    const int nstage = K / kStageK;
    if (nstage < 4) hipLaunchKernelGGL((expert_gemm_tiled_kernel<MODE, PACKED, GATHER, 2, true>), grid, block, 0, stream, a);
    else if (nstage % 4 == 0) hipLaunchKernelGGL((expert_gemm_tiled_kernel<MODE, PACKED, GATHER, 3, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((expert_gemm_tiled_kernel<MODE, PACKED, GATHER, 3, true>), grid, block, 0, stream, a);
}

template <int MODE>
static void launch_tiled_mode(const GemmArgs& a, hipStream_t stream) {
    // the down GEMM reads its activations in expert order (no gather)
    constexpr bool kCanGather = MODE != kGemm2;
    if (kCanGather && a.act_rows) {
        if (a.packed) launch_tiled_variant<MODE, true, kCanGather>(a, stream);
        else launch_tiled_variant<MODE, false, kCanGather>(a, stream);
    } else {
        if (a.packed) launch_tiled_variant<MODE, true, false>(a, stream);
        else launch_tiled_variant<MODE, false, false>(a, stream);
    }
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
