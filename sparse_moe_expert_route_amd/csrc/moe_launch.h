// Host-side declarations shared by the C ABI (abi.cpp) and the HIP
// translation units: constants, the grouped-GEMM argument block and the
// kernel launchers.  Plain C++ over the HIP runtime API: no device code, so
// the host library code also builds with a host compiler (the sanitizer
// build of the C ABI).  Not part of the public ABI (include/moe.h is).
#pragma once

#include <hip/hip_runtime_api.h>
#include <hip/hip_vector_types.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
constexpr int kFp8Block = 128;   // channels per activation scale
constexpr int kMxBlock = 32;     // weight elements per e8m0 scale
constexpr int kPermBlock = 1024; // routing slots per block of the permutation kernels

// Device error words (two uint32 at the start of the workspace; the values
// are those of moe_device_error in moe.h).  Word 0 is written by every
// permutation, word 1 by every grouped-GEMM call, each with a plain store of
// the whole word (no clearing needed, no atomics on global memory).
constexpr uint32_t kErrExpertIdRange = 1u;      // a routed id outside [0, E)
constexpr uint32_t kErrExpertIdDuplicate = 2u;  // one id twice among a token's k slots
constexpr uint32_t kErrExpertOffsets = 4u;      // offsets not 0 = o[0] <= ... <= o[E] = T*k

// ---------------------------------------------------------------------------
// Launchers (host side).  Every launcher enqueues on `stream` and returns the
// launch status; shapes are validated by the caller.
// ---------------------------------------------------------------------------
hipError_t launch_router_logits(const uint16_t* x, const uint16_t* w_router, float* logits,
                                int64_t T, int H, int E, hipStream_t stream);
hipError_t launch_topk(const float* logits, const float* bias, int32_t* ids, float* w, int64_t T, int E,
                       int k, int sigmoid, hipStream_t stream);
// One step of the selection-bias load-balancing rule (moe_update_selection_bias).
hipError_t launch_bias_update(const int32_t* offsets, int E, float step, float* bias, hipStream_t stream);
// Up to kDecodeRouterMaxT tokens the router runs its decode kernel; there it
// can also write the token-order FP8 copy of x (xq [T][H], xs [T][H/128]) in
// the same launch.
constexpr int kDecodeRouterMaxT = 256;
hipError_t launch_router_quant(const uint16_t* x, const uint16_t* w_router, float* logits, int64_t T, int H, int E,
                               uint8_t* xq, void* xs, int f32_scales, hipStream_t stream);

// block_err [ceil(N / kPermBlock)]: error bits of each block of slots, reduced
// by the scan into err_word (word 0)
hipError_t launch_perm_count(const int32_t* ids, int32_t* block_counts, uint32_t* block_err, int64_t N, int E,
                             int k, hipStream_t stream);
hipError_t launch_perm_scan(const int32_t* block_counts, int32_t* block_base, int32_t* offsets,
                            const uint32_t* block_err, uint32_t* err_word, int64_t N, int E, hipStream_t stream);
hipError_t launch_perm_scatter(const int32_t* ids, const int32_t* block_base, const int32_t* offsets,
                               int32_t* sorted_token, int32_t* row_of_slot, int64_t N, int E, int k,
                               hipStream_t stream);
// count + scan + scatter + tile plan in one workgroup, for N <= kPermBlock;
// writes error word 0, and word 1 (= 0) when it writes a tile plan
hipError_t launch_perm_small(const int32_t* ids, int32_t* offsets, int32_t* sorted_token, int32_t* row_of_slot,
                             int32_t* tile_start, int4* tile_info, uint32_t* err_words, int64_t N, int E, int k,
                             int rows_per_tile, int max_tiles, hipStream_t stream);
// xs: e8m0 bytes (power-of-two scales), or float32 when f32_scales is set
hipError_t launch_quant_gather(const uint16_t* x, const int32_t* sorted_token, uint8_t* xq,
                               void* xs, int64_t N, int H, int64_t T, int f32_scales, hipStream_t stream);

// Byte permutation of a matrix of `rows` rows x K e2m1 columns (K/2 bytes per
// row, rows a multiple of 16, K a multiple of 128) into the packed weight
// layout of moe.h (MOE_WEIGHTS_PACKED).
hipError_t launch_prepack(const uint8_t* src, uint8_t* dst, int64_t rows, int K, hipStream_t stream);
hipError_t launch_prepack_scales(const uint8_t* src, uint8_t* dst, int64_t rows, int K, hipStream_t stream);

// tile_info[t] = {expert, first row, rows} of m-tile t for t < max_tiles
// (expert -1 past the last tile); max_tiles = ceil(N / rows_per_tile) + E.
// Offsets that are not 0 = o[0] <= ... <= o[E] = N give an empty plan (no
// tiles) and kErrExpertOffsets in *err_word (word 1); valid ones write 0.
hipError_t launch_tile_plan(const int32_t* offsets, int32_t* tile_start, int4* tile_info, uint32_t* err_word, int E,
                            int rows_per_tile, int max_tiles, int64_t N, hipStream_t stream);
inline int max_tiles(int64_t N, int E, int rows_per_tile) { return (int)((N + rows_per_tile - 1) / rows_per_tile) + E; }

// Height of every m-tile of an expert with n rows cut into nt = ceil(n / rpt)
// tiles (rpt a multiple of 32): the smallest multiple of 32 that covers n in
// nt tiles, so that the tiles of one expert are equally high and the padding
// of its 32-row token tiles stays below 32 rows per tile (one 128-row tile
// per expert would pad up to 127 rows).  Tile t covers rows
// [t h, min((t + 1) h, n)).
__host__ __device__ inline int tile_height(int n, int nt) {
    return nt > 0 ? 32 * ((n + 32 * nt - 1) / (32 * nt)) : 0;
}

enum GemmMode { kGemm1Swiglu = 0, kGemm1Preact = 1, kGemm2 = 2 };

// Grouped expert GEMM over the expert-ordered rows.  For gemm1 modes the
// weights are W13 [E][2I][H/2] and K = H; for gemm2 they are W2 [E][H][I/2]
// and K = I.  FP8 block-scaled experts: codes [E][2I][H] / [E][H][I] e4m3,
// scales float32 [E][rows/128][K/128], activation and h scales float32.
struct GemmArgs {
    const uint8_t* act;        // [N][K] e4m3
    const uint8_t* act_scale;  // [N][K/128] e8m0 (float32 for FP8 block-scaled experts)
    const int32_t* act_rows;   // optional: activation row of each expert-ordered row (gather fused into
                               // the GEMM: act/act_scale then hold one row per token); null = identity
    const int32_t* offsets;    // [E+1]
    const int32_t* tile_start; // tiled kernels: [E+1], first m-tile of each expert
    const int4* tile_info;     // tiled kernels: per m-tile {expert, first row, rows}, expert -1 past the end
    const uint8_t* w;          // codes
    const uint8_t* w_scale;    // e8m0 per 32 (float32 per 128 x 128 block for FP8 block-scaled experts)
    void* out;                 // swiglu: hq [N][I] + hs; preact: float [N][2I]; gemm2: float [N][H]
    uint8_t* out_scale;        // swiglu: hs [N][I/128] (e8m0, or float32 for FP8 block-scaled experts)
    uint32_t* err;             // streaming kernels: error word 1 (offsets check), written by workgroup 0; or null
    int64_t N;
    int H, I, E;
    int packed;                // weight codes in the 16-row packed layout (moe_prepack_weights)
};
constexpr int kRowsPerTile = 16;   // rows per m-tile of the streaming expert GEMM
hipError_t launch_expert_gemm(GemmMode mode, const GemmArgs& a, hipStream_t stream);

// LDS-tiled variant for many rows per expert: m-tiles of 128 rows, needs
// H and I multiples of 512, at most 6144.
constexpr int kRowsPerTileTiled = 128;
constexpr int kTiledMaxK = 6144;      // largest K (H or I) the tiled kernel's LDS scale copies hold
inline bool tiled_gemm_supported(int H, int I) {
    return H % 512 == 0 && I % 512 == 0 && H <= kTiledMaxK && I <= kTiledMaxK;
}
hipError_t launch_expert_gemm_tiled(GemmMode mode, const GemmArgs& a, hipStream_t stream);

// FP8 block-scaled experts (e4m3 weights, float32 128 x 128 block scales),
// streaming structure, any row count.
hipError_t launch_expert_gemm_fp8(GemmMode mode, const GemmArgs& a, hipStream_t stream);
// ... LDS-tiled for many rows per expert: m-tiles of 128 rows, H and I multiples of 512, at most 8192.
constexpr int kF8TiledMaxK = 8192;    // largest K of the FP8 tiled kernel (its LDS block-scale rows)
inline bool fp8_tiled_gemm_supported(int H, int I) {
    return H % 512 == 0 && I % 512 == 0 && H <= kF8TiledMaxK && I <= kF8TiledMaxK;
}
hipError_t launch_expert_gemm_fp8_tiled(GemmMode mode, const GemmArgs& a, hipStream_t stream);

// Device address of the current device's copy of the moe_forward_noalloc
// scratch array (MOE_NOALLOC_SCRATCH_BYTES, 256-byte aligned), looked up once
// per device; null if the HIP runtime reports an error.
void* noalloc_scratch();

hipError_t launch_combine(const float* y_perm, const int32_t* row_of_slot, const float* w, void* y,
                          int out_bf16, int64_t T, int H, int k, hipStream_t stream);

}  // namespace moe
