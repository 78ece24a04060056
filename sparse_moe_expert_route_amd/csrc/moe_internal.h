// Internal declarations shared by the HIP translation units of the MoE library.
// Not part of the public ABI (include/moe.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

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
// FP8 block quantisation rule (shared by the activation quantiser and the
// SwiGLU epilogue): scale 2^e with e the smallest integer such that
// amax / 2^e <= 448 = 1.75 * 2^8; written as e8m0 byte e + 127.  With
// amax = m * 2^x, m in [0.5, 1): e = x - 9 if m <= 0.875, else x - 8.
// An all-zero block gets e = -127 (byte 0).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int fp8_block_exponent(float amax) {
    if (!(amax > 0.0f)) return -127;
    int x = __builtin_amdgcn_frexp_expf(amax);
    float m = __builtin_amdgcn_frexp_mantf(amax);
    int e = (m <= 0.875f) ? x - 9 : x - 8;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// FP8 quantisation with a float32 scale (FP8 block-scaled experts): the
// scale of a 128-channel block is amax / 448 and each code is the e4m3
// rounding of v / scale, both IEEE binary32 divisions (hipcc's default fp32
// division is correctly rounded).  The quotient can exceed 448 by one
// rounding; such values round to 448 anyway, and the clamp keeps the
// conversion away from its saturation path.  An all-zero block stores scale
// 0 and divides by 1.
__device__ __forceinline__ float fp8_f32_scale(float amax) { return amax / 448.0f; }
__device__ __forceinline__ float fp8_f32_quotient(float v, float d) { return fminf(fmaxf(v / d, -448.0f), 448.0f); }

// Four floats (already divided by their block scale, |v| <= 448) -> four
// e4m3 bytes, round to nearest even (v_cvt_pk_fp8_f32), byte i = v[i].
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    return (uint32_t)r;
}

// silu(z) = z / (1 + e^-z), with the hardware exponential and reciprocal
// (v_exp_f32, v_rcp_f32: a few ulp) instead of the correctly rounded
// division sequence, which cost the SwiGLU epilogues about ten instructions
// per element.  e^-z overflowing to +inf gives -0, as the division would.
__device__ __forceinline__ float silu_f32(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

__device__ __forceinline__ uint16_t float_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Block-scaled MFMA, A = FP4 (e2m1) weights, B = FP8 (e4m3) activations:
// D[16 weight rows][16 tokens] += sum_k A[row][k] * B[token][k] over 128 k.
// OPSEL_A / OPSEL_B pick the scale byte within each lane's scale register.
template <int OPSEL_A, int OPSEL_B = 0>
__device__ __forceinline__ v4f mfma_w4a8(v8i a, v8i b, v4f c, int scale_a, int scale_b) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, OPSEL_A, scale_a, OPSEL_B, scale_b);
}

// ---------------------------------------------------------------------------
// Launchers (host side).  Every launcher enqueues on `stream` and returns the
// launch status; shapes are validated by the caller.
// ---------------------------------------------------------------------------
hipError_t launch_router_logits(const uint16_t* x, const uint16_t* w_router, float* logits,
                                int64_t T, int H, int E, hipStream_t stream);
hipError_t launch_topk(const float* logits, const float* bias, int32_t* ids, float* w, int64_t T, int E,
                       int k, int sigmoid, hipStream_t stream);
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

// Error bits of caller-given expert offsets (kErrExpertOffsets unless
// 0 = o[0] <= o[1] <= ... <= o[E] = N), evaluated by one wave; every lane
// returns the same value.
__device__ __forceinline__ uint32_t offsets_error(const int32_t* __restrict__ offsets, int E, int64_t N) {
    const int lane = threadIdx.x & 63;
    bool bad = false;
    for (int e = lane; e < E; e += 64) bad |= offsets[e] > offsets[e + 1];
    if (lane == 0) bad |= offsets[0] != 0 || (int64_t)offsets[E] != N;
    return __ballot(bad) ? kErrExpertOffsets : 0u;
}

// M-tile t of kRowsPerTile rows, looked up from the expert offsets alone
// (expert e owns ceil(n_e / 16) tiles, in expert order), so the streaming
// GEMMs need no tile plan.  One wave: lane l sums the tiles of its run of
// ceil(E/64) <= 8 experts, a wave scan finds the lane whose run holds t, and
// that lane's walk over its run gives the expert.  Every lane returns the
// same {expert, first row, rows, 0}, expert -1 for t past the last tile.
// Offsets are clamped to [0, N] and a decreasing pair counts as an empty
// expert, so invalid offsets (reported through offsets_error) still give
// tiles inside the N rows.  Needs E <= 512.
__device__ __forceinline__ int4 find_stream_tile(const int32_t* __restrict__ offsets, int E, int N, int t) {
    const int lane = threadIdx.x & 63;
    const int c = (E + 63) >> 6;
    const int e0 = min(lane * c, E), e1 = min(e0 + c, E);
    int o[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) o[i] = (e0 + i <= e1) ? min(max(offsets[e0 + i], 0), N) : 0;
    int n = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (e0 + i < e1) n += max(o[i + 1] - o[i] + kRowsPerTile - 1, 0) / kRowsPerTile;
    int incl = n;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d, 64);
        if (lane >= d) incl += v;
    }
    const int total = __shfl(incl, 63, 64);
    if (t >= total) return int4{-1, 0, 0, 0};
    const int excl = incl - n;
    int e = -1, row0 = 0, rows = 0, before = excl;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (e0 + i < e1) {
            const int nt = max(o[i + 1] - o[i] + kRowsPerTile - 1, 0) / kRowsPerTile;
            if (t >= before && t < before + nt) {
                e = e0 + i;
                row0 = o[i] + (t - before) * kRowsPerTile;
                rows = min(kRowsPerTile, o[i + 1] - row0);
            }
            before += nt;
        }
    }
    // exactly one lane's run holds t (runs without tiles are empty ranges)
    const int src = __builtin_ctzll(__ballot(e >= 0));
    return int4{__builtin_amdgcn_readfirstlane(__shfl(e, src, 64)), __builtin_amdgcn_readfirstlane(__shfl(row0, src, 64)),
                __builtin_amdgcn_readfirstlane(__shfl(rows, src, 64)), 0};
}

// LDS-tiled variant for many rows per expert: m-tiles of 128 rows, needs
// H and I multiples of 512, at most 6144.
constexpr int kRowsPerTileTiled = 128;
bool tiled_gemm_supported(int H, int I);
hipError_t launch_expert_gemm_tiled(GemmMode mode, const GemmArgs& a, hipStream_t stream);

// FP8 block-scaled experts (e4m3 weights, float32 128 x 128 block scales),
// streaming structure, any row count.
hipError_t launch_expert_gemm_fp8(GemmMode mode, const GemmArgs& a, hipStream_t stream);
// ... LDS-tiled for many rows per expert: m-tiles of 128 rows, H and I multiples of 512, at most 8192.
bool fp8_tiled_gemm_supported(int H, int I);
hipError_t launch_expert_gemm_fp8_tiled(GemmMode mode, const GemmArgs& a, hipStream_t stream);

hipError_t launch_combine(const float* y_perm, const int32_t* row_of_slot, const float* w, void* y,
                          int out_bf16, int64_t T, int H, int k, hipStream_t stream);

}  // namespace moe
