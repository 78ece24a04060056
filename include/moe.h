/*
 * moe.h - C ABI of the routed Mixture-of-Experts feed-forward layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (pages: "MiMo V2.6 Pro and Flash architecture teardown",
 * sections "What Did Xiaomi Release?", "How Big Is Each Expert?",
 * "How Is the Backbone Built?", "Why Are the V2.6 Files Half the Size of
 * V2.5?"; vLLM recipe "XiaomiMiMo/MiMo-V2.6-Pro-RL", section "Overview"):
 *
 *   L      = x . W_r^T                      bf16 router, fp32 logits
 *   ids    = top-k of (L + b), k of E       ties -> lower expert id
 *   w      = softmax of the k selected L    (b only steers selection)
 *   for each routing slot (t, j), expert e = ids[t][j]:
 *     a    = FP8(x[t])                      e4m3, one e8m0 scale per 128 ch.
 *     g|u  = a . W13_e^T                    W13_e MXFP4 [2I, H]: gate rows, then up rows
 *     h    = FP8(silu(g) * u)               e4m3, one e8m0 scale per 128 ch.
 *     y_s  = h . W2_e^T                     W2_e MXFP4 [H, I]
 *   y[t]   = sum_j w[t][j] * y_(t,j)        no shared expert
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, allocated and owned by the
 *     caller; all layouts are row-major ("[A][B]": B contiguous).
 *   - Work is enqueued on `stream` and runs asynchronously; no entry point
 *     synchronises the host or allocates memory.  Entry points that need
 *     scratch take a caller-provided workspace of at least
 *     moe_workspace_size(problem) bytes (256-byte aligned).
 *   - Outputs are fully overwritten (no pre-zeroing needed).  Inputs and
 *     outputs must not alias.
 *   - Argument errors are detected before anything is enqueued and returned
 *     as a status; nothing is launched then.  A failed launch returns
 *     MOE_ERR_HIP.  num_tokens == 0 returns MOE_OK and launches nothing.
 *   - Inputs must be finite; results for NaN or Inf inputs are unspecified.
 *   - Data errors that only the device can see (expert ids, expert offsets)
 *     are reported in two device error words in the workspace (see
 *     moe_error_words_offset); the kernels clamp every access such an error
 *     would send out of bounds, and the affected results are unspecified.
 *   - Pointers must be 16-byte aligned.
 *   - Limits: hidden and intermediate multiples of 128, 1 <= num_experts
 *     <= 512, 1 <= top_k <= min(num_experts, 8), num_tokens * top_k < 2^31.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same declaration as the HIP runtime's: a stream handle is an opaque pointer. */
typedef struct ihipStream_t* hipStream_t;

#define MOE_ABI_VERSION 6

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARGUMENT = 1,
    MOE_ERR_UNSUPPORTED = 2,
    MOE_ERR_WORKSPACE_TOO_SMALL = 3,
    MOE_ERR_HIP = 4
} moe_status;

/* How experts are scored, selected and weighted (b = optional selection bias).
 * MOE_SCORE_SOFTMAX_TOPK: key = L + b (fp32 add); weights = softmax over the
 *   k selected logits L (the measured workloads).
 * MOE_SCORE_SIGMOID_BIAS: s = sigmoid(L) = 1 / (1 + e^-L), evaluated in
 *   float64 and rounded once to fp32;
 *   key = s + b (fp32 add); weights = the k selected s divided by their sum
 *   (teardown "How Big Is Each Expert?": sigmoid expert scores, plus a
 *   per-expert bias that balances the load across experts).
 * In both, b steers only the selection, ties go to the lower expert id.  */
typedef enum { MOE_SCORE_SOFTMAX_TOPK = 0, MOE_SCORE_SIGMOID_BIAS = 1 } moe_score_func;

typedef enum { MOE_OUT_F32 = 0, MOE_OUT_BF16 = 1 } moe_out_dtype;

/* Storage format of the expert weights, and with it the activation scales.
 * MOE_EXPERTS_MXFP4: the V2.6 experts (teardown, "Why Are the V2.6 Files
 *   Half the Size of V2.5?", table row "Routed experts"): see
 *   moe_expert_weights.  Activation and h scales are e8m0 bytes (powers of
 *   two), one per row per 128 channels.
 * MOE_EXPERTS_FP8_BLOCK: the V2.5 experts of the same table: e4m3 codes with
 *   one float32 scale per 128 x 128 block.  Activation and h scales are
 *   float32, one per row per 128 channels: scale = amax / 448 and codes =
 *   round-to-nearest-even e4m3 of v / scale, both binary32 divisions (an
 *   all-zero run stores scale 0 and the codes of v / 1).                   */
typedef enum { MOE_EXPERTS_MXFP4 = 0, MOE_EXPERTS_FP8_BLOCK = 1 } moe_expert_format;

typedef struct {
    int64_t num_tokens;    /* T  */
    int32_t hidden;        /* H  (multiple of 128) */
    int32_t intermediate;  /* I  (multiple of 128), width of the expert middle layer */
    int32_t num_experts;   /* E  */
    int32_t top_k;         /* k  */
    int32_t score_func;    /* moe_score_func */
    int32_t expert_format; /* moe_expert_format */
} moe_problem;

/* MXFP4 expert weights (teardown, "Why Are the V2.6 Files Half the Size of
 * V2.5?", table row "Routed experts": a byte holds two e2m1 values, and each
 * run of 32 values shares one e8m0 scale).
 * Element 2i of a row is in bits 3:0 of byte i, element 2i+1 in bits 7:4.
 * Scales are e8m0 bytes (2^(b-127)), one per 32 consecutive elements of a row.
 *   w13       [E][2I][H/2]   rows 0..I-1 gate, rows I..2I-1 up
 *   w13_scale [E][2I][H/32]
 *   w2        [E][H][I/2]
 *   w2_scale  [E][H][I/32]
 * FP8 block-scaled experts (problem->expert_format == MOE_EXPERTS_FP8_BLOCK):
 *   w13       [E][2I][H]        e4m3 codes, rows 0..I-1 gate, I..2I-1 up
 *   w13_scale [E][2I/128][H/128] float32, one per 128 x 128 block
 *   w2        [E][H][I]         e4m3 codes
 *   w2_scale  [E][H/128][I/128] float32                                   */
/* Layout of the code and scale bytes (w13, w13_scale, w2, w2_scale).
 * MOE_WEIGHTS_CANONICAL: row-major as above (the checkpoint's layout).
 * MOE_WEIGHTS_PACKED: the layout moe_prepack_weights writes.  For one
 *   expert's matrix of R rows and K columns (w13: R = 2I, K = H; w2: R = H,
 *   K = I), rows go in groups of 16 and columns in steps of 128; experts stay
 *   in order, each the same size as in the canonical layout.
 *   Codes (K/2 bytes per row): group q, step c is a 1024-byte block at byte
 *   offset (q * K/128 + c) * 1024 of the expert's code matrix; in it, bytes
 *   [64c + 16p, 64c + 16p + 16) of row 16q + r (p = 0..3, r = 0..15) sit at
 *   (16p + r) * 16.
 *   Scales (K/32 bytes per row): group q, step c is a 64-byte block at byte
 *   offset (q * K/128 + c) * 64 of the expert's scale matrix; in it, the 4
 *   scale bytes of row 16q + r for columns [128c, 128c + 128) sit at 4r.
 *   FP8 block-scaled experts (K bytes per row): group q, step c is a
 *   2048-byte block at byte offset (q * K/128 + c) * 2048; in it, bytes
 *   [128c + 16p, 128c + 16p + 16) of row 16q + r (p = 0..7) sit at
 *   (16p + r) * 16.  Their float32 scales keep the canonical layout.
 *   Same bytes, reordered so that one 64-lane load covers whole cache lines. */
typedef enum { MOE_WEIGHTS_CANONICAL = 0, MOE_WEIGHTS_PACKED = 1 } moe_weight_layout;

/* Bits of the device error words (moe_error_words_offset).                */
typedef enum {
    MOE_DEVERR_EXPERT_ID_RANGE = 1,      /* a topk_ids entry outside [0, E)          */
    MOE_DEVERR_EXPERT_ID_DUPLICATE = 2,  /* one expert id twice among a token's k     */
    MOE_DEVERR_EXPERT_OFFSETS = 4        /* expert_offsets not 0 = o[0] <= o[1] <= ...
                                            <= o[E] = T*k                           */
} moe_device_error;

typedef struct {
    const uint8_t* w13;
    const uint8_t* w13_scale;
    const uint8_t* w2;
    const uint8_t* w2_scale;
    int32_t layout;        /* moe_weight_layout of w13 and w2 */
} moe_expert_weights;

/* ABI version (MOE_ABI_VERSION of the built library). */
int moe_abi_version(void);

/* Static description of a status code (never NULL). */
const char* moe_status_string(moe_status status);

/* Workspace bytes every entry point of this header needs for `problem`
 * (the maximum over entry points).  Returns 0 for an invalid problem. */
size_t moe_workspace_size(const moe_problem* problem);

/* Byte offset, inside the workspace, of two uint32 device error words
 * (bits: moe_device_error; 0 = no error).  Each is overwritten, in stream
 * order, by the kernels of every call that checks it, so it describes the
 * latest such call on that workspace; read it after that call's stream work
 * has finished (for instance with a device-to-host copy on the same stream).
 *   word 0  moe_permute and moe_forward: the routed expert ids
 *           (MOE_DEVERR_EXPERT_ID_RANGE, MOE_DEVERR_EXPERT_ID_DUPLICATE)
 *   word 1  the grouped-GEMM entry points and moe_forward: the expert offsets
 *           (MOE_DEVERR_EXPERT_OFFSETS); moe_permute writes 0 here when it
 *           also builds the GEMMs' tile plan
 * With an id out of range the slot gets row_of_slot -1 and no row; with
 * invalid offsets the GEMMs write no output rows (LDS-tiled kernels) or only
 * rows inside the clamped offsets (streaming kernels).                     */
size_t moe_error_words_offset(void);

/* Reorder the expert weights into MOE_WEIGHTS_PACKED (a permutation of
 * bytes, nothing is rounded).  Meant to run once, when weights are loaded.
 *   weights           canonical layout (layout == MOE_WEIGHTS_CANONICAL)
 *   w13_packed        [E][2I][H/2] bytes out, w13_scale_packed [E][2I][H/32],
 *   w2_packed         [E][H][I/2] bytes out,  w2_scale_packed  [E][H][I/32];
 *                     (FP8 block-scaled experts: the sizes of w13, w13_scale,
 *                     w2 and w2_scale in that format; scales are copied);
 *                     16-byte aligned, none overlapping another or an input
 * The packed weights are then passed as {w13_packed, w13_scale_packed,
 * w2_packed, w2_scale_packed, MOE_WEIGHTS_PACKED}.                         */
moe_status moe_prepack_weights(const moe_problem* problem, const moe_expert_weights* weights,
                               uint8_t* w13_packed, uint8_t* w13_scale_packed, uint8_t* w2_packed,
                               uint8_t* w2_scale_packed, hipStream_t stream);

/* Router and top-k selection (teardown, "How Big Is Each Expert?": a router
 * picks 8 experts for each token; "Why Are the V2.6 Files Half the Size of
 * V2.5?": BF16 router).
 *   x_bf16        [T][H]  bf16 activations, or NULL
 *   w_router_bf16 [E][H]  bf16 router weights, or NULL
 *   sel_bias      [E]     fp32 selection bias, or NULL (= 0)
 *   logits        [T][E]  fp32: OUTPUT (x . W_r^T, fp32 accumulation of the
 *                         exact bf16 products) when x and w_router are given;
 *                         INPUT when both are NULL (selection on given logits)
 *   topk_ids      [T][k]  int32 out, descending key order, ties -> lower id
 *   topk_w        [T][k]  fp32 out, combine weights per problem->score_func */
moe_status moe_route(const moe_problem* problem, const void* x_bf16, const void* w_router_bf16,
                     const float* sel_bias, float* logits, int32_t* topk_ids, float* topk_w,
                     hipStream_t stream);

/* One step of the rule that keeps the load spread over the experts through
 * the selection bias (teardown, "How Big Is Each Expert?": the sigmoid
 * scores get a small per-expert correction bias that evens out the load
 * without an extra training loss; the page gives no update formula).  With
 * n_e = expert_offsets[e+1] - expert_offsets[e] (the rows moe_permute gave
 * expert e) and N = expert_offsets[E] - expert_offsets[0]:
 *   sel_bias[e] += step   if E * n_e < N  (below the mean load),
 *   sel_bias[e] -= step   if E * n_e > N  (above it),
 *   unchanged             if E * n_e == N,
 * the comparison exact (64-bit integers), the update one fp32 addition.
 *   expert_offsets [E+1]  int32 device, as written by moe_permute
 *   step                  fp32, finite (the caller's step size, e.g. 1e-3)
 *   sel_bias       [E]    fp32 device, updated in place; 16-byte aligned
 * Returns MOE_ERR_INVALID_ARGUMENT for a NULL pointer, a misaligned bias or
 * a non-finite step.  Enqueued on `stream`, not waited for.               */
moe_status moe_update_selection_bias(const moe_problem* problem, const int32_t* expert_offsets, float step,
                                     float* sel_bias, hipStream_t stream);

/* Permutation of the T*k routing slots by expert, and the FP8 activations in
 * expert order.  Slots are s = t*k + j.  Rows of one expert keep ascending
 * token order (a stable counting sort).
 *   topk_ids       [T][k]       int32 in [0, E), distinct per token
 *   x_bf16         [T][H]       bf16
 *   expert_offsets [E+1]        int32 out: rows of expert e are [off[e], off[e+1])
 *   sorted_token   [T*k]        int32 out: token of each expert-ordered row
 *   row_of_slot    [T*k]        int32 out: expert-ordered row of each slot
 *   xq_perm        [T*k][H]     e4m3 out: FP8 codes of x[sorted_token[r]]
 *   xs_perm        [T*k][H/128] out: per-128-channel scale, e8m0 bytes
 *                               (MXFP4 experts) or float32 (FP8 block-scaled)
 * The FP8 rule for MXFP4 experts: amax of each 128-channel run, scale 2^e
 * with e the smallest integer such that amax / 2^e <= 448, codes =
 * round-to-nearest-even e4m3 of x / 2^e (an all-zero run gets scale byte 0).
 * For FP8 block-scaled experts: the float32 rule of moe_expert_format.     */
moe_status moe_permute(const moe_problem* problem, const int32_t* topk_ids, const void* x_bf16,
                       int32_t* expert_offsets, int32_t* sorted_token, int32_t* row_of_slot,
                       uint8_t* xq_perm, void* xs_perm, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* The experts on their rows: gate/up projection, SwiGLU, FP8 requantisation
 * of h, down projection (teardown, "How Big Is Each Expert?": each expert is
 * a gate, an up and a down matrix with an intermediate width of 2,048; vLLM
 * recipe "Overview": MXFP4-stored weights, FP8 arithmetic).
 *   xq_perm, xs_perm, expert_offsets  as produced by moe_permute
 *   y_perm [T*k][H] fp32 out: expert output of each row (unweighted)       */
moe_status moe_grouped_gemm_swiglu(const moe_problem* problem, const uint8_t* xq_perm,
                                   const void* xs_perm, const int32_t* expert_offsets,
                                   const moe_expert_weights* weights, float* y_perm,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* First half of moe_grouped_gemm_swiglu: gate/up projection, SwiGLU
 * h = silu(g) * u with silu(z) = z / (1 + e^-z), and FP8 quantisation of h
 * with the rule of moe_permute.
 *   hq_perm [T*k][I] e4m3 out, hs_perm [T*k][I/128] out (e8m0 bytes, or
 *   float32 for FP8 block-scaled experts)                                 */
moe_status moe_grouped_gemm1_swiglu(const moe_problem* problem, const uint8_t* xq_perm,
                                    const void* xs_perm, const int32_t* expert_offsets,
                                    const moe_expert_weights* weights, uint8_t* hq_perm,
                                    void* hs_perm, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* Gate/up pre-activations only (for exactness checks of the block-scaled
 * product): gu_perm [T*k][2I] fp32 out, columns 0..I-1 gate, I..2I-1 up.  */
moe_status moe_grouped_gemm1_preact(const moe_problem* problem, const uint8_t* xq_perm,
                                    const void* xs_perm, const int32_t* expert_offsets,
                                    const moe_expert_weights* weights, float* gu_perm,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Second half of moe_grouped_gemm_swiglu: y_perm = h . W2_e^T per row.     */
moe_status moe_grouped_gemm2(const moe_problem* problem, const uint8_t* hq_perm,
                             const void* hs_perm, const int32_t* expert_offsets,
                             const moe_expert_weights* weights, float* y_perm,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Weighted combine: y[t] = sum_{j=0..k-1} topk_w[t][j] * y_perm[row_of_slot[t*k+j]],
 * accumulated in fp32 in slot order; out_dtype MOE_OUT_BF16 stores the
 * round-to-nearest-even bf16 of that fp32 sum.  A slot whose row lies
 * outside [0, T*k) (row -1: moe_permute's answer to an id out of range)
 * contributes nothing and is not read.
 *   y [T][H] fp32 or bf16 out                                             */
moe_status moe_combine(const moe_problem* problem, const float* y_perm, const int32_t* row_of_slot,
                       const float* topk_w, void* y, int32_t out_dtype, hipStream_t stream);

/* The whole layer: moe_route, moe_permute, moe_grouped_gemm_swiglu and
 * moe_combine in one stream, all intermediates in the workspace.  The FP8
 * gather is fused into the gate/up GEMM (x is quantised once per token and
 * read through the permutation), which gives the same values as the staged
 * path.                                                                   */
moe_status moe_forward(const moe_problem* problem, const void* x_bf16, const void* w_router_bf16,
                       const float* sel_bias, const moe_expert_weights* weights, void* y,
                       int32_t out_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Size of the scratch array behind moe_forward_noalloc (96 MiB). */
#define MOE_NOALLOC_SCRATCH_BYTES (96u << 20)

/* moe_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, computation, kernels and results as moe_forward, without the
 * workspace: the library keeps it in a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES on every device it runs on (held until the process
 * ends), found on the first call on each device.  Nothing is allocated and no
 * allocating routine is called.  The caller still provides the inputs and y.
 * Limits: moe_workspace_size(problem) <= MOE_NOALLOC_SCRATCH_BYTES, which
 * covers the decode and speculative-verify batches (up to 2048 routed rows
 * at hidden 6144); a larger problem returns MOE_ERR_WORKSPACE_TOO_SMALL
 * before anything is enqueued.  Every call on one device shares that device's
 * array and leaves its own intermediates there (no part of it needs to start
 * at zero: each call writes everything it reads), so calls that can overlap
 * on one device (other streams, other host threads) race: order them, or use
 * moe_forward with a workspace each.  The device error words of the call are
 * at moe_error_words_offset() in the array; they cannot be read without its
 * address, so this entry point is for callers that do not check them.      */
moe_status moe_forward_noalloc(const moe_problem* problem, const void* x_bf16, const void* w_router_bf16,
                               const float* sel_bias, const moe_expert_weights* weights, void* y,
                               int32_t out_dtype, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
