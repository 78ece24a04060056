// Host side of the C ABI declared in include/moe.h: argument validation,
// workspace carving and the launch sequence of each entry point.
//
// Nothing here allocates, synchronises or throws; every check happens before
// the first launch, so a rejected call enqueues nothing.
#include <hip/hip_runtime_api.h>

#include <cmath>

#include "moe.h"
#include "moe_launch.h"

namespace {

using namespace moe;

constexpr size_t kAlign = 256;

static_assert(kErrExpertIdRange == MOE_DEVERR_EXPERT_ID_RANGE && kErrExpertIdDuplicate == MOE_DEVERR_EXPERT_ID_DUPLICATE &&
                  kErrExpertOffsets == MOE_DEVERR_EXPERT_OFFSETS,
              "device error bits of the kernels and of moe.h");

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Layout {
    size_t errors, logits, ids, w, offsets, sorted_token, row_of_slot, block_counts, block_base, block_err;
    size_t tile_start, tile_info;
    size_t xq, xs, hq, hs, y_perm, total;
};

moe_status check_problem(const moe_problem* p) {
    if (!p) return MOE_ERR_INVALID_ARGUMENT;
    if (p->num_tokens < 0) return MOE_ERR_INVALID_ARGUMENT;
    if (p->hidden <= 0 || p->hidden % kFp8Block) return MOE_ERR_INVALID_ARGUMENT;
    if (p->intermediate <= 0 || p->intermediate % kFp8Block) return MOE_ERR_INVALID_ARGUMENT;
    if (p->num_experts < 1 || p->num_experts > 512) return MOE_ERR_INVALID_ARGUMENT;
    if (p->top_k < 1 || p->top_k > 8 || p->top_k > p->num_experts) return MOE_ERR_INVALID_ARGUMENT;
    if (p->score_func != MOE_SCORE_SOFTMAX_TOPK && p->score_func != MOE_SCORE_SIGMOID_BIAS) return MOE_ERR_UNSUPPORTED;
    if (p->expert_format != MOE_EXPERTS_MXFP4 && p->expert_format != MOE_EXPERTS_FP8_BLOCK) return MOE_ERR_UNSUPPORTED;
    if (p->num_tokens * (int64_t)p->top_k >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

bool fp8_block(const moe_problem& p) { return p.expert_format == MOE_EXPERTS_FP8_BLOCK; }
// bytes of one activation / h scale: e8m0, or float32 with FP8 block-scaled experts
size_t scale_bytes(const moe_problem& p) { return fp8_block(p) ? 4 : 1; }

Layout layout_of(const moe_problem& p) {
    const size_t T = (size_t)p.num_tokens, k = (size_t)p.top_k, N = T * k;
    const size_t E = (size_t)p.num_experts, H = (size_t)p.hidden, I = (size_t)p.intermediate;
    const size_t nblk = N ? (N + kPermBlock - 1) / kPermBlock : 1;
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off += round_up(bytes ? bytes : 1); return o; };
    L.errors = take(2 * sizeof(uint32_t));   // first: moe_error_words_offset() is 0
    L.logits = take(T * E * 4);
    L.ids = take(N * 4);
    L.w = take(N * 4);
    L.offsets = take((E + 1) * 4);
    L.sorted_token = take(N * 4);
    L.row_of_slot = take(N * 4);
    L.block_counts = take(nblk * E * 4);
    L.block_base = take(nblk * E * 4);
    L.block_err = take(nblk * 4);
    L.tile_start = take((E + 1) * 4);
    L.tile_info = take((size_t)max_tiles((int64_t)N, (int)E, kRowsPerTile) * 16);   // a bound for any tile size
    const size_t sb = scale_bytes(p);
    L.xq = take(N * H);
    L.xs = take(N * (H / kFp8Block) * sb);
    L.hq = take(N * I);
    L.hs = take(N * (I / kFp8Block) * sb);
    L.y_perm = take(N * H * 4);
    L.total = off;
    return L;
}

template <typename T>
T* at(void* ws, size_t off) { return (T*)((char*)ws + off); }

moe_status check_ws(const moe_problem& p, const void* ws, size_t ws_bytes) {
    if (!ws || !aligned16(ws)) return MOE_ERR_INVALID_ARGUMENT;
    if (((uintptr_t)ws % kAlign) != 0) return MOE_ERR_INVALID_ARGUMENT;
    if (ws_bytes < layout_of(p).total) return MOE_ERR_WORKSPACE_TOO_SMALL;
    return MOE_OK;
}

moe_status check_weights(const moe_expert_weights* w) {
    if (!w || !w->w13 || !w->w13_scale || !w->w2 || !w->w2_scale) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(w->w13) || !aligned16(w->w13_scale) || !aligned16(w->w2) || !aligned16(w->w2_scale))
        return MOE_ERR_INVALID_ARGUMENT;
    if (w->layout != MOE_WEIGHTS_CANONICAL && w->layout != MOE_WEIGHTS_PACKED) return MOE_ERR_INVALID_ARGUMENT;
    return MOE_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

#define MOE_CHECK(expr)                          \
    do {                                         \
        const moe_status st_ = (expr);           \
        if (st_ != MOE_OK) return st_;           \
    } while (0)
#define MOE_LAUNCH(expr)                         \
    do {                                         \
        if ((expr) != hipSuccess) return MOE_ERR_HIP; \
    } while (0)

bool all_aligned() { return true; }
template <typename P, typename... R>
bool all_aligned(P p, R... rest) { return p && aligned16(p) && all_aligned(rest...); }

// ---- launch sequences (arguments already validated) ----------------------

// With xq/xs given and a decode-sized batch, the router launch also writes the
// token-order FP8 copy of x; *quantised tells the caller.
moe_status run_route(const moe_problem& p, const void* x, const void* wr, const float* bias, float* logits,
                     int32_t* ids, float* w, hipStream_t stream, uint8_t* xq = nullptr, void* xs = nullptr,
                     bool* quantised = nullptr) {
    const bool with_quant = x && xq && p.num_tokens <= kDecodeRouterMaxT;
    if (quantised) *quantised = with_quant;
    if (with_quant)
        MOE_LAUNCH(launch_router_quant((const uint16_t*)x, (const uint16_t*)wr, logits, p.num_tokens, p.hidden,
                                       p.num_experts, xq, xs, fp8_block(p), stream));
    else if (x)
        MOE_LAUNCH(launch_router_logits((const uint16_t*)x, (const uint16_t*)wr, logits, p.num_tokens, p.hidden,
                                        p.num_experts, stream));
    MOE_LAUNCH(launch_topk(logits, bias, ids, w, p.num_tokens, p.num_experts, p.top_k,
                           p.score_func == MOE_SCORE_SIGMOID_BIAS, stream));
    return MOE_OK;
}

bool use_tiled(const moe_problem& p);

moe_status check_forward_args(const moe_problem* p, const void* x_bf16, const void* w_router_bf16,
                              const float* sel_bias, const moe_expert_weights* weights, const void* y,
                              int32_t out_dtype) {
    MOE_CHECK(check_problem(p));
    MOE_CHECK(check_weights(weights));
    if (out_dtype != MOE_OUT_F32 && out_dtype != MOE_OUT_BF16) return MOE_ERR_INVALID_ARGUMENT;
    if (!all_aligned(x_bf16, w_router_bf16, y)) return MOE_ERR_INVALID_ARGUMENT;
    if (sel_bias && !aligned16(sel_bias)) return MOE_ERR_INVALID_ARGUMENT;
    return MOE_OK;
}

// Permutation and FP8 gather.  Up to kPermBlock slots (decode) one workgroup
// does the whole permutation and, when the tiled GEMMs will run, also writes
// their tile plan into the workspace (the streaming GEMMs need none);
// *planned tells the caller that it may skip the plan.
moe_status run_permute(const moe_problem& p, const int32_t* ids, const void* x, int32_t* offsets,
                       int32_t* sorted_token, int32_t* row_of_slot, uint8_t* xq, void* xs, void* ws,
                       hipStream_t stream, bool* planned = nullptr, bool fuse_gather = false,
                       bool x_quantised = false) {
    const Layout L = layout_of(p);
    const int64_t N = p.num_tokens * p.top_k;
    if (N <= kPermBlock) {
        const int plan_tiles = use_tiled(p) ? max_tiles(N, p.num_experts, kRowsPerTileTiled) : 0;
        MOE_LAUNCH(launch_perm_small(ids, offsets, sorted_token, row_of_slot, at<int32_t>(ws, L.tile_start),
                                     at<int4>(ws, L.tile_info), at<uint32_t>(ws, L.errors), N, p.num_experts,
                                     p.top_k, kRowsPerTileTiled, plan_tiles, stream));
        if (planned) *planned = true;
    } else {
        int32_t* bc = at<int32_t>(ws, L.block_counts);
        int32_t* bb = at<int32_t>(ws, L.block_base);
        uint32_t* be = at<uint32_t>(ws, L.block_err);
        MOE_LAUNCH(launch_perm_count(ids, bc, be, N, p.num_experts, p.top_k, stream));
        MOE_LAUNCH(launch_perm_scan(bc, bb, offsets, be, at<uint32_t>(ws, L.errors), N, p.num_experts, stream));
        MOE_LAUNCH(launch_perm_scatter(ids, bb, offsets, sorted_token, row_of_slot, N, p.num_experts, p.top_k,
                                       stream));
        if (planned) *planned = false;
    }
    // fused gather: quantise the T tokens once (unless the router launch already
    // did); GEMM-1 reads them through sorted_token
    if (fuse_gather) {
        if (!x_quantised)
            MOE_LAUNCH(launch_quant_gather((const uint16_t*)x, nullptr, xq, xs, p.num_tokens, p.hidden, p.num_tokens,
                                           fp8_block(p), stream));
    } else {
        MOE_LAUNCH(launch_quant_gather((const uint16_t*)x, sorted_token, xq, xs, N, p.hidden, p.num_tokens,
                                       fp8_block(p), stream));
    }
    return MOE_OK;
}

GemmArgs gemm_args(const moe_problem& p, const uint8_t* act, const void* act_scale, const int32_t* offsets,
                   const int32_t* tile_start, const int4* tile_info, const uint8_t* w, const uint8_t* w_scale, void* out,
                   void* out_scale) {
    GemmArgs a;
    a.act = act; a.act_scale = (const uint8_t*)act_scale; a.offsets = offsets; a.tile_start = tile_start; a.tile_info = tile_info;
    a.act_rows = nullptr;
    a.w = w; a.w_scale = w_scale; a.out = out; a.out_scale = (uint8_t*)out_scale;
    a.packed = 0;
    a.err = nullptr;
    a.N = p.num_tokens * p.top_k;
    a.H = p.hidden; a.I = p.intermediate; a.E = p.num_experts;
    return a;
}

// Weight-streaming kernel when experts get few rows (decode); LDS-tiled
// kernel when the average expert has at least 32 rows (prefill).  The choice
// depends on host-known sizes only, so both GEMMs of one call agree on it.
// The tiled kernel addresses activations with 32-bit offsets: every
// activation matrix it reads ([T*k][H] or [T][H], [T*k][I]) stays under 2 GiB.
// FP8 block-scaled experts have their own pair of kernels, chosen the same way.
bool use_tiled(const moe_problem& p) {
    const int64_t rows = p.num_tokens * p.top_k;
    const int64_t widest = p.hidden > p.intermediate ? p.hidden : p.intermediate;
    const bool shape_ok = fp8_block(p) ? fp8_tiled_gemm_supported(p.hidden, p.intermediate)
                                       : tiled_gemm_supported(p.hidden, p.intermediate);
    return shape_ok && rows >= 32 * (int64_t)p.num_experts && rows * widest < ((int64_t)1 << 31);
}

moe_status launch_gemm(const moe_problem& p, GemmMode mode, const GemmArgs& a, hipStream_t stream) {
    if (fp8_block(p))
        MOE_LAUNCH(use_tiled(p) ? launch_expert_gemm_fp8_tiled(mode, a, stream) : launch_expert_gemm_fp8(mode, a, stream));
    else
        MOE_LAUNCH(use_tiled(p) ? launch_expert_gemm_tiled(mode, a, stream) : launch_expert_gemm(mode, a, stream));
    return MOE_OK;
}

moe_status run_gemm1(const moe_problem& p, GemmMode mode, const uint8_t* xq, const void* xs,
                     const int32_t* offsets, const moe_expert_weights& wt, void* out, void* out_scale,
                     void* ws, bool plan, hipStream_t stream, const int32_t* act_rows = nullptr) {
    const Layout L = layout_of(p);
    int32_t* ts = at<int32_t>(ws, L.tile_start);
    int4* ti = at<int4>(ws, L.tile_info);
    // only the tiled kernels read a tile plan; the streaming ones find their
    // m-tile from the offsets
    const int rpt = kRowsPerTileTiled;
    const int64_t N = p.num_tokens * p.top_k;
    uint32_t* err1 = at<uint32_t>(ws, L.errors) + 1;
    if (plan && use_tiled(p))
        MOE_LAUNCH(launch_tile_plan(offsets, ts, ti, err1, p.num_experts, rpt, max_tiles(N, p.num_experts, rpt), N,
                                    stream));
    GemmArgs a = gemm_args(p, xq, xs, offsets, ts, ti, wt.w13, wt.w13_scale, out, out_scale);
    a.packed = wt.layout == MOE_WEIGHTS_PACKED;
    a.act_rows = act_rows;
    a.err = use_tiled(p) ? nullptr : err1;   // the streaming kernels check the offsets themselves
    return launch_gemm(p, mode, a, stream);
}

moe_status run_gemm2(const moe_problem& p, const uint8_t* hq, const void* hs, const int32_t* offsets,
                     const moe_expert_weights& wt, float* y_perm, void* ws, bool plan, hipStream_t stream) {
    const Layout L = layout_of(p);
    int32_t* ts = at<int32_t>(ws, L.tile_start);
    int4* ti = at<int4>(ws, L.tile_info);
    // only the tiled kernels read a tile plan; the streaming ones find their
    // m-tile from the offsets
    const int rpt = kRowsPerTileTiled;
    const int64_t N = p.num_tokens * p.top_k;
    uint32_t* err1 = at<uint32_t>(ws, L.errors) + 1;
    if (plan && use_tiled(p))
        MOE_LAUNCH(launch_tile_plan(offsets, ts, ti, err1, p.num_experts, rpt, max_tiles(N, p.num_experts, rpt), N,
                                    stream));
    GemmArgs a = gemm_args(p, hq, hs, offsets, ts, ti, wt.w2, wt.w2_scale, y_perm, nullptr);
    a.packed = wt.layout == MOE_WEIGHTS_PACKED;
    a.err = use_tiled(p) ? nullptr : err1;
    return launch_gemm(p, kGemm2, a, stream);
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported problem";
        case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case MOE_ERR_HIP: return "HIP launch failure";
    }
    return "unknown status";
}

size_t moe_workspace_size(const moe_problem* p) {
    if (check_problem(p) != MOE_OK) return 0;
    return layout_of(*p).total;
}

size_t moe_error_words_offset(void) { return 0; }

moe_status moe_prepack_weights(const moe_problem* p, const moe_expert_weights* weights, uint8_t* w13_packed,
                               uint8_t* w13_scale_packed, uint8_t* w2_packed, uint8_t* w2_scale_packed,
                               hipStream_t stream) {
    MOE_CHECK(check_problem(p));
    MOE_CHECK(check_weights(weights));
    if (weights->layout != MOE_WEIGHTS_CANONICAL) return MOE_ERR_INVALID_ARGUMENT;
    if (!all_aligned(w13_packed, w13_scale_packed, w2_packed, w2_scale_packed)) return MOE_ERR_INVALID_ARGUMENT;
    const size_t E = (size_t)p->num_experts, H = (size_t)p->hidden, I = (size_t)p->intermediate;
    const bool f8 = fp8_block(*p);
    const uint8_t* in[4] = {weights->w13, weights->w13_scale, weights->w2, weights->w2_scale};
    const uint8_t* out[4] = {w13_packed, w13_scale_packed, w2_packed, w2_scale_packed};
    const size_t n[4] = {f8 ? E * 2 * I * H : E * 2 * I * (H / 2),
                         f8 ? E * (2 * I / 128) * (H / 128) * 4 : E * 2 * I * (H / 32),
                         f8 ? E * H * I : E * H * (I / 2),
                         f8 ? E * (H / 128) * (I / 128) * 4 : E * H * (I / 32)};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 4; ++j) {
            if (overlaps(out[i], n[i], in[j], n[j])) return MOE_ERR_INVALID_ARGUMENT;
            if (j != i && overlaps(out[i], n[i], out[j], n[j])) return MOE_ERR_INVALID_ARGUMENT;
        }
    }
    if (f8) {
        // e4m3 rows of K bytes are packed like e2m1 rows of 2K columns; the
        // float32 block scales keep their layout
        MOE_LAUNCH(launch_prepack(weights->w13, w13_packed, (int64_t)(E * 2 * I), (int)(2 * H), stream));
        MOE_LAUNCH(launch_prepack(weights->w2, w2_packed, (int64_t)(E * H), (int)(2 * I), stream));
        MOE_LAUNCH(hipMemcpyAsync(w13_scale_packed, weights->w13_scale, n[1], hipMemcpyDeviceToDevice, stream));
        MOE_LAUNCH(hipMemcpyAsync(w2_scale_packed, weights->w2_scale, n[3], hipMemcpyDeviceToDevice, stream));
        return MOE_OK;
    }
    MOE_LAUNCH(launch_prepack(weights->w13, w13_packed, (int64_t)(E * 2 * I), (int)H, stream));
    MOE_LAUNCH(launch_prepack_scales(weights->w13_scale, w13_scale_packed, (int64_t)(E * 2 * I), (int)H, stream));
    MOE_LAUNCH(launch_prepack(weights->w2, w2_packed, (int64_t)(E * H), (int)I, stream));
    MOE_LAUNCH(launch_prepack_scales(weights->w2_scale, w2_scale_packed, (int64_t)(E * H), (int)I, stream));
    return MOE_OK;
}

moe_status moe_route(const moe_problem* p, const void* x_bf16, const void* w_router_bf16, const float* sel_bias,
                     float* logits, int32_t* topk_ids, float* topk_w, hipStream_t stream) {
    MOE_CHECK(check_problem(p));
    if ((x_bf16 == nullptr) != (w_router_bf16 == nullptr)) return MOE_ERR_INVALID_ARGUMENT;
    if (x_bf16 && !all_aligned(x_bf16, w_router_bf16)) return MOE_ERR_INVALID_ARGUMENT;
    if (!all_aligned(logits, topk_ids, topk_w)) return MOE_ERR_INVALID_ARGUMENT;
    if (sel_bias && !aligned16(sel_bias)) return MOE_ERR_INVALID_ARGUMENT;
    if (p->num_tokens == 0) return MOE_OK;
    return run_route(*p, x_bf16, w_router_bf16, sel_bias, logits, topk_ids, topk_w, stream);
}

moe_status moe_permute(const moe_problem* p, const int32_t* topk_ids, const void* x_bf16, int32_t* expert_offsets,
                       int32_t* sorted_token, int32_t* row_of_slot, uint8_t* xq_perm, void* xs_perm,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
    MOE_CHECK(check_problem(p));
    if (!all_aligned(topk_ids, x_bf16, expert_offsets, sorted_token, row_of_slot, xq_perm, xs_perm))
        return MOE_ERR_INVALID_ARGUMENT;
    MOE_CHECK(check_ws(*p, ws, ws_bytes));
    if (p->num_tokens == 0) return MOE_OK;
    return run_permute(*p, topk_ids, x_bf16, expert_offsets, sorted_token, row_of_slot, xq_perm, xs_perm, ws, stream);
}

moe_status moe_grouped_gemm1_swiglu(const moe_problem* p, const uint8_t* xq_perm, const void* xs_perm,
                                    const int32_t* expert_offsets, const moe_expert_weights* weights,
                                    uint8_t* hq_perm, void* hs_perm, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
    MOE_CHECK(check_problem(p));
    MOE_CHECK(check_weights(weights));
    if (!all_aligned(xq_perm, xs_perm, expert_offsets, hq_perm, hs_perm)) return MOE_ERR_INVALID_ARGUMENT;
    MOE_CHECK(check_ws(*p, ws, ws_bytes));
    if (p->num_tokens == 0) return MOE_OK;
    return run_gemm1(*p, kGemm1Swiglu, xq_perm, xs_perm, expert_offsets, *weights, hq_perm, hs_perm, ws, true,
                     stream);
}

moe_status moe_grouped_gemm1_preact(const moe_problem* p, const uint8_t* xq_perm, const void* xs_perm,
                                    const int32_t* expert_offsets, const moe_expert_weights* weights,
                                    float* gu_perm, void* ws, size_t ws_bytes, hipStream_t stream) {
    MOE_CHECK(check_problem(p));
    MOE_CHECK(check_weights(weights));
    if (!all_aligned(xq_perm, xs_perm, expert_offsets, gu_perm)) return MOE_ERR_INVALID_ARGUMENT;
    MOE_CHECK(check_ws(*p, ws, ws_bytes));
    if (p->num_tokens == 0) return MOE_OK;
    return run_gemm1(*p, kGemm1Preact, xq_perm, xs_perm, expert_offsets, *weights, gu_perm, nullptr, ws, true,
                     stream);
}

moe_status moe_grouped_gemm2(const moe_problem* p, const uint8_t* hq_perm, const void* hs_perm,
                             const int32_t* expert_offsets, const moe_expert_weights* weights, float* y_perm,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
    MOE_CHECK(check_problem(p));
    MOE_CHECK(check_weights(weights));
    if (!all_aligned(hq_perm, hs_perm, expert_offsets, y_perm)) return MOE_ERR_INVALID_ARGUMENT;
    MOE_CHECK(check_ws(*p, ws, ws_bytes));
    if (p->num_tokens == 0) return MOE_OK;
    return run_gemm2(*p, hq_perm, hs_perm, expert_offsets, *weights, y_perm, ws, true, stream);
}

moe_status moe_grouped_gemm_swiglu(const moe_problem* p, const uint8_t* xq_perm, const void* xs_perm,
                                   const int32_t* expert_offsets, const moe_expert_weights* weights, float* y_perm,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
    MOE_CHECK(check_problem(p));
    MOE_CHECK(check_weights(weights));
    if (!all_aligned(xq_perm, xs_perm, expert_offsets, y_perm)) return MOE_ERR_INVALID_ARGUMENT;
    MOE_CHECK(check_ws(*p, ws, ws_bytes));
    if (p->num_tokens == 0) return MOE_OK;
    const Layout L = layout_of(*p);
    uint8_t* hq = at<uint8_t>(ws, L.hq);
    void* hs = at<uint8_t>(ws, L.hs);
    MOE_CHECK(run_gemm1(*p, kGemm1Swiglu, xq_perm, xs_perm, expert_offsets, *weights, hq, hs, ws, true, stream));
    return run_gemm2(*p, hq, hs, expert_offsets, *weights, y_perm, ws, false, stream);
}

moe_status moe_update_selection_bias(const moe_problem* p, const int32_t* expert_offsets, float step, float* sel_bias,
                                     hipStream_t stream) {
    MOE_CHECK(check_problem(p));
    if (!expert_offsets || !all_aligned(sel_bias) || !std::isfinite(step)) return MOE_ERR_INVALID_ARGUMENT;
    MOE_LAUNCH(launch_bias_update(expert_offsets, p->num_experts, step, sel_bias, stream));
    return MOE_OK;
}

moe_status moe_combine(const moe_problem* p, const float* y_perm, const int32_t* row_of_slot, const float* topk_w,
                       void* y, int32_t out_dtype, hipStream_t stream) {
    MOE_CHECK(check_problem(p));
    if (out_dtype != MOE_OUT_F32 && out_dtype != MOE_OUT_BF16) return MOE_ERR_INVALID_ARGUMENT;
    if (!all_aligned(y_perm, row_of_slot, topk_w, y)) return MOE_ERR_INVALID_ARGUMENT;
    if (p->num_tokens == 0) return MOE_OK;
    MOE_LAUNCH(launch_combine(y_perm, row_of_slot, topk_w, y, out_dtype == MOE_OUT_BF16, p->num_tokens, p->hidden,
                              p->top_k, stream));
    return MOE_OK;
}

moe_status moe_forward(const moe_problem* p, const void* x_bf16, const void* w_router_bf16, const float* sel_bias,
                       const moe_expert_weights* weights, void* y, int32_t out_dtype, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
    MOE_CHECK(check_forward_args(p, x_bf16, w_router_bf16, sel_bias, weights, y, out_dtype));
    MOE_CHECK(check_ws(*p, ws, ws_bytes));
    if (p->num_tokens == 0) return MOE_OK;
    const Layout L = layout_of(*p);
    float* logits = at<float>(ws, L.logits);
    int32_t* ids = at<int32_t>(ws, L.ids);
    float* w = at<float>(ws, L.w);
    int32_t* offsets = at<int32_t>(ws, L.offsets);
    int32_t* st = at<int32_t>(ws, L.sorted_token);
    int32_t* ros = at<int32_t>(ws, L.row_of_slot);
    uint8_t* xq = at<uint8_t>(ws, L.xq);
    void* xs = at<uint8_t>(ws, L.xs);
    uint8_t* hq = at<uint8_t>(ws, L.hq);
    void* hs = at<uint8_t>(ws, L.hs);
    float* y_perm = at<float>(ws, L.y_perm);
    // the FP8 gather is fused into GEMM-1: x is quantised once per token (T rows
    // instead of T*k; on decode batches in the router's launch) and GEMM-1 reads
    // its rows through sorted_token
    bool quantised = false;
    MOE_CHECK(run_route(*p, x_bf16, w_router_bf16, sel_bias, logits, ids, w, stream, xq, xs, &quantised));
    bool planned = false;
    MOE_CHECK(run_permute(*p, ids, x_bf16, offsets, st, ros, xq, xs, ws, stream, &planned, true, quantised));
    MOE_CHECK(run_gemm1(*p, kGemm1Swiglu, xq, xs, offsets, *weights, hq, hs, ws, !planned, stream, st));
    MOE_CHECK(run_gemm2(*p, hq, hs, offsets, *weights, y_perm, ws, false, stream));
    MOE_LAUNCH(launch_combine(y_perm, ros, w, y, out_dtype == MOE_OUT_BF16, p->num_tokens, p->hidden, p->top_k,
                              stream));
    return MOE_OK;
}

}  // extern "C"

extern "C" moe_status moe_forward_noalloc(const moe_problem* p, const void* x_bf16, const void* w_router_bf16,
                                          const float* sel_bias, const moe_expert_weights* weights, void* y,
                                          int32_t out_dtype, hipStream_t stream) {
    MOE_CHECK(check_forward_args(p, x_bf16, w_router_bf16, sel_bias, weights, y, out_dtype));
    if (p->num_tokens == 0) return MOE_OK;
    if (layout_of(*p).total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE_TOO_SMALL;
    // the scratch array's device address on the current device (found once per
    // device), used exactly as moe_forward uses a caller's workspace
    void* ws = noalloc_scratch();
    if (!ws) return MOE_ERR_HIP;
    return moe_forward(p, x_bf16, w_router_bf16, sel_bias, weights, y, out_dtype, ws, MOE_NOALLOC_SCRATCH_BYTES,
                       stream);
}
