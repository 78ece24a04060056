// Host-only stand-ins for the kernel launchers of the MoE library, linked with
// the C ABI's host code (abi.cpp) into a library that runs without a GPU:
// the sanitizer build of the host code (AddressSanitizer and
// UndefinedBehaviorSanitizer, g++) that tests/test_abi_sanitize.py runs the
// ABI tests against.
//
// Test infrastructure: nothing here computes any part of the layer.  Each
// stand-in checks the arguments the host code hands to the launcher (required
// pointers present, sizes in range), aborts on a violation (which fails the
// test), counts the call, and returns success without touching memory.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>

#include "moe_launch.h"

namespace {

std::mutex g_mu;
std::map<std::string, int>& counts() {
    static std::map<std::string, int> m;
    return m;
}

void need(bool ok, const char* fn, const char* what) {
    if (!ok) {
        std::fprintf(stderr, "stub %s: %s\n", fn, what);
        std::abort();
    }
}

void count(const char* fn) {
    std::lock_guard<std::mutex> lk(g_mu);
    ++counts()[fn];
}

void check_gemm(const char* fn, const moe::GemmArgs& a) {
    need(a.act && a.act_scale && a.offsets && a.w && a.w_scale && a.out, fn, "null pointer");
    need(a.N >= 1 && a.H >= 128 && a.I >= 128 && a.E >= 1 && a.E <= 512, fn, "sizes");
    count(fn);
}

}  // namespace

extern "C" int moe_stub_calls(const char* name) {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = counts().find(name);
    return it == counts().end() ? 0 : it->second;
}

extern "C" void moe_stub_reset(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    counts().clear();
}

extern "C" hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
    need(dst && src && n > 0, "hipMemcpyAsync", "arguments");
    count("hipMemcpyAsync");
    return hipSuccess;
}

namespace moe {

// the no-allocation entry point's scratch array: a fake aligned address
void* noalloc_scratch() { return reinterpret_cast<void*>(uintptr_t(1) << 30); }

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* w, float* logits, int64_t T, int H, int E,
                                hipStream_t) {
    need(x && w && logits && T >= 1 && H >= 128 && E >= 1, "launch_router_logits", "arguments");
    count("launch_router_logits");
    return hipSuccess;
}

hipError_t launch_topk(const float* logits, const float*, int32_t* ids, float* w, int64_t T, int E, int k, int,
                       hipStream_t) {
    need(logits && ids && w && T >= 1 && E >= 1 && E <= 512 && k >= 1 && k <= 8 && k <= E, "launch_topk",
         "arguments");
    count("launch_topk");
    return hipSuccess;
}

hipError_t launch_bias_update(const int32_t* off, int E, float, float* bias, hipStream_t) {
    need(off && bias && E >= 1 && E <= 512, "launch_bias_update", "arguments");
    count("launch_bias_update");
    return hipSuccess;
}

hipError_t launch_router_quant(const uint16_t* x, const uint16_t* w, float* logits, int64_t T, int H, int E,
                               uint8_t* xq, void* xs, int, hipStream_t) {
    need(x && w && logits && xq && xs && T >= 1 && T <= kDecodeRouterMaxT && H >= 128 && E >= 1,
         "launch_router_quant", "arguments");
    count("launch_router_quant");
    return hipSuccess;
}

hipError_t launch_perm_count(const int32_t* ids, int32_t* bc, uint32_t* be, int64_t N, int E, int k, hipStream_t) {
    need(ids && bc && be && N > kPermBlock && E >= 1 && k >= 1, "launch_perm_count", "arguments");
    count("launch_perm_count");
    return hipSuccess;
}

hipError_t launch_perm_scan(const int32_t* bc, int32_t* bb, int32_t* off, const uint32_t* be, uint32_t* err,
                            int64_t N, int E, hipStream_t) {
    need(bc && bb && off && be && err && N > kPermBlock && E >= 1, "launch_perm_scan", "arguments");
    count("launch_perm_scan");
    return hipSuccess;
}

hipError_t launch_perm_scatter(const int32_t* ids, const int32_t* bb, const int32_t* off, int32_t* st, int32_t* ros,
                               int64_t N, int E, int k, hipStream_t) {
    need(ids && bb && off && st && ros && N > kPermBlock && E >= 1 && k >= 1, "launch_perm_scatter", "arguments");
    count("launch_perm_scatter");
    return hipSuccess;
}

hipError_t launch_perm_small(const int32_t* ids, int32_t* off, int32_t* st, int32_t* ros, int32_t* ts, int4* ti,
                             uint32_t* err, int64_t N, int E, int k, int rpt, int maxt, hipStream_t) {
    need(ids && off && st && ros && ts && ti && err && N >= 1 && N <= kPermBlock && E >= 1 && k >= 1 && rpt >= 32 &&
             maxt >= 0,
         "launch_perm_small", "arguments");
    count("launch_perm_small");
    return hipSuccess;
}

hipError_t launch_quant_gather(const uint16_t* x, const int32_t*, uint8_t* xq, void* xs, int64_t N, int H, int64_t T,
                               int, hipStream_t) {
    need(x && xq && xs && N >= 1 && H >= 128 && T >= 1, "launch_quant_gather", "arguments");
    count("launch_quant_gather");
    return hipSuccess;
}

hipError_t launch_prepack(const uint8_t* src, uint8_t* dst, int64_t rows, int K, hipStream_t) {
    need(src && dst && rows % 16 == 0 && K % 128 == 0, "launch_prepack", "arguments");
    count("launch_prepack");
    return hipSuccess;
}

hipError_t launch_prepack_scales(const uint8_t* src, uint8_t* dst, int64_t rows, int K, hipStream_t) {
    need(src && dst && rows % 16 == 0 && K % 128 == 0, "launch_prepack_scales", "arguments");
    count("launch_prepack_scales");
    return hipSuccess;
}

hipError_t launch_tile_plan(const int32_t* off, int32_t* ts, int4* ti, uint32_t* err, int E, int rpt, int maxt,
                            int64_t N, hipStream_t) {
    need(off && ts && ti && err && E >= 1 && rpt >= 32 && maxt >= 1 && N >= 1, "launch_tile_plan", "arguments");
    count("launch_tile_plan");
    return hipSuccess;
}

hipError_t launch_expert_gemm(GemmMode, const GemmArgs& a, hipStream_t) {
    check_gemm("launch_expert_gemm", a);
    return hipSuccess;
}
hipError_t launch_expert_gemm_tiled(GemmMode, const GemmArgs& a, hipStream_t) {
    need(a.tile_start && a.tile_info, "launch_expert_gemm_tiled", "tile plan");
    check_gemm("launch_expert_gemm_tiled", a);
    return hipSuccess;
}
hipError_t launch_expert_gemm_fp8(GemmMode, const GemmArgs& a, hipStream_t) {
    check_gemm("launch_expert_gemm_fp8", a);
    return hipSuccess;
}
hipError_t launch_expert_gemm_fp8_tiled(GemmMode, const GemmArgs& a, hipStream_t) {
    need(a.tile_start && a.tile_info, "launch_expert_gemm_fp8_tiled", "tile plan");
    check_gemm("launch_expert_gemm_fp8_tiled", a);
    return hipSuccess;
}

hipError_t launch_combine(const float* yp, const int32_t* ros, const float* w, void* y, int, int64_t T, int H, int k,
                          hipStream_t) {
    need(yp && ros && w && y && T >= 1 && H >= 128 && k >= 1, "launch_combine", "arguments");
    count("launch_combine");
    return hipSuccess;
}

}  // namespace moe
