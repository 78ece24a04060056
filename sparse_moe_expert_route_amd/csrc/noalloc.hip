// Scratch memory of moe_forward_noalloc (include/moe.h): the workspace of the
// forward as a file-scope device array, for callers that cannot allocate.
//
// Every device the library runs on holds its own copy of the array, from the
// library's first use on that device until the process ends.  In host code the
// array's name only stands for the symbol: its device address comes from
// hipGetSymbolAddress, asked once per device (with that device current, on the
// first moe_forward_noalloc call there) and kept in g_scratch; the kernels
// receive that address as their workspace pointer.
#include <mutex>

#include <hip/hip_runtime.h>

#include "moe.h"
#include "moe_launch.h"

namespace moe {

namespace {

static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

}  // namespace

void* noalloc_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

}  // namespace moe
