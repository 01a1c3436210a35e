// The fixed device scratch of tide_reduce_scatter_bf16_fp32_noalloc: a
// file-scope device array, so that a caller that cannot allocate (code under
// graph capture, tight serving loops, harnesses that forbid allocation) still
// gets a reduce-scatter whose per-call tables live in device memory.
//
// Each GPU the library runs on holds its own copy of the array, at its own
// address, until the process ends. In host code the array's name is only a
// host-side stand-in: its device address, per device, comes from
// hipGetSymbolAddress with that device current, and only that address is
// ever handed to a kernel or a copy.
#include <mutex>

#include "tide_internal.hpp"

static __device__ __align__(256) unsigned char scratch[tide::kScratchBytes];

namespace tide {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_address(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_addr[dev]) {
        int prev = -1;
        hipError_t e = hipGetDevice(&prev);
        if (e != hipSuccess) return e;
        if (prev != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (prev != dev) {
            const hipError_t e2 = hipSetDevice(prev);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_addr[dev] = p;
    }
    *out = g_addr[dev];
    return hipSuccess;
}

}  // namespace tide
