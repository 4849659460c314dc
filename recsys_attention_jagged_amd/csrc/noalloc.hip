// The library's fixed device scratch array, for entry points that must not
// allocate (callers under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  One array per GPU, resident until the process ends;
// every call on one GPU shares it and it keeps the last call's contents, so
// calls that overlap in time on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"

namespace gdpa {

// file-scope scratch: in host code this name is only a stand-in for the device
// symbol; host code uses the address hipGetSymbolAddress returns for the current
// device (below), never the name itself
static __device__ __align__(256) char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** out) {
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        // once per device, with that device current (hipGetDevice above)
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace gdpa
