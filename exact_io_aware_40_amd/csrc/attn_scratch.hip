// attn_scratch.hip -- the fixed per-GPU workspace of attn_bwd_noalloc, the
// backward entry point for callers that cannot allocate device memory.
#include <hip/hip_runtime.h>

#include <mutex>

#include "attn_launch.h"

namespace attn {

// The backward's workspace for callers that cannot allocate (attn_bwd_noalloc):
// a fixed array in every GPU's memory, from when the library's code object is
// loaded on that GPU until the process ends.  Host code must not use the
// array's name as an address (on the host it is only a stand-in for the
// symbol); bwd_scratch looks the device address up once per GPU.
static __device__ __align__(256) char scratch[kBwdScratchBytes];

hipError_t bwd_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace attn
