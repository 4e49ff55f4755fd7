// noalloc.hip -- the library's own fixed device scratch, for det_attn_noalloc
// (callers that cannot allocate device memory: code under graph capture,
// serving loops, harnesses that forbid hipMalloc).
//
// The scratch is one file-scope __device__ array; every GPU the library runs
// on holds its own copy for the life of the process.  In host code the
// array's name is only a host-side stand-in, not a device address: the device
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and kept, and only that address is ever handed to kernels.
#include "kernels.hpp"

#include <hip/hip_runtime.h>

#include <mutex>

namespace det {

static __device__ __align__(256) char scratch[kNoAllocBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void **ptr, size_t *bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    *bytes = kNoAllocBytes;
    return hipSuccess;
}

}  // namespace det
