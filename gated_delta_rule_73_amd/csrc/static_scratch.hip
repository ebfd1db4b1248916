// static_scratch.hip -- the prefill workspace of gdr_prefill_chunked_static:
// a fixed device array of the library instead of a buffer the caller
// allocates, for callers that cannot allocate device memory.
//
// Every GPU the library runs on holds its own copy of the array until the
// process ends.  In host code the array's name is only a stand-in for the
// symbol: its device address on the current GPU comes from
// hipGetSymbolAddress, looked up once per device and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

static __device__ __align__(256) char scratch[gdr::kStaticScratchBytes];

namespace gdr {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t static_scratch(void **ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with device dev current
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace gdr
