// The library's static device scratch: device memory that pn_eval_noalloc
// uses in place of a workspace, for callers that cannot allocate.
//
// One copy of `scratch` exists on every GPU the library runs on, at its own
// address, and stays allocated until the process ends.  Host code never
// passes the array's name to a kernel or a copy (on the host it is only a
// stand-in for the symbol): it asks the runtime for the device address once
// per device, with that device current, and uses that address everywhere.

#include <hip/hip_runtime.h>

#include <mutex>

#include "pn_internal.hpp"

namespace pn {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(void** ptr, size_t* bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_addr[dev] = p;
    }
    *ptr = g_scratch_addr[dev];
    *bytes = kStaticScratchBytes;
    return hipSuccess;
}

}  // namespace pn
