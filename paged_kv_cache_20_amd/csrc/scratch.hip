// scratch.hip -- the device scratch array behind attn_paged_decode_noalloc.
//
// Callers that cannot allocate device memory (code under graph capture,
// tight serving loops) get the decode step's split partials placed in one
// file-scope device array instead of a caller workspace.  The array exists
// once per GPU the library runs on and lives until the process ends; every
// call on a GPU shares it, so calls that overlap on one GPU race (the
// partials of one call are written before they are read within that call,
// so nothing in it needs clearing between calls).
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace pa {
namespace {

static __device__ __align__(256) char scratch[kScratchBytes];

// Device address of `scratch` on each GPU, taken once per device with that
// device current.  In host code the array's name is only a stand-in for
// the symbol: kernels receive these addresses, never `scratch` itself.
std::mutex g_mu;
void* g_ptr[kMaxDevices];

}  // namespace

hipError_t scratch_address(void** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace pa
