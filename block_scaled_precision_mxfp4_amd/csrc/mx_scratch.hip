// Fixed device scratch for mxgemm_run_noalloc: one file-scope device array
// per GPU, from library load to process exit.  Host code never passes the
// array's name to a kernel (in host code it is a host-side stand-in, not a
// device address): scratch_address() looks up each device's own copy once,
// with that device current, and every kernel argument uses that address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mx_args.hpp"

static __device__ __align__(256) unsigned char scratch[mx::kScratchBytes];

namespace mx {

namespace {
constexpr int kScratchDevices = 64;
void *g_scratch_ptr[kScratchDevices];
std::mutex g_scratch_mutex;
}  // namespace

hipError_t scratch_address(void **ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kScratchDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace mx
