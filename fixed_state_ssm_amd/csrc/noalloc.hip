// The library's own scratch memory, for idattn_forward_noalloc: a file-scope
// device array that stands in for the caller's workspace, so that a call
// allocates nothing.  Each GPU the library runs on holds its own copy of the
// array (kNoallocScratchBytes) from the moment the code object is loaded on
// that device until the process ends.
//
// In host code the name `scratch` is a host-side stand-in, not a device
// address.  The device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and only that address is
// ever handed to kernels.  Every call on one GPU shares the array, so calls
// that overlap on one GPU (on different streams, or from different threads)
// race; the kernels write every byte they read in the same call, so nothing
// has to be cleared between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace idattn {

namespace {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace idattn
