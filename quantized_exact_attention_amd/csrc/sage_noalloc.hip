// sage_noalloc.hip -- the workspace of the allocation-free one-call entry
// point: a fixed-size device array held by the library, one copy per GPU.
//
// The array's name is a host-side stand-in in host code, not a device
// address, so host code never passes it to a kernel: the first call on each
// device, with that device current, resolves the array's device address with
// hipGetSymbolAddress and keeps it, and every later use goes through that
// address.  Resolving needs no allocation (the array lives in the code
// object's device memory, loaded with the library's kernels).
#include <hip/hip_runtime.h>

#include <mutex>

#include "sage_launch.hpp"
#include "sage_mi355x.h"

static __device__ __align__(256) unsigned char scratch[SAGE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 256;

struct DeviceScratch {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
};

DeviceScratch g_scratch[kMaxDevices];

}  // namespace

namespace sage {

hipError_t noalloc_scratch(void** out) {
    *out = nullptr;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    DeviceScratch& d = g_scratch[dev];
    std::call_once(d.once, [&d] { d.err = hipGetSymbolAddress(&d.ptr, HIP_SYMBOL(scratch)); });
    if (d.err != hipSuccess) return d.err;
    *out = d.ptr;
    return hipSuccess;
}

}  // namespace sage
