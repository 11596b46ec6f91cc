// scratch.hip -- the library's one statically allocated device buffer, for
// callers that cannot allocate (ptq1_ffn_block_noalloc).
//
// `scratch` is a file-scope device array: each GPU the library runs on holds
// its own copy, at its own address, until the process ends.  In host code
// the array's name is only a host-side stand-in for the symbol, never a
// device address, so host code uses the address hipGetSymbolAddress returns
// for the current device; it is looked up once per device (with that device
// current) and kept.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <mutex>

#include "ptq1_launch.h"

namespace ptq1 {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_device_ptr(void **ptr)
{
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace ptq1
