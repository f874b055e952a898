// gdn_scratch.hip -- the device-resident scratch behind
// gdn_chunked_prefill_noalloc, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).
//
// The buffer is a file-scope __device__ array, so every GPU the library runs
// on holds its own copy from the moment the library's code is loaded on it
// until the process ends.  In host code the array's name is only a host-side
// stand-in: its device address is obtained once per device with
// hipGetSymbolAddress (with that device current) and kept, and only that
// address is ever passed to kernels.
#include <atomic>

#include "gdn_internal.h"

namespace gdn {
namespace {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

}  // namespace

hipError_t scratch_buffer(void **ptr, size_t *bytes)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        // the current device is `dev`: its copy of the array
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    *bytes = kScratchBytes;
    return hipSuccess;
}

}  // namespace gdn
