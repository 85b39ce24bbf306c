// noalloc.hip -- the device scratch array behind ar_all_reduce_noalloc, for
// callers that cannot allocate device memory (HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope device array: every GPU that loads this library
// holds its own copy, at its own address, until the process ends. Host code
// never passes the array's name to a kernel or a copy (in host code the name
// is a host-side stand-in, not a device address): it looks up each device's
// address once, with that device current, and uses that pointer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace ar {
namespace {

static __device__ __align__(256) unsigned char scratch[AR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_address(int device, void** out)
{
    *out = nullptr;
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != device) return hipErrorInvalidDevice;  // the caller makes `device` current
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[device] = p;
    }
    *out = g_scratch_ptr[device];
    return hipSuccess;
}

}  // namespace ar
