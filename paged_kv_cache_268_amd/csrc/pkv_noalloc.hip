// pkv_noalloc.hip -- the static scratch behind paged_attn_decode_noalloc.
//
// Callers that cannot allocate device memory (code under graph capture, tight
// serving loops, harnesses that forbid hipMalloc) get a decode whose
// workspace is this file-scope array instead of a caller buffer.  Each GPU the
// library runs on holds its own copy, at its own address, until the process
// ends.  In host code `scratch` names a host-side stand-in, not the device
// memory: the device address comes from hipGetSymbolAddress, looked up once per
// device with that device current, and only that address is ever handed to a
// kernel.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pkv_noalloc.h"

static __device__ __align__(256) unsigned char scratch[pkv::kScratchBytes];

namespace pkv {

hipError_t static_scratch(void** ptr, size_t* bytes) {
    static std::mutex mu;
    static void* addr[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    *bytes = kScratchBytes;
    return hipSuccess;
}

}  // namespace pkv
