// decode_scratch.hip -- the device array behind attn_decode_noalloc.
//
// The split kernels' partial results live here instead of in a
// caller-provided workspace.  Each device holds its own copy until the
// process ends.  The array sits in a source file of its own: the runtime
// loads a source file's device code on the first use of anything in it, and
// setting up 32 MiB of device memory took the first decode call from about
// 0.9 ms to 14 ms when the array shared the decode kernels' file; now only the
// first attn_decode_noalloc call pays it.
#include <hip/hip_runtime.h>

#include <atomic>

#include "kernels.h"

namespace attn {

// In host code `scratch` is only a stand-in for the symbol; its device
// address comes from hipGetSymbolAddress.
static __device__ __align__(256) char scratch[DECODE_SCRATCH_BYTES];

hipError_t decode_scratch(void **out) {
    static std::atomic<void *> addr[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    void *p = addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev].store(p, std::memory_order_release);  // concurrent first calls store the same address
    }
    *out = p;
    return hipSuccess;
}

}  // namespace attn
