// The library's one device-resident scratch array, for callers that cannot
// allocate device memory (kvc_decode_attn_noalloc): code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc.
//
// Each GPU the library runs on holds its own copy of `scratch` until the
// process ends.  In host code the array's name is only a host-side stand-in,
// never a device address: the device address is looked up once per device
// with hipGetSymbolAddress (with that device current) and kept per device,
// and only that address is ever handed to a kernel.
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/kvc.h"
#include "kvc_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[KVC_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::atomic<void*> scratch_addr[MAX_DEVICES];

}  // namespace

namespace kvc {

hipError_t noalloc_scratch(hipStream_t stream, void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    if (stream) {
        // the stream must belong to the current device: its kernels read
        // that device's copy of the array
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess) return e;
        if (sdev != dev) return hipErrorInvalidDevice;
    }
    void* p = scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        scratch_addr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace kvc
