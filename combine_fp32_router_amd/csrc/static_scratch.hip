// The library's one static device buffer: histogram scratch of the fused
// route + layout for callers that cannot allocate device memory
// (moe_route_layout_chunks_noalloc).  Every GPU the library runs on holds its
// own copy of the array, at its own device address, until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is taken once per device with hipGetSymbolAddress (that
// device current) and kept here; only that address is ever handed to a
// kernel.  The device is the launch stream's, so a stream created on another
// device than the current one still gets that device's copy.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/moe_route.h"
#include "launch.hpp"

static __device__ __align__(256) int32_t scratch[MOE_NOALLOC_SCRATCH_BYTES / sizeof(int32_t)];

namespace moe {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

}  // namespace

hipError_t static_scratch(hipStream_t stream, void **ptr)
{
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess)
        return e;
    int dev = cur;
    if (stream) {  // the null stream belongs to the current device
        if ((e = hipStreamGetDevice(stream, &dev)) != hipSuccess)
            return e;
    }
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
            return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess)
                e = r;
        }
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace moe
