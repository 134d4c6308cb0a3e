// The library's static scratch buffer: the workspace of kda_prefill_noalloc, the
// prefill entry point for callers that cannot allocate device memory.
//
// `scratch` is a device array of KDA_NOALLOC_SCRATCH_BYTES in every GPU the library
// runs on, held until the process ends. Its name in host code is only a host-side
// stand-in: the host never passes it to a kernel or a copy. The device address is
// looked up once per device with hipGetSymbolAddress (with that device current) and
// cached; the kernels receive that address as the workspace pointer, exactly as they
// receive a caller's workspace.
#include <mutex>

#include "kda.h"
#include "kda_internal.h"

static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace kda {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up
}  // namespace

size_t static_scratch_bytes() { return sizeof(scratch); }

hipError_t static_scratch(hipStream_t stream, void** ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t back = hipSetDevice(cur);
            if (e == hipSuccess) e = back;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace kda
