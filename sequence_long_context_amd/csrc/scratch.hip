// Device memory for the entry points that allocate nothing: a file-scope
// array in each GPU's memory, used where the other entry points take a
// caller's workspace.  The array's name is only a host-side stand-in; its
// device address is looked up once per device (hipGetSymbolAddress, with that
// device current) and kept, and only that address is handed to kernels.
// Every call on one GPU shares that GPU's array, which keeps the contents the
// last call left; calls that overlap on one GPU race on it.
#include "internal.h"

#include <mutex>

namespace uly {
namespace {

__device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 256;
float *g_scratch[kMaxDevices];  // device address of `scratch` per device, once looked up
std::mutex g_scratch_mutex;

}  // namespace

hipError_t scratch_floats(void *stream, float **ptr) {
    int cur = 0, dev = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    dev = cur;
    if (stream) {
        e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev);
        if (e != hipSuccess) return e;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t back = hipSetDevice(cur);
            if (e == hipSuccess) e = back;
        }
        if (e != hipSuccess) return e;
        g_scratch[dev] = static_cast<float *>(p);
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

}  // namespace uly
