// wkv7_static.hip -- the fixed device scratch of the entry point that allocates
// nothing (wkv7_forward_split_static).
//
// `scratch` is a file-scope device array: every device that loads the library
// holds its own copy, at its own address, until the process ends.  In host
// code the array's name stands for a host-side shadow, not a device address,
// so host code never passes it to a kernel: it looks the device address up
// once per device with hipGetSymbolAddress (with that device current) and
// uses that pointer from then on.

#include <hip/hip_runtime.h>

#include <mutex>

#include "wkv7.h"
#include "wkv7_internal.h"

namespace wkv7 {

namespace {

static __device__ __align__(256) unsigned char scratch[WKV7_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_addr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(void** ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> guard(g_lock);
    if (g_addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_addr[dev] = p;
    }
    *ptr = g_addr[dev];
    return hipSuccess;
}

}  // namespace wkv7
