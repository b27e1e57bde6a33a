// noalloc.hip -- the device scratch array behind r2l_scan_noalloc, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// A chunked plan keeps its carry data (the chunks' local final states, their
// Delta sums and the chunk entry states) in a workspace. r2l_scan_noalloc
// takes that workspace from `scratch`, a file-scope device array that every
// GPU the library runs on holds for the life of the process. In host code
// `scratch` is only a stand-in for the device symbol: its device address is
// looked up once per device, with that device current, and only that address
// is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "scan_internal.h"

static __device__ __align__(256) unsigned char scratch[r2l::kNoallocScratchBytes];

namespace r2l {
namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mutex;
void *g_addr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void **ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_addr[dev] = p;
    }
    *ptr = g_addr[dev];
    return hipSuccess;
}

}  // namespace r2l
