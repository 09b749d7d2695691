// Device-resident decode workspace for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).  The array lives in the library's code object:
// every GPU the library is loaded on holds its own copy until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol); the device address is looked up
// once per device and kept.
#include <mutex>

#include "kernels.h"

namespace mkv {

static __device__ __align__(256) uint8_t scratch[kStaticWorkspaceBytes];

hipError_t static_workspace(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with this device current: its own copy
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace mkv
