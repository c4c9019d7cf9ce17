// noalloc.hip -- the library's fixed device scratch buffer, for the entry
// point that allocates nothing (attn_fwd_noalloc).
//
// `scratch` is a file-scope device array: every GPU the library runs on
// holds its own copy at its own address until the process ends.  In host
// code the array's name is only a host-side stand-in, so its device address
// is looked up once per device with hipGetSymbolAddress (with that device
// current) and kept; only that address is ever handed to kernels.  The
// lookup allocates nothing.
#include <mutex>

#include "internal.hpp"

namespace rocattn {
namespace {

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_addr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
    *ptr = nullptr;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_addr[dev] = p;
    }
    *ptr = g_addr[dev];
    return hipSuccess;
}

}  // namespace rocattn
