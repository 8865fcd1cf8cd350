// noalloc.hip -- the static device scratch array behind ra_share_backward_noalloc.
//
// The backward kernels keep two floats per query row (D = dO . O and lse * log2 e) in a
// workspace.  ra_share_backward takes that workspace from the caller; the allocation-free
// entry point uses this file-scope array instead, so the call needs no hipMalloc.  Each
// GPU holds its own copy of the array at its own address for the life of the process;
// host code never passes the array's name to a kernel, only the address that
// hipGetSymbolAddress returns for the current device.
#include <mutex>

#include "../../include/ra.h"
#include "ra_internal.h"

namespace ra {
namespace {

__device__ __align__(256) unsigned char scratch[RA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_addr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_addr[dev] = p;
    }
    *ptr = g_addr[dev];
    return hipSuccess;
}

}  // namespace ra
