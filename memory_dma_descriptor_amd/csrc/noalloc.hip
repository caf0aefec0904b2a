// noalloc.hip - the device-resident scratch of the allocation-free entry
// point dmadesc_build_prp_packed_noalloc.
//
// The packed PRP build needs a workspace (a 256-byte header with the block
// ticket and the count of expired waits, then one look-back status word per
// block: 256 requests per block up to 2^19 requests, 1,024 above, so 8 bytes
// per 1,024 requests bound it either way). Callers that cannot allocate device memory use
// this file-scope array instead: every GPU the library runs on holds one
// copy, at its own address, until the process ends. Host code never passes
// the array's name to a kernel (in host code it is a stand-in, not a device
// address); the device address comes from hipGetSymbolAddress, looked up
// once per device with that device current, and is kept per device.
#include <mutex>

#include "dd_internal.h"
#include "dmadesc.h"

namespace dd {
namespace {

constexpr size_t kScratchBytes = 256 + 8 * (DMADESC_NOALLOC_MAX_N / 1024);
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void *g_scratch[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void **ptr, size_t *bytes)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    *bytes = kScratchBytes;
    return hipSuccess;
}

}  // namespace dd
