// The device scratch array behind shard_linear_group_noalloc: the workspace
// of a grouped shard product (activation copies, k-partials, arrival
// counters) for callers that cannot allocate device memory.
//
// One array per GPU, part of the library's code object: the runtime places
// a copy in each device's memory when the library is first used there, and
// it stays until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol): the
// device address of the current GPU's copy is looked up once per device with
// hipGetSymbolAddress and kept in a table; every use goes through it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.hpp"

static __device__ __align__(256) unsigned char scratch[tsl::kNoAllocScratchBytes];

namespace tsl {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices]; // device address per device id, null until looked up

} // namespace

hipError_t noalloc_scratch(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

} // namespace tsl
