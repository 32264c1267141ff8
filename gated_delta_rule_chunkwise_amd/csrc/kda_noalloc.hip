// Library-held device scratch for the chunk forward that allocates nothing
// (kda_chunk_fwd_noalloc).  Each device that runs the library holds its own
// copy of the array from the loading of the code object until the process
// ends; the host finds the copy of a device through hipGetSymbolAddress, once
// per device, and passes that address to the kernels as their workspace.
#include <hip/hip_runtime.h>
#include <stdio.h>

#include <mutex>

#include "kda_launch.h"

namespace kda {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 256;
void *g_scratch_ptr[kMaxDevices];   // the current device's copy, once looked up
std::mutex g_scratch_mu;
}  // namespace

int noalloc_scratch(void **ptr, char *err, size_t err_len) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        snprintf(err, err_len, "hipGetDevice: %s", hipGetErrorString(e));
        return -1;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        snprintf(err, err_len, "device index %d out of range", dev);
        return -1;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with device dev current
        if (e != hipSuccess || !p) {
            snprintf(err, err_len, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
            return -1;
        }
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return 0;
}

}  // namespace kda
