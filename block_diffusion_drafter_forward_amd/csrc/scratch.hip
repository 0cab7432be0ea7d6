// Device-resident scratch of the allocation-free drafter pass (dflash_draft_block_noalloc): a file-scope
// __device__ array that every GPU the library runs on holds from the code object's load until the process
// ends.  Host code never passes the array's name to a kernel (on the host it only names a stand-in, not the
// device address): the address is looked up once per device with hipGetSymbolAddress, with that device
// current, and kept here.  Every call on one GPU shares the array; overlapping calls on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

static __device__ __align__(256) unsigned char scratch[DFLASH_NOALLOC_SCRATCH_BYTES];

namespace df {

#define DF_SCRATCH_MAX_DEVICES 64

hipError_t scratch_region(void** ptr, size_t* bytes) {
    static std::mutex mu;
    static void* addr[DF_SCRATCH_MAX_DEVICES] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= DF_SCRATCH_MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p || ((uintptr_t)p & 255)) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    *bytes = DFLASH_NOALLOC_SCRATCH_BYTES;
    return hipSuccess;
}

}  // namespace df
