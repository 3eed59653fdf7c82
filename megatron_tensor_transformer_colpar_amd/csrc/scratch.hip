// The library's one file-scope device buffer: the staging area of
// tp_mlp_shard_fwd_noalloc (rank i's activations Y_i between its two GEMMs),
// for callers that cannot allocate device memory (code under graph capture,
// serving loops, harnesses that forbid allocation).  Every GPU the library
// runs on holds its own copy, of kScratchBytes, until the process ends.
//
// In host code `scratch` names a host-side stand-in, not the device copy:
// its device address is looked up once per device, with that device
// current, and only that address is ever handed to a kernel.
#include <hip/hip_runtime.h>

#include <mutex>

#include "tp_kernels.h"

namespace tpk {
namespace {

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];

}  // namespace

hipError_t scratch_base(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p || (reinterpret_cast<uintptr_t>(p) & 255u)) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace tpk
