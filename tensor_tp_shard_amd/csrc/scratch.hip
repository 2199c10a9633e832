// scratch.hip -- the library's one static device buffer: the workspace of
// decode_step_noalloc, the entry point for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// Each GPU the library runs on holds its own copy of `scratch` (at its own
// address) until the process ends. In host code the array's name is only a
// host-side stand-in, never a device address: its address on the current
// device comes from hipGetSymbolAddress, looked up once per device at set-up
// (load_weights) and kept; kernels get that address as an argument.
#include <mutex>

#include "common.h"

namespace tps {

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices] = {};
} // namespace

hipError_t scratch_address(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_scratch_addr[dev] = p;
    }
    *ptr = g_scratch_addr[dev];
    return hipSuccess;
}

} // namespace tps
