// The workspace of the no-allocation fused entry: a file-scope device array,
// so that the entry makes no allocation of its own.  The code object gives
// every GPU it is loaded on its own copy of the array, held until the process
// ends.  Host code never uses the array's name as a device address: the
// address of the current device's copy is looked up with
// hipGetSymbolAddress (once per device) and that pointer is what the kernels
// receive.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "kernels.h"

namespace convrot_detail {
namespace {

static __device__ __align__(256) int8_t scratch[kStaticWorkspaceBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_lookup;

}  // namespace

hipError_t static_workspace(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_lookup);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            // with device `dev` current: its own copy of the array
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess)
                return e;
            if (!p)
                return hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace convrot_detail
