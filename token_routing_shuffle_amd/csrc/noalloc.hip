// Device scratch for the entry point that allocates nothing
// (moe_shuffle_noalloc): a file-scope device array, one copy per GPU, held
// until the process ends.  Host code never passes the array's name to a
// kernel (in host code it is a host-side stand-in, not a device address):
// the address of each device's copy comes from hipGetSymbolAddress, taken
// once per device with that device current, and every later use goes
// through that pointer.
#include <atomic>
#include <mutex>

#include "internal.h"

namespace moe {
namespace {

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_init;

}  // namespace

hipError_t noalloc_scratch(void** out)
{
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_init);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (p == nullptr) return hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace moe
