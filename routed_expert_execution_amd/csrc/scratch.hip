// The chunk path's scratch memory for callers that cannot allocate device
// memory (moe_expert_ffn_static): one file-scope device array per GPU, of a
// fixed size, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol): the device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and kernels receive that address.
#include <mutex>

#include "internal.h"

namespace moe {
namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;

}  // namespace

hipError_t static_scratch(void** out) {
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

}  // namespace moe
