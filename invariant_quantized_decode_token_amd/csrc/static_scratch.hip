// Library-owned device scratch for the entry points that allocate nothing.
//
// One file-scope array per GPU (each device the library runs on holds its own
// copy until the process ends).  In host code the array's name is only a
// host-side stand-in, never a device address: its device address is taken
// once per device with hipGetSymbolAddress, with that device current, and
// kept; everything that hands the scratch to a kernel uses that address.
// Every call on one GPU shares that GPU's array and leaves its contents
// behind, so calls that overlap on one GPU (different streams, different
// host threads) race on it.
#include <mutex>

#include "kernels.hpp"

namespace iqd {
namespace {

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;

}  // namespace

hipError_t static_scratch(void **out) {
    static void *ptrs[kMaxDevices] = {};
    static std::mutex mu;
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (ptrs[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        ptrs[dev] = p;
    }
    *out = ptrs[dev];
    return hipSuccess;
}

}  // namespace iqd
