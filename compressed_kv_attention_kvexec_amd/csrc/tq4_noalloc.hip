// tq4_noalloc.hip -- a fixed device scratch area for decode calls whose callers cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
//
// The array below lives in the library's code object, so every GPU the library runs on holds its
// own copy, at its own address, until the process ends.  Host code never passes the array's name
// to a kernel (on the host it is only a stand-in for the symbol): the device address is taken once
// per device with hipGetSymbolAddress, with that device current, and kept here.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "tq4_launch.h"

// Split partials of one decode call (see plan_decode); every call on a device shares them.
static __device__ __align__(256) unsigned char scratch[tq4::kStaticScratchBytes];

namespace tq4 {
namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

hipError_t static_scratch(void **out) {
    *out = nullptr;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
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

}  // namespace tq4
