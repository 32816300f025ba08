// Scratch memory of the allocation-free two-shot (ar_twoshot_noalloc): a
// file-scope device array that holds the n segments and the arrival slots,
// so the call needs no allocation from its caller or from the runtime.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and kept; only that address is handed to kernels.
// Each device that runs the call holds its own copy of the array until the
// process ends.
#include <mutex>

#include "ar_launch.hpp"

namespace ar {
namespace {

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxScratchDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** base) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *base = g_scratch[dev];
    return hipSuccess;
}

}  // namespace ar
