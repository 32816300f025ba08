// Flag-region reset for gfx950: a fill kernel (vector stores of zero) rather
// than a runtime memset, so the call can sit inside a captured HIP graph.
#include "ar_device.hpp"
#include "ar_launch.hpp"

namespace ar {
namespace {

__global__ __launch_bounds__(256) void flag_reset_kernel(u32x4* flags, size_t nvec) {
    for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < nvec;
         i += size_t(gridDim.x) * blockDim.x)
        flags[i] = u32x4{0u, 0u, 0u, 0u};
}

}  // namespace

hipError_t launch_flag_reset(uint32_t* flags, size_t words, hipStream_t s) {
    const size_t nvec = (words + 3) / 4;  // the region is a whole number of 16-byte vectors
    size_t grid = (nvec + 255) / 256;
    if (grid > 64) grid = 64;
    hipLaunchKernelGGL(flag_reset_kernel, dim3(uint32_t(grid)), dim3(256), 0, s,
                       reinterpret_cast<u32x4*>(flags), nvec);
    return hipGetLastError();
}

}  // namespace ar
