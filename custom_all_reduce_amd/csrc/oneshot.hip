// One-shot all-reduce for gfx950: one output = the fp32 sum of n rank
// buffers, rank 0 first, rounded once ("0-custom-all-reduce", 实现 steps 1-5;
// "集合通信：NCCL 的算法、协议与推理框架的定制 all-reduce", 算法, one-shot).
//
// Layout: each lane owns 16-byte vectors; a workgroup of kBlock lanes covers
// U * kBlock consecutive vectors, lane-consecutive within each of the U rows,
// so every load and store instruction of a wave touches 1 KiB of contiguous
// memory.  All U * n loads of a lane are issued before the first add, which
// keeps U * n * 16 bytes per lane in flight.  The partial last vector (numel
// not a multiple of 4 fp32 / 8 bf16) is summed element by element by the last
// workgroup, so nothing past numel is touched.
#include "ar_device.hpp"
#include "ar_launch.hpp"

namespace ar {
namespace {

// One-wavefront workgroups: measured 5-6% faster than 128 lanes at 8 MiB
// per rank (n = 8 and 16) and equal from 128 KiB to 64 MiB otherwise.
constexpr int kBlock = 64;

template <int NR> struct RankVecs { const u32x4* p[NR]; };

template <typename T, int NR, int U>
__global__ __launch_bounds__(kBlock) void oneshot_kernel(RankVecs<NR> in, u32x4* __restrict__ out,
                                                         uint32_t nvec, uint32_t ntail) {
    const uint32_t base = blockIdx.x * (kBlock * U) + threadIdx.x;
    u32x4 x[U][NR];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t idx = base + u * kBlock;
        if (idx < nvec) {
#pragma unroll
            for (int r = 0; r < NR; ++r) x[u][r] = ld_stream(in.p[r] + idx);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t idx = base + u * kBlock;
        if (idx < nvec) {
            Acc<T> acc;
#pragma unroll
            for (int r = 0; r < NR; ++r) acc.add(x[u][r]);
            st_stream(out + idx, acc.result());
        }
    }
    if (ntail != 0 && blockIdx.x == gridDim.x - 1 && threadIdx.x < ntail) {
        const size_t k = size_t(nvec) * elem<T>::per_vec + threadIdx.x;
        float acc = 0.0f;
#pragma unroll
        for (int r = 0; r < NR; ++r) acc = acc + load_scalar(in.p[r], k, (T*)nullptr);
        store_scalar(out, k, acc, (T*)nullptr);
    }
}

template <typename T, int NR>
hipError_t launch_t(const void* const* in, void* out, size_t numel, hipStream_t s) {
    // One vector per lane per rank and small workgroups: measured fastest
    // from 128 KiB to 64 MiB per rank (more workgroups in flight beat deeper
    // per-lane unrolling on this part).
    constexpr int U = 1;
    const uint32_t nvec = uint32_t(numel / elem<T>::per_vec);
    const uint32_t ntail = uint32_t(numel % elem<T>::per_vec);
    RankVecs<NR> p;
    for (int r = 0; r < NR; ++r) p.p[r] = static_cast<const u32x4*>(in[r]);
    uint32_t grid = (nvec + kBlock * U - 1) / (kBlock * U);
    if (grid == 0) grid = 1;
    hipLaunchKernelGGL((oneshot_kernel<T, NR, U>), dim3(grid), dim3(kBlock), 0, s, p,
                       static_cast<u32x4*>(out), nvec, ntail);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_oneshot(const void* const* in, int n, void* out, size_t numel, int dtype,
                          hipStream_t s) {
    return dispatch_ranks(n, [&](auto nr) {
        constexpr int NR = decltype(nr)::value;
        return dtype == 0 ? launch_t<float, NR>(in, out, numel, s)
                          : launch_t<bf16_t, NR>(in, out, numel, s);
    });
}

}  // namespace ar
