// One-shot all-reduce for gfx950: one output = the fp32 sum of n rank
// buffers, rank 0 first, rounded once ("0-custom-all-reduce", 实现 steps 1-5;
// "集合通信：NCCL 的算法、协议与推理框架的定制 all-reduce", 算法, one-shot).
//
// Layout: each lane owns one 8-byte vector (2 fp32 or 4 bf16) of every rank
// and of the output; a one-wavefront workgroup covers 64 consecutive
// vectors, so every load and store instruction of a wave touches 512
// contiguous bytes.  All n loads of a lane are issued before the first add.
// The partial last vector (numel not a multiple of 2 fp32 / 4 bf16) is
// summed element by element by the last workgroup, so nothing past numel is
// touched.
//
// Why 8 bytes per lane and not 16: once the loads land, a wave's time is
// its arithmetic (widening, n adds per element, rounding), issued one
// instruction per four cycles.  Half the elements per lane and twice the
// wavefronts spread that tail over twice the SIMDs; measured faster at
// every size from 16 KiB to 8 MiB per rank (n = 8: 2.65 -> 2.51 us at
// 128 KiB, 14.45 -> 13.80 us at 8 MiB).
#include "ar_device.hpp"
#include "ar_launch.hpp"

namespace ar {
namespace {

constexpr int kBlock = 64;

template <int NR> struct RankVecs { const u32x2* p[NR]; };

template <typename T> constexpr int per_vec8() { return 8 / elem<T>::bytes; }

template <typename T, int NR>
__global__ __launch_bounds__(kBlock) void oneshot_kernel(RankVecs<NR> in, u32x2* __restrict__ out,
                                                         size_t nvec, uint32_t ntail) {
    const size_t idx = size_t(blockIdx.x) * kBlock + threadIdx.x;
    if (idx < nvec) {
        u32x2 x[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) x[r] = __builtin_nontemporal_load(in.p[r] + idx);
        Acc8<T> acc;
#pragma unroll
        for (int r = 0; r < NR; ++r) acc.add(x[r].x, x[r].y);
        __builtin_nontemporal_store(acc.result(), out + idx);
    }
    if (ntail != 0 && blockIdx.x == gridDim.x - 1 && threadIdx.x < ntail) {
        const size_t k = nvec * per_vec8<T>() + threadIdx.x;
        float acc = 0.0f;
#pragma unroll
        for (int r = 0; r < NR; ++r) acc = acc + load_scalar(in.p[r], k, (T*)nullptr);
        store_scalar(out, k, acc, (T*)nullptr);
    }
}

template <typename T, int NR>
hipError_t launch_t(const void* const* in, void* out, size_t numel, hipStream_t s) {
    const size_t nvec = numel / per_vec8<T>();
    const uint32_t ntail = uint32_t(numel % per_vec8<T>());
    RankVecs<NR> p;
    for (int r = 0; r < NR; ++r) p.p[r] = static_cast<const u32x2*>(in[r]);
    size_t grid = (nvec + kBlock - 1) / kBlock;
    if (grid == 0) grid = 1;
    hipLaunchKernelGGL((oneshot_kernel<T, NR>), dim3(uint32_t(grid)), dim3(kBlock), 0, s, p,
                       static_cast<u32x2*>(out), nvec, ntail);
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
