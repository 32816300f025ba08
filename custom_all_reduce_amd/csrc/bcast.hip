// Store-side variants of the reduction for gfx950 ("0-custom-all-reduce",
// 实现: the kBroadcast store path of step 5 and the one-shot push named among
// the algorithms there; "集合通信：NCCL 的算法、协议与推理框架的定制 all-reduce",
// 算法, two-shot).
//
// reduce_bcast: emulated rank r reduces its own 1/n of the 16-byte vectors of
// every input (the same fold as the one-shot: fp32, rank 0 first, one
// rounding) and stores each result into all n outputs.  Over all ranks this
// is a reduce-scatter whose all-gather is pushed by the producer itself, so no
// barrier separates the phases.  One rank's share reads S and writes S.
//
// push: a rank's message copied into n destinations (one slot of every
// rank's staging buffer); the receivers then reduce their staging slots with
// the one-shot.  One sender reads S and writes n * S.  With one destination
// it is the staging copy of a caller's tensor into its registered buffer.
//
// The reduce-broadcast takes one 8-byte half of a 16-byte vector per lane
// (half the arithmetic per lane and twice the wavefronts, as in the
// one-shot: measured equal or up to 8% faster, 3-4% for every rank's share
// at 64 MiB); the push, which has no arithmetic, one 16-byte vector.  Both
// stream their stores past the caches.  Their loads are plain: measured,
// that is 15-20% faster at 64 MiB per rank than nontemporal loads for these
// store-heavy kernels (the read-heavy one-shot, two-shot and LL kernels
// measure the other way round).
#include "ar_device.hpp"
#include "ar_launch.hpp"

namespace ar {
namespace {

constexpr int kBlock = 128;

template <int NR> struct InVecs { const u32x4* p[NR]; };
template <int NR> struct OutVecs { u32x4* p[NR]; };

// Vectors [vb, ve) (16-byte units, the ownership unit) of every input
// reduced and stored into all NR outputs, one 8-byte half per lane.  With
// ntail != 0 (the launch owns the end of the message, ve = all full
// vectors) the last workgroup also sums the ntail trailing elements.
template <typename T, int NR>
__global__ __launch_bounds__(kBlock) void reduce_bcast_kernel(InVecs<NR> in, OutVecs<NR> out, uint32_t vb,
                                                              uint32_t ve, uint32_t ntail) {
    const size_t h = size_t(vb) * 2 + size_t(blockIdx.x) * kBlock + threadIdx.x;
    if (h < size_t(ve) * 2) {
        u32x2 x[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) x[r] = reinterpret_cast<const u32x2*>(in.p[r])[h];
        __builtin_amdgcn_sched_barrier(0);  // every load ahead of the first add
        Acc8<T> acc;
#pragma unroll
        for (int r = 0; r < NR; ++r) acc.add(x[r]);
        const u32x2 y = acc.result();
#pragma unroll
        for (int r = 0; r < NR; ++r) __builtin_nontemporal_store(y, reinterpret_cast<u32x2*>(out.p[r]) + h);
    }
    if (ntail != 0 && blockIdx.x == gridDim.x - 1 && threadIdx.x < ntail) {
        const size_t k = size_t(ve) * elem<T>::per_vec + threadIdx.x;
        float acc = 0.0f;
#pragma unroll
        for (int r = 0; r < NR; ++r) acc = acc + load_scalar(in.p[r], k, (T*)nullptr);
#pragma unroll
        for (int r = 0; r < NR; ++r) store_scalar(out.p[r], k, acc, (T*)nullptr);
    }
}

template <int ND> struct PushArgs {
    const u32x4* src;
    u32x4* dst[ND];
};

// One sender's nvec vectors copied to ND destinations; the last workgroup
// also copies the ntail trailing 16-bit units.
template <int ND>
__global__ __launch_bounds__(kBlock) void push_kernel(PushArgs<ND> a, uint32_t nvec, uint32_t ntail) {
    const uint32_t idx = blockIdx.x * kBlock + threadIdx.x;
    if (idx < nvec) {
        const u32x4 x = a.src[idx];
#pragma unroll
        for (int j = 0; j < ND; ++j) st_stream(a.dst[j] + idx, x);
    }
    if (ntail != 0 && blockIdx.x == gridDim.x - 1 && threadIdx.x < ntail) {
        const size_t k = size_t(nvec) * 8 + threadIdx.x;
        const uint16_t v = reinterpret_cast<const uint16_t*>(a.src)[k];
#pragma unroll
        for (int j = 0; j < ND; ++j) reinterpret_cast<uint16_t*>(a.dst[j])[k] = v;
    }
}

template <typename T, int NR>
hipError_t launch_bcast_t(const void* const* in, void* const* out, size_t numel, int r0, int r1, hipStream_t s) {
    const uint64_t nvec = numel / elem<T>::per_vec;
    const uint32_t ntail = r1 == NR ? uint32_t(numel % elem<T>::per_vec) : 0u;
    const uint32_t vb = uint32_t(nvec * uint64_t(r0) / NR);
    const uint32_t ve = uint32_t(nvec * uint64_t(r1) / NR);
    if (ve == vb && ntail == 0) return hipSuccess;  // this range owns no data
    InVecs<NR> pi;
    OutVecs<NR> po;
    for (int r = 0; r < NR; ++r) {
        pi.p[r] = static_cast<const u32x4*>(in[r]);
        po.p[r] = static_cast<u32x4*>(out[r]);
    }
    uint32_t grid = uint32_t((size_t(ve - vb) * 2 + kBlock - 1) / kBlock);
    if (grid == 0) grid = 1;
    hipLaunchKernelGGL((reduce_bcast_kernel<T, NR>), dim3(grid), dim3(kBlock), 0, s, pi, po, vb, ve, ntail);
    return hipGetLastError();
}

template <int ND>
hipError_t launch_push_t(const void* src, void* const* dst, size_t nbytes, hipStream_t s) {
    const uint32_t nvec = uint32_t(nbytes / 16);
    const uint32_t ntail = uint32_t(nbytes % 16) / 2;
    PushArgs<ND> a;
    a.src = static_cast<const u32x4*>(src);
    for (int j = 0; j < ND; ++j) a.dst[j] = static_cast<u32x4*>(dst[j]);
    uint32_t grid = (nvec + kBlock - 1) / kBlock;
    if (grid == 0) grid = 1;
    hipLaunchKernelGGL((push_kernel<ND>), dim3(grid), dim3(kBlock), 0, s, a, nvec, ntail);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_reduce_bcast(const void* const* in, int n, void* const* out, size_t numel, int dtype, int r0,
                               int r1, hipStream_t s) {
    return dispatch_ranks(n, [&](auto nr) {
        constexpr int NR = decltype(nr)::value;
        return dtype == 0 ? launch_bcast_t<float, NR>(in, out, numel, r0, r1, s)
                          : launch_bcast_t<bf16_t, NR>(in, out, numel, r0, r1, s);
    });
}

hipError_t launch_push(const void* const* src, int nsrc, void* const* dst, int ndst, size_t nbytes,
                       hipStream_t s) {
    for (int i = 0; i < nsrc; ++i) {
        // one destination: the staging copy into a registered buffer
        const hipError_t e = ndst == 1 ? launch_push_t<1>(src[i], dst + i, nbytes, s)
                                       : dispatch_ranks(ndst, [&](auto nd) {
                                             constexpr int ND = decltype(nd)::value;
                                             return launch_push_t<ND>(src[i], dst + size_t(i) * ndst, nbytes, s);
                                         });
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace ar
