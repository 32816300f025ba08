// One-shot all-reduce for gfx950: one output = the fp32 sum of n rank
// buffers, rank 0 first, rounded once ("0-custom-all-reduce", 实现 steps 1-5;
// "集合通信：NCCL 的算法、协议与推理框架的定制 all-reduce", 算法, one-shot).
//
// Layout: each lane owns one W-word vector (W = 1 or 2 32-bit words: 1-2
// fp32 or 2-4 bf16) of every rank and of the output; a one-wavefront
// workgroup covers 64 consecutive vectors, so every load and store
// instruction of a wave touches 64 * 4 * W contiguous bytes.  All n loads of
// a lane are issued before the first add.  The partial last vector (numel
// not a multiple of the vector) is summed element by element by the last
// workgroup, so nothing past numel is touched.
//
// Why narrow lanes: once the loads land, a wave's time is its arithmetic
// (widening, n adds per element, rounding), issued one instruction per four
// cycles.  Fewer elements per lane and more wavefronts spread that tail over
// more SIMDs, as long as the grid has fewer wavefronts than the device has
// SIMDs.  Measured (n = 8 / 16): 16-byte lanes 2.75 us at 128 KiB, 8-byte
// lanes 2.60, 4-byte lanes 2.52 / 2.71 (8-byte: 2.63 / 2.96); from 1 MiB on
// 8-byte lanes are the fastest (13.8 us at 8 MiB against 14.6 and 14.1).
//
// Why one vector per lane and a workgroup per 64 vectors, not more work per
// wave: two or four consecutive 64-vector units per wave (all loads first)
// measured 14.7 / 15.2 us at n = 8, 8 MiB bf16 against 13.5; a persistent
// grid of 1024-8192 one-wave workgroups that loads the next unit while it
// sums the current one measured 13.6-16.3 us at 8 MiB and 100-113 us at
// 64 MiB against 95 us.  Letting the dispatcher refill finished waves keeps
// more loads in flight than either.
#include "ar_device.hpp"
#include "ar_launch.hpp"

namespace ar {
namespace {

constexpr int kBlock = 64;
// Below this many bytes per rank the 8-byte grid has fewer wavefronts than
// the device has SIMDs (1024), and 4-byte lanes are used.
constexpr size_t kNarrowMaxBytes = size_t(512) << 10;

template <int W> struct Lane;
template <> struct Lane<1> {
    typedef uint32_t type;
    static __device__ __forceinline__ uint32_t word(type v, int) { return v; }
    static __device__ __forceinline__ type make(const uint32_t* w) { return w[0]; }
};
template <> struct Lane<2> {
    typedef u32x2 type;
    static __device__ __forceinline__ uint32_t word(type v, int i) { return i == 0 ? v.x : v.y; }
    static __device__ __forceinline__ type make(const uint32_t* w) { return u32x2{w[0], w[1]}; }
};

// fp32 accumulation of W words per rank, rank order, one rounding at the end
template <typename T, int W> struct LaneAcc;
template <int W> struct LaneAcc<float, W> {
    float a[W];
    __device__ __forceinline__ LaneAcc() {
#pragma unroll
        for (int i = 0; i < W; ++i) a[i] = 0.0f;
    }
    __device__ __forceinline__ void add(typename Lane<W>::type v) {
#pragma unroll
        for (int i = 0; i < W; ++i) a[i] = a[i] + __uint_as_float(Lane<W>::word(v, i));
    }
    __device__ __forceinline__ typename Lane<W>::type result() const {
        uint32_t w[W];
#pragma unroll
        for (int i = 0; i < W; ++i) w[i] = __float_as_uint(a[i]);
        return Lane<W>::make(w);
    }
};
template <int W> struct LaneAcc<bf16_t, W> {
    float a[2 * W];
    __device__ __forceinline__ LaneAcc() {
#pragma unroll
        for (int i = 0; i < 2 * W; ++i) a[i] = 0.0f;
    }
    __device__ __forceinline__ void add(typename Lane<W>::type v) {
#pragma unroll
        for (int i = 0; i < W; ++i) {
            a[2 * i] = a[2 * i] + bf16_lo(Lane<W>::word(v, i));
            a[2 * i + 1] = a[2 * i + 1] + bf16_hi(Lane<W>::word(v, i));
        }
    }
    __device__ __forceinline__ typename Lane<W>::type result() const {
        uint32_t w[W];
#pragma unroll
        for (int i = 0; i < W; ++i) w[i] = pack_bf16x2(a[2 * i], a[2 * i + 1]);
        return Lane<W>::make(w);
    }
};

template <int NR, int W> struct RankVecs { const typename Lane<W>::type* p[NR]; };

template <typename T, int W> constexpr int per_vec() { return 4 * W / elem<T>::bytes; }

template <typename T, int NR, int W>
__global__ __launch_bounds__(kBlock) void oneshot_kernel(RankVecs<NR, W> in, typename Lane<W>::type* __restrict__ out,
                                                         size_t nvec, uint32_t ntail) {
    typedef typename Lane<W>::type V;
    const size_t idx = size_t(blockIdx.x) * kBlock + threadIdx.x;
    if (idx < nvec) {
        V x[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) x[r] = __builtin_nontemporal_load(in.p[r] + idx);
        LaneAcc<T, W> acc;
#pragma unroll
        for (int r = 0; r < NR; ++r) acc.add(x[r]);
        __builtin_nontemporal_store(acc.result(), out + idx);
    }
    if (ntail != 0 && blockIdx.x == gridDim.x - 1 && threadIdx.x < ntail) {
        const size_t k = nvec * per_vec<T, W>() + threadIdx.x;
        float acc = 0.0f;
#pragma unroll
        for (int r = 0; r < NR; ++r) acc = acc + load_scalar(in.p[r], k, (T*)nullptr);
        store_scalar(out, k, acc, (T*)nullptr);
    }
}

template <typename T, int NR, int W>
hipError_t launch_w(const void* const* in, void* out, size_t numel, hipStream_t s) {
    typedef typename Lane<W>::type V;
    const size_t nvec = numel / per_vec<T, W>();
    const uint32_t ntail = uint32_t(numel % per_vec<T, W>());
    RankVecs<NR, W> p;
    for (int r = 0; r < NR; ++r) p.p[r] = static_cast<const V*>(in[r]);
    size_t grid = (nvec + kBlock - 1) / kBlock;
    if (grid == 0) grid = 1;
    hipLaunchKernelGGL((oneshot_kernel<T, NR, W>), dim3(uint32_t(grid)), dim3(kBlock), 0, s, p,
                       static_cast<V*>(out), nvec, ntail);
    return hipGetLastError();
}

template <typename T, int NR>
hipError_t launch_t(const void* const* in, void* out, size_t numel, hipStream_t s) {
    return numel * elem<T>::bytes < kNarrowMaxBytes ? launch_w<T, NR, 1>(in, out, numel, s)
                                                    : launch_w<T, NR, 2>(in, out, numel, s);
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
