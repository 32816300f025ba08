// One-shot all-reduce fused with a residual add and RMSNorm, for gfx950.
//
// "集合通信：NCCL 的算法、协议与推理框架的定制 all-reduce" names, among the
// inference frameworks' communication paths, an all-reduce fused with
// RMSNorm (the FlashInfer kernel SGLang integrates) without defining it.
// This library's reading, per element (i, k) of rows x hidden data:
//   h = (the one-shot's fold of the ranks' element: fp32, rank 0 first,
//        from +0) + residual[i, k]
//   residual_out[i, k] = h rounded once to the data type
//   y[i, k] = h * (1 / sqrt(mean over row i of h^2 + eps)) * weight[k],
//            computed in fp32 and rounded once to the data type.
// residual_out may be the residual buffer itself (updated in place).
//
// Work.  A workgroup owns a row (above 2^20 rows the workgroups stride over
// the rows): each lane takes 16-byte vectors v = lane + j * blockDim
// (j < VPT) of the row, loads the ranks' vectors and the residual's with
// nontemporal loads, folds them, stores residual_out and keeps h in
// registers.  The row's sum of h^2 goes lane -> wavefront (xor shuffles) ->
// workgroup (LDS), then every lane scales its h by the row's factor and the
// weight (plain loads, issued with the data: the same hidden-length vector
// for every row, so it stays in the caches) and stores the output.  One pass
// over HBM: the inputs and the residual are read once, residual_out and the
// output written once.
//
// Few heavy rows (a decode step's handful of tokens) put a whole row's
// n + 1 streams through one compute unit with a workgroup per row, so with a
// workspace a fixed grid of kCoopGrid one-wavefront workgroups splits such
// rows into parts of 64 vectors: each part folds its vectors, stores
// residual_out, and publishes
// the partial sum of its h^2 to its own slot as one 8-byte store of the
// value and the call's step id (written together, so a reader that sees the
// step sees the value, with no store wait, as in an LL line).  The parts of
// a row poll their siblings' slots (bounded; a timeout is reported in the
// workspace's status words), add the partials in slot order with the same
// shuffle tree, so every part gets the same factor, and scale their own h.
// The step id is the workgroup's epoch in the workspace plus one, stored
// back at the end: every call advances every workgroup's epoch by one, so
// all epochs agree and calls captured once into a graph need no host step.
#include "ar_device.hpp"
#include "ar_launch.hpp"

namespace ar {
namespace {

constexpr int kMaxBlock = 1024;
constexpr int kMaxWaves = kMaxBlock / kWave;

struct RmsParams {
    const u32x4* in[kMaxRanks];
    const u32x4* residual;
    const u32x4* weight;
    u32x4* residual_out;
    u32x4* out;
    size_t rows;
    uint32_t vecs;     // 16-byte vectors per row
    float hidden;      // elements per row (exact in fp32 up to 2^24)
    float eps;
};

// Elements of a 16-byte vector as fp32 and back (rounded once to T).
template <typename T> struct Vec;
template <> struct Vec<float> {
    static constexpr int E = 4;
    __device__ __forceinline__ static void widen(u32x4 v, float (&f)[4]) {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    }
    __device__ __forceinline__ static u32x4 narrow(const float (&f)[4]) {
        return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
    }
};
template <> struct Vec<bf16_t> {
    static constexpr int E = 8;
    __device__ __forceinline__ static void widen(u32x4 v, float (&f)[8]) {
        f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
        f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
    }
    __device__ __forceinline__ static u32x4 narrow(const float (&f)[8]) {
        return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                     pack_bf16x2(f[6], f[7])};
    }
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = kWave / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m);
    return x;
}

// Row accesses through raw buffer resources: the row's base is wavefront-
// uniform (scalar registers) and a lane's offset 32-bit, so no lane holds a
// 64-bit address per rank.  Inputs, residual and outputs are streamed
// (nontemporal); the weight, the same for every row, is read plainly.
constexpr int kCachePolicyNt = 2;  // the nt bit of the cache-policy operand
template <int kPolicy>
__device__ __forceinline__ u32x4 row_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, kPolicy);
}
__device__ __forceinline__ void row_store(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, int(off), 0, kCachePolicyNt);
}

template <typename T, int NR, int VPT>
__device__ __forceinline__ void rmsnorm_row(const RmsParams& p, size_t row, float (&part)[kMaxWaves],
                                            float& factor) {
    constexpr int E = Vec<T>::E;
    constexpr int RB = VPT == 1 || NR <= 8 ? NR : 8;  // loads in flight per vector
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & (kWave - 1);
    const uint32_t wave = tid / kWave;
    const uint32_t nwaves = blockDim.x / kWave;
    const size_t base = row * p.vecs;
    const uint32_t row_bytes = p.vecs * 16u;
    float h[VPT][E];
    u32x4 wv[VPT];  // the weight, loaded with the data: it does not wait for the row's factor
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const uint32_t v = tid + uint32_t(j) * blockDim.x;
        const bool valid = v < p.vecs;
        const uint32_t off = (valid ? v : 0u) * 16u;  // lanes past the row re-read its first vector
        wv[j] = row_load<0>(buffer_range(p.weight, row_bytes), off);
        const u32x4 rv = row_load<kCachePolicyNt>(buffer_range(p.residual + base, row_bytes), off);
        // the ranks in batches of RB loads, each folded (rank order) before
        // the next is issued: with several vectors per lane all n loads at
        // once would not fit in registers beside the kept h
        Acc<T> acc;
#pragma unroll
        for (int r0 = 0; r0 < NR; r0 += RB) {
            u32x4 x[RB];
#pragma unroll
            for (int i = 0; i < RB; ++i)
                if (r0 + i < NR) x[i] = row_load<kCachePolicyNt>(buffer_range(p.in[r0 + i] + base, row_bytes), off);
#pragma unroll
            for (int i = 0; i < RB; ++i)
                if (r0 + i < NR) acc.add(x[i]);
            __builtin_amdgcn_sched_barrier(0);
        }
        float res[E];
        Vec<T>::widen(rv, res);
#pragma unroll
        for (int e = 0; e < E; ++e) h[j][e] = acc.a[e] + res[e];
        if (valid) {
            row_store(buffer_range(p.residual_out + base, row_bytes), off, Vec<T>::narrow(h[j]));
#pragma unroll
            for (int e = 0; e < E; ++e) ss += h[j][e] * h[j][e];
        }
    }
    ss = wave_sum(ss);
    if (lane == 0) part[wave] = ss;
    __syncthreads();
    if (wave == 0) {
        float t = lane < nwaves ? part[lane] : 0.0f;
        t = wave_sum(t);
        if (lane == 0) factor = 1.0f / sqrtf(t / p.hidden + p.eps);
    }
    __syncthreads();
    const float f = factor;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const uint32_t v = tid + uint32_t(j) * blockDim.x;
        if (v < p.vecs) {
            float w[E];
            Vec<T>::widen(wv[j], w);
            float y[E];
#pragma unroll
            for (int e = 0; e < E; ++e) y[e] = (h[j][e] * f) * w[e];
            row_store(buffer_range(p.out + base, row_bytes), v * 16u, Vec<T>::narrow(y));
        }
    }
}

// kLoop: the workgroups stride over the rows (more rows than the grid);
// otherwise one row per workgroup.
template <typename T, int NR, int VPT, bool kLoop>
__global__ __launch_bounds__(kMaxBlock) void oneshot_rmsnorm_kernel(RmsParams p) {
    __shared__ float part[kMaxWaves];
    __shared__ float factor;
    if constexpr (kLoop) {
        for (size_t row = blockIdx.x; row < p.rows; row += gridDim.x) {
            rmsnorm_row<T, NR, VPT>(p, row, part, factor);
            __syncthreads();  // part and factor are rewritten by the next row
        }
    } else {
        rmsnorm_row<T, NR, VPT>(p, blockIdx.x, part, factor);
    }
}

// Cooperative path (few rows): workspace layout in 32-bit words, after the
// 32 status words: kCoopGrid epochs, then kCoopGrid 8-byte slots {partial
// sum of h^2 as fp32 bits, step id}.
constexpr uint32_t kEpochBase = kStatusWords;
constexpr uint32_t kSlotBase = kStatusWords + kCoopGrid;  // word index of slot 0 (8-byte aligned)

template <typename T, int NR>
__global__ __launch_bounds__(kWave) void oneshot_rmsnorm_coop_kernel(RmsParams p, uint32_t* ws, uint32_t parts,
                                                                     uint64_t timeout_ticks) {
    constexpr int E = Vec<T>::E;
    const uint32_t lane = threadIdx.x;
    const uint32_t g = blockIdx.x;
    // the epoch load goes out first and is used only after the data loads
    // are issued, so its round trip overlaps theirs
    const uint32_t epoch = flag_load_relaxed(ws + kEpochBase + g);
    const uint32_t row = g / parts, part = g - row * parts;
    uint32_t step = 0;
    if (row < p.rows) {
        const size_t base = size_t(row) * p.vecs;
        const uint32_t row_bytes = p.vecs * 16u;
        const uint32_t v = part * kWave + lane;
        const bool valid = v < p.vecs;
        const uint32_t off = (valid ? v : 0u) * 16u;
        const u32x4 wv = row_load<0>(buffer_range(p.weight, row_bytes), off);
        const u32x4 rv = row_load<kCachePolicyNt>(buffer_range(p.residual + base, row_bytes), off);
        u32x4 x[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) x[r] = row_load<kCachePolicyNt>(buffer_range(p.in[r] + base, row_bytes), off);
        Acc<T> acc;
#pragma unroll
        for (int r = 0; r < NR; ++r) acc.add(x[r]);
        step = __builtin_amdgcn_readfirstlane(epoch) + 1u;
        float res[E], h[E];
        Vec<T>::widen(rv, res);
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) h[e] = acc.a[e] + res[e];
        if (valid) {
            row_store(buffer_range(p.residual_out + base, row_bytes), off, Vec<T>::narrow(h));
#pragma unroll
            for (int e = 0; e < E; ++e) ss += h[e] * h[e];
        }
        ss = wave_sum(ss);
        // this part's slot: the value and the step in one 8-byte store
        const __amdgpu_buffer_rsrc_t slots = buffer_range(ws + kSlotBase, kCoopGrid * 8u);
        if (lane == 0)
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(ss), step}, slots, int(g * 8u), 0,
                                                  kCachePolicySc1);
        // the row's parts: lane q < parts polls slot row * parts + q
        const bool mine = lane < parts;
        const uint32_t soff = (row * parts + (mine ? lane : 0u)) * 8u;
        u32x2 sl = __builtin_amdgcn_raw_buffer_load_b64(slots, int(soff), 0, kCachePolicySc1);
        const uint64_t t0 = now_ticks();
        bool timed_out = false;
        while (true) {
            const uint64_t missing = ~wave_ballot(!mine || sl.y >= step) & wave_exec();
            if (missing == 0) break;
            if (now_ticks() - t0 > timeout_ticks) {
                if (lane == 0) report_timeout(ws, 4u, 0u, row);
                timed_out = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
            if (mine && sl.y < step) sl = __builtin_amdgcn_raw_buffer_load_b64(slots, int(soff), 0, kCachePolicySc1);
        }
        if (!timed_out) {
            // the same values in the same lanes in every part of the row: the
            // same total, the same factor
            const float total = wave_sum(mine ? __uint_as_float(sl.x) : 0.0f);
            const float f = 1.0f / sqrtf(total / p.hidden + p.eps);
            if (valid) {
                float w[E], y[E];
                Vec<T>::widen(wv, w);
#pragma unroll
                for (int e = 0; e < E; ++e) y[e] = (h[e] * f) * w[e];
                row_store(buffer_range(p.out + base, row_bytes), off, Vec<T>::narrow(y));
            }
        }
    }
    if (row >= p.rows) step = __builtin_amdgcn_readfirstlane(epoch) + 1u;
    if (lane == 0) flag_store_relaxed(ws + kEpochBase + g, step);
}

// Rows up to this many get a workgroup each; beyond, the grid strides.
constexpr size_t kRmsMaxGrid = size_t(1) << 20;

// The cooperative path where it measured faster than a workgroup per row:
// rows whose n + 1 input streams hold at least kCoopMinRowBytes (one
// compute unit pulling that much is the bottleneck; below it the slot
// exchange costs more than it saves) and at most kCoopMaxParts parts in all
// (n = 8 bf16, hidden 8192: 4.8 against 5.1 us at 1 row, 5.2 against 5.6 at
// 8, equal at 32, slower at 64; n = 16, 8 rows: 5.6 against 7.8; n = 2 and
// hidden 4096 at n = 8: slower).
constexpr uint32_t kCoopMinRowBytes = 128u << 10;
constexpr uint32_t kCoopMaxParts = 512;

template <typename T, int NR>
hipError_t launch_t(const RmsParams& p, uint32_t* ws, uint64_t timeout_ticks, hipStream_t s) {
    const uint32_t V = p.vecs;
    const uint32_t parts = (V + kWave - 1) / kWave;
    if (ws && p.rows * parts <= kCoopMaxParts && uint32_t(NR + 1) * V * 16u >= kCoopMinRowBytes) {
        hipLaunchKernelGGL((oneshot_rmsnorm_coop_kernel<T, NR>), dim3(kCoopGrid), dim3(kWave), 0, s, p, ws, parts,
                           timeout_ticks);
        return hipGetLastError();
    }
    // vectors per lane and workgroup size: every row fits one workgroup of
    // at most 1024 lanes with 1, 2 or 4 vectors each
    const int vpt = V <= 1024u ? 1 : (V <= 2048u ? 2 : 4);
    uint32_t block = (V + uint32_t(vpt) - 1) / uint32_t(vpt);
    block = (block + kWave - 1) / kWave * kWave;
    if (p.rows > kRmsMaxGrid) {
        // at least 2^20 rows within the size limit: a row is at most 16 KiB,
        // one vector per lane
        if (vpt != 1) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((oneshot_rmsnorm_kernel<T, NR, 1, true>), dim3(uint32_t(kRmsMaxGrid)), dim3(block), 0, s,
                           p);
    } else if (vpt == 1) {
        hipLaunchKernelGGL((oneshot_rmsnorm_kernel<T, NR, 1, false>), dim3(uint32_t(p.rows)), dim3(block), 0, s, p);
    } else if (vpt == 2) {
        hipLaunchKernelGGL((oneshot_rmsnorm_kernel<T, NR, 2, false>), dim3(uint32_t(p.rows)), dim3(block), 0, s, p);
    } else {
        hipLaunchKernelGGL((oneshot_rmsnorm_kernel<T, NR, 4, false>), dim3(uint32_t(p.rows)), dim3(block), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_oneshot_rmsnorm(const void* const* in, int n, const void* residual, const void* weight,
                                  void* residual_out, void* out, size_t rows, size_t hidden, float eps, int dtype,
                                  uint32_t* ws, uint64_t timeout_ticks, hipStream_t s) {
    RmsParams p{};
    for (int r = 0; r < n; ++r) p.in[r] = static_cast<const u32x4*>(in[r]);
    p.residual = static_cast<const u32x4*>(residual);
    p.weight = static_cast<const u32x4*>(weight);
    p.residual_out = static_cast<u32x4*>(residual_out);
    p.out = static_cast<u32x4*>(out);
    p.rows = rows;
    p.vecs = uint32_t(hidden * (dtype == 0 ? 4u : 2u) / 16u);
    p.hidden = float(hidden);
    p.eps = eps;
    return dispatch_ranks(n, [&](auto nr) {
        constexpr int NR = decltype(nr)::value;
        return dtype == 0 ? launch_t<float, NR>(p, ws, timeout_ticks, s) : launch_t<bf16_t, NR>(p, ws, timeout_ticks, s);
    });
}

}  // namespace ar
