// Two-shot all-reduce for gfx950: reduce-scatter of 1/n segments, a flag
// barrier in HBM, then an all-gather copy ("集合通信：NCCL 的算法、协议与推理框架的
// 定制 all-reduce", 算法, two-shot; "多 GPU 与 NCCL", 集合通信: all-reduce =
// reduce-scatter + all-gather; "0-custom-all-reduce", 实现 step 6 for the
// synchronisation between the phases).
//
// Work decomposition.  Segment r (m = numel/n elements, mvec 16-byte vectors)
// is cut into ktiles tiles of `tile` vectors (a multiple of 64; only a
// segment's last tile may be shorter).  The tiling depends on mvec only, so
// launches with different grids or rank ranges agree on it.
//   phase 1 item (r, t): sum tile t of segment r over every rank -> seg[r]
//   phase 2 item (ro, j, t): copy tile t of seg[j] into out[ro] at j*mvec
// Items are dealt to wavefronts round-robin; a wavefront walks its items as a
// flat list of 64-vector units (one vector per lane) and keeps U units of
// loads in flight before it adds or stores.
//
// Barrier.  Each tile (r, t) has a 32-bit arrival slot.  After its last
// phase-1 store a wavefront issues one agent-scope release fence (writes back
// its XCD's L2) and then stores `step` into the slot of every tile it
// produced.  In phase 2 a wavefront polls the slots of all its items, one
// slot per lane, until a ballot shows every lane sees slot >= step, then
// issues one agent-scope acquire fence (invalidates stale L2 lines) and
// copies.  Waits are bounded by a wall-clock budget; on expiry the first
// missing (rank, tile) goes to the status words and the wavefront skips its
// copies.  In the fused form the whole grid is co-resident (cooperative
// launch) and every wavefront finishes phase 1 before it polls, so every
// slot a poller needs is eventually written.
#include "ar_device.hpp"
#include "ar_launch.hpp"

namespace ar {
namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kCopyUnroll = 8;

struct TwoShotParams {
    const u32x4* in[kMaxRanks];
    u32x4* seg[kMaxRanks];
    u32x4* out[kMaxRanks];
    uint32_t* flags;
    uint64_t timeout_ticks;
    uint32_t mvec;
    uint32_t tile;
    uint32_t ktiles;
    uint32_t step;
    int r0, r1;
    int do_rs, do_ag;
};

template <typename T, int NR, int U>
__device__ __forceinline__ void reduce_scatter_phase(const TwoShotParams& p, uint32_t wave,
                                                     uint32_t nwaves, int lane) {
    const uint32_t R = uint32_t(p.r1 - p.r0);
    const uint32_t items = R * p.ktiles;
    if (wave >= items) return;
    const uint32_t my_items = (items - wave + nwaves - 1) / nwaves;
    const uint32_t upt = p.tile / kWave;
    const uint32_t my_units = my_items * upt;
    for (uint32_t q0 = 0; q0 < my_units; q0 += U) {
        u32x4 x[U][NR];
        uint32_t dst_idx[U];
        int dst_rank[U];
        bool valid[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t q = q0 + u;
            const uint32_t k = q / upt, sub = q - k * upt;
            const uint32_t it = wave + k * nwaves;
            const uint32_t r = uint32_t(p.r0) + it / p.ktiles;
            const uint32_t t = it % p.ktiles;
            const uint32_t idx = t * p.tile + sub * kWave + uint32_t(lane);
            valid[u] = (q < my_units) && (idx < p.mvec);
            dst_idx[u] = idx;
            dst_rank[u] = int(r);
            if (valid[u]) {
                const size_t src = size_t(r) * p.mvec + idx;
#pragma unroll
                for (int i = 0; i < NR; ++i) x[u][i] = ld_stream(p.in[i] + src);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (valid[u]) {
                Acc<T> acc;
#pragma unroll
                for (int i = 0; i < NR; ++i) acc.add(x[u][i]);
                st_stream(p.seg[dst_rank[u]] + dst_idx[u], acc.result());
            }
        }
    }
    // Publish: one release for everything this wavefront stored, then one
    // slot store per produced tile (lane k stores the slot of item k).
    fence_release_agent();
    __builtin_amdgcn_wave_barrier();
    uint32_t* slots = p.flags + kStatusWords;
    for (uint32_t k = uint32_t(lane); k < my_items; k += kWave) {
        const uint32_t it = wave + k * nwaves;
        const uint32_t r = uint32_t(p.r0) + it / p.ktiles;
        const uint32_t t = it % p.ktiles;
        flag_store_relaxed(slots + r * kSlotsPerRank + t, p.step);
    }
}

__device__ __forceinline__ void all_gather_phase(const TwoShotParams& p, int n, uint32_t wave,
                                                 uint32_t nwaves, int lane) {
    const uint32_t R = uint32_t(p.r1 - p.r0);
    const uint32_t per_out = uint32_t(n) * p.ktiles;
    const uint32_t items = R * per_out;
    if (wave >= items) return;
    const uint32_t my_items = (items - wave + nwaves - 1) / nwaves;
    const uint32_t* slots = p.flags + kStatusWords;

    // Wait for the slot of every item, 64 items (one per lane) at a time.
    for (uint32_t kb = 0; kb < my_items; kb += kWave) {
        const uint32_t k = kb + uint32_t(lane);
        const bool need = k < my_items;
        uint32_t j = 0, t = 0;
        if (need) {
            const uint32_t it = wave + k * nwaves;
            const uint32_t rem = it % per_out;
            j = rem / p.ktiles;
            t = rem % p.ktiles;
        }
        const uint32_t* slot = slots + j * kSlotsPerRank + t;
        const uint64_t t0 = now_ticks();
        while (true) {
            const bool ok = !need || flag_load_relaxed(slot) >= p.step;
            const uint64_t missing = ~wave_ballot(ok) & wave_exec();
            if (missing == 0) break;
            if (now_ticks() - t0 > p.timeout_ticks) {
                const int bad_lane = __ffsll((unsigned long long)missing) - 1;
                const uint32_t bj = __shfl(j, bad_lane);
                const uint32_t bt = __shfl(t, bad_lane);
                if (lane == 0) report_timeout(p.flags, 1u, bj, bt);
                return;  // skip every copy of this wavefront
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    fence_acquire_agent();

    const uint32_t upt = p.tile / kWave;
    const uint32_t my_units = my_items * upt;
    for (uint32_t q0 = 0; q0 < my_units; q0 += kCopyUnroll) {
        u32x4 x[kCopyUnroll];
        u32x4* dst[kCopyUnroll];
        bool valid[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const uint32_t q = q0 + u;
            const uint32_t k = q / upt, sub = q - k * upt;
            const uint32_t it = wave + k * nwaves;
            const uint32_t ro = uint32_t(p.r0) + it / per_out;
            const uint32_t rem = it % per_out;
            const uint32_t j = rem / p.ktiles;
            const uint32_t t = rem % p.ktiles;
            const uint32_t idx = t * p.tile + sub * kWave + uint32_t(lane);
            valid[u] = (q < my_units) && (idx < p.mvec);
            if (valid[u]) {
                x[u] = ld_plain(p.seg[j] + idx);
                dst[u] = p.out[ro] + size_t(j) * p.mvec + idx;
            }
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u)
            if (valid[u]) st_stream(dst[u], x[u]);
    }
}

template <typename T, int NR, int U>
__global__ __launch_bounds__(kBlock) void twoshot_kernel(TwoShotParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t wave = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    const uint32_t nwaves = gridDim.x * kWavesPerBlock;
    if (p.do_rs) reduce_scatter_phase<T, NR, U>(p, wave, nwaves, lane);
    if (p.do_ag) all_gather_phase(p, NR, wave, nwaves, lane);
}

template <typename T, int NR>
hipError_t launch_t(const TwoShotRequest& rq, hipStream_t s) {
    constexpr int U = NR <= 4 ? 4 : (NR <= 8 ? 2 : 1);
    DeviceInfo info;
    hipError_t e = device_info(&info);
    if (e != hipSuccess) return e;

    TwoShotParams p{};
    for (int r = 0; r < NR; ++r) {
        p.in[r] = rq.in ? static_cast<const u32x4*>(rq.in[r]) : nullptr;
        p.seg[r] = static_cast<u32x4*>(rq.seg[r]);
        p.out[r] = (rq.out && r >= rq.r0 && r < rq.r1) ? static_cast<u32x4*>(rq.out[r]) : nullptr;
    }
    const size_t seg_bytes = rq.numel / size_t(NR) * size_t(elem<T>::bytes);
    p.mvec = uint32_t(seg_bytes / 16);
    const uint32_t per_slot = (p.mvec + kSlotsPerRank - 1) / kSlotsPerRank;  // vectors per slot at least
    p.tile = ((per_slot + kWave - 1) / kWave) * kWave;
    if (p.tile == 0) p.tile = kWave;
    p.ktiles = (p.mvec + p.tile - 1) / p.tile;
    p.flags = rq.flags;
    p.timeout_ticks = rq.timeout_ticks;
    p.step = rq.step;
    p.r0 = rq.r0;
    p.r1 = rq.r1;
    p.do_rs = rq.do_rs;
    p.do_ag = rq.do_ag;

    auto kern = twoshot_kernel<T, NR, U>;
    if (rq.do_rs && rq.do_ag) {
        int per_cu = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kBlock, 0);
        if (e != hipSuccess) return e;
        if (per_cu < 1) return hipErrorCooperativeLaunchTooLarge;
        if (per_cu > 2) per_cu = 2;
        const dim3 grid(uint32_t(info.cu_count * per_cu)), block(kBlock);
        void* args[] = {&p};
        return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kern), grid, block, args, 0, s);
    }
    // Split launches: size the grid to the work, at most two blocks per CU.
    const uint32_t R = uint32_t(rq.r1 - rq.r0);
    const uint32_t items = rq.do_rs ? R * p.ktiles : R * uint32_t(NR) * p.ktiles;
    uint32_t grid = (items + kWavesPerBlock - 1) / kWavesPerBlock;
    const uint32_t cap = uint32_t(info.cu_count) * 2u;
    if (grid > cap) grid = cap;
    if (grid == 0) grid = 1;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kBlock), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_twoshot(const TwoShotRequest& rq, hipStream_t s) {
    return dispatch_ranks(rq.n, [&](auto nr) {
        constexpr int NR = decltype(nr)::value;
        return rq.dtype == 0 ? launch_t<float, NR>(rq, s) : launch_t<bf16_t, NR>(rq, s);
    });
}

}  // namespace ar
