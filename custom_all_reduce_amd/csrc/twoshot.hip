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
//   phase 1 item (r, t): sum tile t of segment r over every rank -> seg[r];
//                        in the fused form also -> out[r] at r*mvec (rank r's
//                        own segment of its all-gather, from registers)
//   phase 2 item (ro, j, t): copy tile t of seg[j] into out[ro] at j*mvec, for
//                        every j (split form) or every j != ro (fused form)
// Items are dealt to wavefronts round-robin (phase 2 starting after the
// wavefronts that have phase-1 items); a wavefront walks its items as a flat
// list of 64-vector units (one vector per lane) and keeps U units of loads in
// flight before it adds or stores.  A unit's item, rank and tile come from
// divisions by launch-invariant values, done as multiply-high and shift with
// multipliers computed on the host (fastdiv.hpp).
//
// Barrier.  Each tile (r, t) has a 32-bit arrival slot.  Segments are
// written and read with device-coherent (sc1) accesses, so after its last
// phase-1 store a wavefront only waits for its stores to complete and then
// stores `step` into the slot of every tile it produced.  In phase 2 a
// wavefront polls the slots of all its items, one slot per lane, until a
// ballot shows every lane sees slot >= step, then copies.  (An agent-scope
// release/acquire fence pair per wavefront would write back and invalidate
// a whole XCD L2 each time; measured, that costs several times the copy.)
// Waits are bounded by a wall-clock budget; on expiry the first missing
// (rank, tile) goes to the status words and the wavefront skips its copies.  In the fused form the grid is no larger than what the device
// holds at once (occupancy-checked, persistent), and every wavefront finishes
// phase 1 before it polls, so every slot a poller needs is eventually written
// while nothing else occupies the CUs; if something does, the bounded wait
// turns the stall into a reported timeout instead of a hang.
//
// Step ids.  An explicit step id comes with the call.  With step 0 (auto) it
// comes from the flag region instead, so a launch captured once into a graph
// gets a fresh id on every replay.  Every wavefront keeps its own copy of
// each rank's epoch (the id of the rank's last reduce-scatter) after the
// arrival slots; auto launches always use the same grid, so all copies move
// in step.  A wavefront loads its copies right behind the first loads of
// its first phase (reduce-scatter data or all-gather slot polls; on their
// own if it has no work) and, if the launch reduces, stores epoch + 1 back
// at its end.  No other wavefront touches those copies, so there is no
// counter, atomic or barrier.  A split all-gather uses the current epoch,
// the id of the reduce-scatter before it.
#include <mutex>

#include "ar_device.hpp"
#include "ar_launch.hpp"
#include "fastdiv.hpp"

namespace ar {
namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kCopyUnroll = 4;
// One-rank share kernel (explicit step ids): 64-vector units per all-gather
// wavefront; reduce-scatter units in flight per wavefront by rank count
// (NR loads each; more units per wavefront only where NR loads are few);
// 4-wavefront workgroups from this many wavefronts per CU on, one-wavefront
// workgroups below.  Measured on MI355X, n = 8 bf16: 4-wave workgroups
// 6.07 us at 8 MiB per rank against 6.51 with one wave (dispatching 8192
// one-wave workgroups alone costs 2.8 us), one wave 3.66 us at 1 MiB
// against 3.83.  Reduce-scatter units in flight at 64 MiB per rank: n = 2,
// 4 units 30.6 us against 36.2 with one; n = 8, 1 unit 31.4 against 32.6
// with two; n = 16, 1 unit 32.1 against 38.8 with two.
constexpr int kShareChunk = 1;
constexpr int kShareWideMinWavesPerCu = 16;
template <int NR> constexpr int share_rs_unroll() { return NR <= 4 ? 4 : (NR <= 6 ? 2 : 1); }

// n / d for the launch-invariant divisors of the tiling (FastDiv, built on
// the host by make_fastdiv): a multiply-high, an add and a shift.
__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) { return (__umulhi(n, f.mlo) + n) >> f.s; }

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
    int auto_step;
    int r0, r1;
    int do_rs, do_ag;
    FastDiv div_upt;      // units per tile
    FastDiv div_ktiles;   // tiles per segment
    FastDiv div_per_out;  // all-gather items per output rank
    uint32_t ag_chunks;   // one-rank share kernel: all-gather chunks per segment
    FastDiv div_chunks;   // ... as a divisor
};

template <typename T, int NR, int U, bool kLL>
__device__ __forceinline__ bool reduce_scatter_phase(const TwoShotParams& p, const uint32_t* epoch,
                                                     uint32_t& epoch_lane, uint32_t wave, uint32_t nwaves,
                                                     int lane) {
    const uint32_t R = uint32_t(p.r1 - p.r0);
    const uint32_t items = R * p.ktiles;
    if (wave >= items) return false;
    // Auto step ids: lane l < R loads this wavefront's epoch copy of rank
    // r0 + l right behind the first unit's loads, so that it travels with
    // them instead of costing a round trip of its own before them.
    const bool load_epoch = p.auto_step && uint32_t(lane) < R;
    const uint32_t my_items = (items - wave + nwaves - 1) / nwaves;
    const uint32_t upt = p.tile / kWave;
    const uint32_t my_units = my_items * upt;
    const u32x4* in[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) in[i] = p.in[i];
    for (uint32_t q0 = 0; q0 < my_units; q0 += U) {
        // Unit q = 64 consecutive vectors of one tile.  wave, q0 and hence the
        // tile and rank of every unit are wavefront-uniform (scalar); only the
        // vector index carries the lane.  Units past the end re-read unit q0's
        // tile start and are discarded, so the U * NR loads issue unbroken.
        u32x4 x[U][NR];
        uint32_t dst_idx[U];
        uint32_t dst_rank[U];
        uint32_t dst_t0[U];  // first vector of the unit's tile (wavefront-uniform)
        bool valid[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool unit_ok = q0 + u < my_units;
            const uint32_t q = unit_ok ? q0 + u : q0;
            const uint32_t k = fdiv(q, p.div_upt), sub = q - k * upt;
            const uint32_t it = wave + k * nwaves;
            const uint32_t rr = fdiv(it, p.div_ktiles);
            const uint32_t r = uint32_t(p.r0) + rr;
            const uint32_t t = it - rr * p.ktiles;
            const uint32_t idx = t * p.tile + sub * kWave + uint32_t(lane);
            valid[u] = unit_ok && idx < p.mvec;
            dst_idx[u] = idx;
            dst_rank[u] = r;
            dst_t0[u] = t * p.tile;
            const size_t src = size_t(r) * p.mvec + (valid[u] ? idx : t * p.tile);
#pragma unroll
            for (int i = 0; i < NR; ++i) x[u][i] = ld_stream(in[i] + src);
        }
        if (q0 == 0 && load_epoch) epoch_lane = flag_load_relaxed(epoch + lane);
        __builtin_amdgcn_sched_barrier(0);  // every load ahead of the first add
#pragma unroll
        for (int u = 0; u < U; ++u) {
            Acc<T> acc;
#pragma unroll
            for (int i = 0; i < NR; ++i) acc.add(x[u][i]);
            const u32x4 v = acc.result();
            // LL lines carry the step id of the unit's rank (every lane
            // active here: auto ids are read from lane r - r0)
            uint32_t lstep = p.step;
            if constexpr (kLL)
                if (p.auto_step) lstep = __shfl(epoch_lane + 1u, int(dst_rank[u]) - p.r0);
            if (valid[u]) {
                // the tile of seg[r] as one wavefront-uniform buffer range
                const uint32_t t0 = dst_t0[u];
                const uint32_t tile_bytes = min(p.tile, p.mvec - t0) * 16u;
                if constexpr (kLL) {
                    // four LL lines: each 4 data bytes beside the step id
                    const __amdgpu_buffer_rsrc_t rs = buffer_range(p.seg[dst_rank[u]] + 2 * t0, 2 * tile_bytes);
                    st_coherent(rs, (dst_idx[u] - t0) * 32u, u32x4{v.x, lstep, v.y, lstep});
                    st_coherent(rs, (dst_idx[u] - t0) * 32u + 16u, u32x4{v.z, lstep, v.w, lstep});
                } else {
                    st_coherent(buffer_range(p.seg[dst_rank[u]] + t0, tile_bytes), (dst_idx[u] - t0) * 16u, v);
                }
                // fused form: rank r's own segment of its output comes straight
                // from registers (the all-gather copy of seg[r] into out[r])
                if (p.do_ag) st_stream(p.out[dst_rank[u]] + size_t(dst_rank[u]) * p.mvec + dst_idx[u], v);
            }
        }
    }
    // LL segments carry their flags: nothing to wait for or publish.
    if constexpr (kLL) return true;
    // Publish: wait until this wavefront's coherent segment stores have
    // completed, then one slot store per produced tile (lane k stores the
    // slot of item k; the loop runs with every lane active so the step id
    // of the item's rank can be read from lane r - r0).
    wait_stores();
    __builtin_amdgcn_wave_barrier();
    uint32_t* slots = p.flags + kStatusWords;
    for (uint32_t kb = 0; kb < my_items; kb += kWave) {
        const uint32_t k = kb + uint32_t(lane);
        const uint32_t it = wave + (k < my_items ? k : 0u) * nwaves;
        const uint32_t rr = fdiv(it, p.div_ktiles);
        const uint32_t r = uint32_t(p.r0) + rr;
        const uint32_t t = it - rr * p.ktiles;
        const uint32_t st = __shfl(p.auto_step ? epoch_lane + 1u : p.step, int(r) - p.r0);
        if (k < my_items) flag_store_relaxed(slots + r * kSlotsPerRank + t, st);
    }
    return true;
}

// Source segment of the jj-th all-gather copy into out[ro]: every segment in
// order, or, when the reduce-scatter of the same launch already wrote out[ro]'s
// own segment, every segment but ro's.
// Integer arithmetic only (jj, ro < 2^31: the sign bit of ro - jj - 1 is
// jj >= ro), so that wavefront-uniform operands stay in scalar registers.
__device__ __forceinline__ uint32_t ag_source(uint32_t jj, uint32_t ro, bool skip_own) {
    return jj + (((ro - jj - 1u) >> 31) & uint32_t(skip_own));
}

// Unit q (64 consecutive vectors, one per lane) of a wavefront's all-gather
// list: the output rank ro, the source segment j, the tile t, the unit's
// place sub in its tile, and this lane's vector index idx in the segment.
// Every field but idx is wavefront-uniform.
struct AgUnit {
    uint32_t ro, j, t, sub, idx;
};

__device__ __forceinline__ AgUnit ag_unit(const TwoShotParams& p, uint32_t per_out, bool skip_own, uint32_t wave,
                                          uint32_t nwaves, uint32_t upt, uint32_t q, int lane) {
    AgUnit a;
    const uint32_t k = fdiv(q, p.div_upt);
    a.sub = q - k * upt;
    const uint32_t it = wave + k * nwaves;
    const uint32_t oo = fdiv(it, p.div_per_out);
    a.ro = uint32_t(p.r0) + oo;
    const uint32_t rem = it - oo * per_out;
    const uint32_t jj = fdiv(rem, p.div_ktiles);
    a.j = ag_source(jj, a.ro, skip_own);
    a.t = rem - jj * p.ktiles;
    a.idx = a.t * p.tile + a.sub * kWave + uint32_t(lane);
    return a;
}

// With auto step ids and no epoch loaded yet (have_epoch false), the
// wavefront loads its epoch copies right behind its first slot poll, so the
// two loads share one round trip; the step id a slot must reach is epoch +
// step_inc.
__device__ __forceinline__ void all_gather_phase(const TwoShotParams& p, const uint32_t* epoch,
                                                 uint32_t& epoch_lane, bool& have_epoch, uint32_t step_inc,
                                                 int n, uint32_t wave, uint32_t nwaves, int lane) {
    const uint32_t R = uint32_t(p.r1 - p.r0);
    const bool skip_own = p.do_rs != 0;
    const uint32_t per_out = uint32_t(skip_own ? n - 1 : n) * p.ktiles;
    const uint32_t items = R * per_out;
    if (wave >= items) return;
    const uint32_t my_items = (items - wave + nwaves - 1) / nwaves;
    const uint32_t* slots = p.flags + kStatusWords;

    // Wait for the slot of every item, 64 items (one per lane) at a time.
    for (uint32_t kb = 0; kb < my_items; kb += kWave) {
        const uint32_t k = kb + uint32_t(lane);
        const bool need = k < my_items;
        // every lane active here: the output rank's step id is read from
        // lane ro - r0
        const uint32_t it = wave + (need ? k : 0u) * nwaves;
        const uint32_t oo = fdiv(it, p.div_per_out);
        const uint32_t ro = uint32_t(p.r0) + oo;
        uint32_t j = 0, t = 0;
        if (need) {
            const uint32_t rem = it - oo * per_out;
            const uint32_t jj = fdiv(rem, p.div_ktiles);
            j = ag_source(jj, ro, skip_own);
            t = rem - jj * p.ktiles;
        }
        const uint32_t* slot = slots + j * kSlotsPerRank + t;
        uint32_t seen = need ? flag_load_relaxed(slot) : 0u;
        if (!have_epoch) {
            if (uint32_t(lane) < R) epoch_lane = flag_load_relaxed(epoch + lane);
            have_epoch = true;
        }
        const uint32_t want = __shfl(p.auto_step ? epoch_lane + step_inc : p.step, int(ro) - p.r0);
        const uint64_t t0 = now_ticks();
        while (true) {
            const bool ok = !need || seen >= want;
            const uint64_t missing = ~wave_ballot(ok) & wave_exec();
            if (missing == 0) break;
            if (now_ticks() - t0 > p.timeout_ticks) {
                const int bad_lane = __ffsll((unsigned long long)missing) - 1;
                const uint32_t bj = __shfl(j, bad_lane);
                const uint32_t bt = __shfl(t, bad_lane);
                if (lane == 0) report_timeout(p.flags, kPhaseTwoshotAg, bj, bt);
                return;  // skip every copy of this wavefront
            }
            __builtin_amdgcn_s_sleep(1);
            if (need) seen = flag_load_relaxed(slot);
        }
    }
    const uint32_t upt = p.tile / kWave;
    const uint32_t my_units = my_items * upt;
    for (uint32_t q0 = 0; q0 < my_units; q0 += kCopyUnroll) {
        u32x4 x[kCopyUnroll];
        u32x4* dst[kCopyUnroll];
        bool valid[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const bool unit_ok = q0 + u < my_units;
            const uint32_t q = unit_ok ? q0 + u : q0;
            const AgUnit a = ag_unit(p, per_out, skip_own, wave, nwaves, upt, q, lane);
            valid[u] = unit_ok && a.idx < p.mvec;
            const uint32_t t0 = a.t * p.tile;
            const uint32_t tile_bytes = min(p.tile, p.mvec - t0) * 16u;
            x[u] = ld_coherent(buffer_range(p.seg[a.j] + t0, tile_bytes), (a.sub * kWave + uint32_t(lane)) * 16u);
            dst[u] = p.out[a.ro] + size_t(a.j) * p.mvec + a.idx;
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u)
            if (valid[u]) st_stream(dst[u], x[u]);
    }
}

// LL all-gather: the segments are LL wires (each 4 data bytes beside the
// step id in one 8-byte line), so a copy checks the flags of the lines it
// reads instead of waiting on slots first: one memory round trip instead of
// two.  A lane reads 32 wire bytes (16 data bytes) per unit with coherent
// loads; one ballot decides whether every flag of the wavefront's units has
// reached the step.  If not, the lanes re-read the units that are behind
// until they are there or the wall-clock budget runs out (reported: phase 1,
// segment, tile).  With auto step ids a unit waits for its output rank's
// epoch + 1 (the id that rank's reduce-scatter of this launch writes); a
// wavefront without reduce-scatter items loads its epoch copies with its
// first unit's loads.
__device__ __forceinline__ void all_gather_ll_phase(const TwoShotParams& p, const uint32_t* epoch,
                                                    uint32_t& epoch_lane, bool& have_epoch, int n, uint32_t wave,
                                                    uint32_t nwaves, int lane) {
    const uint32_t R = uint32_t(p.r1 - p.r0);
    const bool skip_own = p.do_rs != 0;
    const uint32_t per_out = uint32_t(skip_own ? n - 1 : n) * p.ktiles;
    const uint32_t items = R * per_out;
    if (wave >= items) return;
    const uint32_t my_items = (items - wave + nwaves - 1) / nwaves;
    const uint32_t upt = p.tile / kWave;
    const uint32_t my_units = my_items * upt;
    for (uint32_t q0 = 0; q0 < my_units; q0 += kCopyUnroll) {
        u32x4 a[kCopyUnroll], b[kCopyUnroll];
        u32x4* dst[kCopyUnroll];
        __amdgpu_buffer_rsrc_t rs[kCopyUnroll];
        uint32_t off[kCopyUnroll], seg_of[kCopyUnroll], tile_of[kCopyUnroll], out_of[kCopyUnroll];
        bool valid[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const bool unit_ok = q0 + u < my_units;
            const uint32_t q = unit_ok ? q0 + u : q0;
            const AgUnit au = ag_unit(p, per_out, skip_own, wave, nwaves, upt, q, lane);
            valid[u] = unit_ok && au.idx < p.mvec;
            const uint32_t t0 = au.t * p.tile;
            const uint32_t tile_bytes = min(p.tile, p.mvec - t0) * 16u;
            rs[u] = buffer_range(p.seg[au.j] + 2 * t0, 2 * tile_bytes);
            off[u] = (au.sub * kWave + uint32_t(lane)) * 32u;
            a[u] = ld_coherent(rs[u], off[u]);
            b[u] = ld_coherent(rs[u], off[u] + 16u);
            dst[u] = p.out[au.ro] + size_t(au.j) * p.mvec + au.idx;
            seg_of[u] = au.j;
            tile_of[u] = au.t;
            out_of[u] = au.ro;
        }
        if (!have_epoch) {
            if (uint32_t(lane) < R) epoch_lane = flag_load_relaxed(epoch + lane);
            have_epoch = true;
        }
        __builtin_amdgcn_sched_barrier(0);  // every load ahead of the first use
        uint32_t want[kCopyUnroll];
        bool behind = false;
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            want[u] = p.auto_step ? __shfl(epoch_lane + 1u, int(out_of[u]) - p.r0) : p.step;
            const uint32_t f = min(min(a[u].y, a[u].w), min(b[u].y, b[u].w));
            behind |= valid[u] && f < want[u];
        }
        if (wave_ballot(behind) != 0) {
            const uint64_t t_start = now_ticks();
            while (true) {
                bool good = true;
                uint32_t bad_j = 0, bad_t = 0;
#pragma unroll
                for (int u = 0; u < kCopyUnroll; ++u) {
                    const uint32_t f = min(min(a[u].y, a[u].w), min(b[u].y, b[u].w));
                    if (valid[u] && f < want[u]) {
                        a[u] = ld_coherent(rs[u], off[u]);
                        b[u] = ld_coherent(rs[u], off[u] + 16u);
                        const uint32_t g = min(min(a[u].y, a[u].w), min(b[u].y, b[u].w));
                        if (g < want[u] && good) { good = false; bad_j = seg_of[u]; bad_t = tile_of[u]; }
                    }
                }
                const uint64_t missing = ~wave_ballot(good) & wave_exec();
                if (missing == 0) break;
                if (now_ticks() - t_start > p.timeout_ticks) {
                    const int bl = __ffsll((unsigned long long)missing) - 1;
                    if (lane == bl) report_timeout(p.flags, kPhaseTwoshotAg, bad_j, bad_t);
                    return;  // skip every remaining copy of this wavefront
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u)
            if (valid[u]) st_stream(dst[u], u32x4{a[u].x, a[u].z, b[u].x, b[u].z});
    }
}

template <typename T, int NR, int U, bool kLL>
__global__ __launch_bounds__(kBlock) void twoshot_kernel(TwoShotParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    // the wavefront index, made explicitly uniform so item arithmetic is scalar
    const uint32_t wave = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerBlock + threadIdx.x / kWave);
    const uint32_t nwaves = gridDim.x * kWavesPerBlock;
    // Lane l < r1 - r0 holds the step id of rank r0 + l (this wavefront's
    // epoch copy in auto mode).
    const uint32_t R = uint32_t(p.r1 - p.r0);
    // this wavefront's epoch copies, one word per rank (lane l: rank r0 + l)
    uint32_t* epoch = p.flags + kStatusWords + NR * kSlotsPerRank + size_t(wave) * NR + p.r0;
    // Auto step ids: the epoch copies are loaded by whichever phase runs
    // first in this wavefront, together with that phase's first loads (or
    // on their own at the end if the wavefront has no work), and epoch + 1
    // is stored back at the end if the launch reduces.
    uint32_t epoch_lane = 0;
    bool have_epoch = !p.auto_step;
    if (p.do_rs && reduce_scatter_phase<T, NR, U, kLL>(p, epoch, epoch_lane, wave, nwaves, lane)) have_epoch = true;
    if (p.do_ag) {
        // In the fused form the all-gather items are dealt starting after the
        // wavefronts that hold reduce-scatter items, so that when the grid has
        // a wavefront per item the two phases run side by side instead of one
        // after the other in the same wavefronts.
        const uint32_t rs_busy = p.do_rs ? min(R * p.ktiles, nwaves) : 0u;
        const uint32_t ag_wave = wave >= rs_busy ? wave - rs_busy : wave + (nwaves - rs_busy);
        if constexpr (kLL) all_gather_ll_phase(p, epoch, epoch_lane, have_epoch, NR, ag_wave, nwaves, lane);
        else all_gather_phase(p, epoch, epoch_lane, have_epoch, p.do_rs ? 1u : 0u, NR, ag_wave, nwaves, lane);
    }
    if (p.auto_step && p.do_rs) {
        if (!have_epoch && uint32_t(lane) < R) epoch_lane = flag_load_relaxed(epoch + lane);
        if (uint32_t(lane) < R) flag_store_relaxed(epoch + lane, epoch_lane + 1u);
    }
}

// One GPU's share, [me, me+1) with an explicit step id: a grid sized to the
// work, not a persistent one.  The all-gather copies only the peers'
// segments (rank me's own comes from the reduce-scatter's registers), and
// those were published by the peers' launches, not by this one, so no
// wavefront of this launch waits on another and the grid may be as large as
// the work; workgroups the device cannot hold yet simply start later (the
// dispatcher starting a fresh wavefront measured faster than wavefronts
// looping over several items).
//   wavefronts [0, ktiles)     reduce-scatter: one tile of segment me each,
//                              then its slot (after the tile's stores); with
//                              kLL the tile goes out as LL lines carrying the
//                              step id, with no store wait and no slot
//   wavefronts [ktiles, ...)   all-gather: one chunk of C 64-vector units of
//                              one peer segment each -- poll the chunk's
//                              slots, then every load of the chunk, then its
//                              stores (kLL: load the chunk's lines, check
//                              their flags, re-read the ones behind)
// The reduce-scatter wavefronts come first in the grid, so they are
// dispatched first: a wavefront that waits on a late peer never keeps this
// launch's own reduce-scatter (which that peer may be waiting for) from
// starting.
template <typename T, int NR, int C, int WB, int RU, bool kLL>
__global__ __launch_bounds__(kWave * WB) void twoshot_share_kernel(TwoShotParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(blockIdx.x * WB + threadIdx.x / kWave);
    const uint32_t me = uint32_t(p.r0);
    uint32_t* slots = p.flags + kStatusWords;
    if (wave < p.ktiles) {
        const uint32_t t0 = wave * p.tile;
        const uint32_t tv = min(p.tile, p.mvec - t0);  // vectors in this tile
        const uint32_t units = (tv + kWave - 1) / kWave;
        // the tile of seg[me]: 16-byte vectors, or as LL lines 32 wire bytes each
        const __amdgpu_buffer_rsrc_t rs = buffer_range(p.seg[me] + (kLL ? 2u : 1u) * t0, tv * (kLL ? 32u : 16u));
        const uint32_t st = p.step;
        u32x4* own = p.out[me] + size_t(me) * p.mvec + t0;
        const size_t base = size_t(me) * p.mvec + t0;
        const u32x4* in[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) in[i] = p.in[i];
        // RU whole units in flight while at least that many are left (every
        // load unconditional), then one unit at a time, the partial last one
        // with its lanes past the tile clamped
        const uint32_t whole = tv / kWave;
        uint32_t u = 0;
        for (; u + RU <= whole; u += RU) {
            u32x4 x[RU][NR];
#pragma unroll
            for (int w = 0; w < RU; ++w)
#pragma unroll
                for (int i = 0; i < NR; ++i) x[w][i] = ld_stream(in[i] + base + (u + w) * kWave + uint32_t(lane));
            __builtin_amdgcn_sched_barrier(0);  // every load ahead of the first add
#pragma unroll
            for (int w = 0; w < RU; ++w) {
                Acc<T> acc;
#pragma unroll
                for (int i = 0; i < NR; ++i) acc.add(x[w][i]);
                const u32x4 r = acc.result();
                const uint32_t v = (u + w) * kWave + uint32_t(lane);
                if constexpr (kLL) {
                    st_coherent(rs, v * 32u, u32x4{r.x, st, r.y, st});
                    st_coherent(rs, v * 32u + 16u, u32x4{r.z, st, r.w, st});
                } else {
                    st_coherent(rs, v * 16u, r);
                }
                st_stream(own + v, r);
            }
        }
        for (; u < units; ++u) {
            const uint32_t v = u * kWave + uint32_t(lane);
            const bool valid = v < tv;
            const size_t src = base + (valid ? v : 0u);
            u32x4 x[NR];
#pragma unroll
            for (int i = 0; i < NR; ++i) x[i] = ld_stream(in[i] + src);
            __builtin_amdgcn_sched_barrier(0);  // every load ahead of the first add
            Acc<T> acc;
#pragma unroll
            for (int i = 0; i < NR; ++i) acc.add(x[i]);
            const u32x4 r = acc.result();
            if (valid) {
                if constexpr (kLL) {
                    st_coherent(rs, v * 32u, u32x4{r.x, st, r.y, st});
                    st_coherent(rs, v * 32u + 16u, u32x4{r.z, st, r.w, st});
                } else {
                    st_coherent(rs, v * 16u, r);
                }
                st_stream(own + v, r);
            }
        }
        // LL lines carry their flags: nothing to wait for or publish
        if constexpr (kLL) return;
        // publish the tile once its segment stores have completed
        wait_stores();
        if (lane == 0) flag_store_relaxed(slots + me * kSlotsPerRank + wave, p.step);
        return;
    }
    const uint32_t c = wave - p.ktiles;
    const uint32_t jj = fdiv(c, p.div_chunks);
    if (jj >= uint32_t(NR - 1)) return;  // past the last chunk (grid rounding)
    const uint32_t k = c - jj * p.ag_chunks;
    const uint32_t j = ag_source(jj, me, true);
    const uint32_t v0 = k * uint32_t(C * kWave);
    const uint32_t vend = min(v0 + uint32_t(C * kWave), p.mvec);
    // the tiles the chunk covers (tiles are whole 64-vector units): at most C
    const uint32_t tf = fdiv(k * uint32_t(C), p.div_upt);
    u32x4* dst = p.out[me] + size_t(j) * p.mvec + v0;
    if constexpr (kLL) {
        // LL segment lines: load the chunk's wire bytes (32 per vector), check
        // their flags with one ballot, re-read the units that are behind
        const __amdgpu_buffer_rsrc_t rs = buffer_range(p.seg[j] + 2u * v0, (vend - v0) * 32u);
        u32x4 a[C], b[C];
#pragma unroll
        for (int u = 0; u < C; ++u) {
            const uint32_t off = (uint32_t(u * kWave) + uint32_t(lane)) * 32u;
            a[u] = ld_coherent(rs, off);
            b[u] = ld_coherent(rs, off + 16u);
        }
        __builtin_amdgcn_sched_barrier(0);  // every load ahead of the first use
        bool behind = false;
#pragma unroll
        for (int u = 0; u < C; ++u) {
            const bool valid = v0 + uint32_t(u * kWave) + uint32_t(lane) < vend;
            behind |= valid && min(min(a[u].y, a[u].w), min(b[u].y, b[u].w)) < p.step;
        }
        if (wave_ballot(behind) != 0) {
            const uint64_t t_start = now_ticks();
            while (true) {
                bool good = true;
                uint32_t bad_u = 0;
#pragma unroll
                for (int u = 0; u < C; ++u) {
                    const bool valid = v0 + uint32_t(u * kWave) + uint32_t(lane) < vend;
                    if (valid && min(min(a[u].y, a[u].w), min(b[u].y, b[u].w)) < p.step) {
                        const uint32_t off = (uint32_t(u * kWave) + uint32_t(lane)) * 32u;
                        a[u] = ld_coherent(rs, off);
                        b[u] = ld_coherent(rs, off + 16u);
                        if (min(min(a[u].y, a[u].w), min(b[u].y, b[u].w)) < p.step && good) {
                            good = false;
                            bad_u = uint32_t(u);
                        }
                    }
                }
                const uint64_t missing = ~wave_ballot(good) & wave_exec();
                if (missing == 0) break;
                if (now_ticks() - t_start > p.timeout_ticks) {
                    const int bl = __ffsll((unsigned long long)missing) - 1;
                    if (lane == bl) report_timeout(p.flags, kPhaseTwoshotAg, j, fdiv(k * uint32_t(C) + bad_u, p.div_upt));
                    return;  // skip the chunk's copies
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
#pragma unroll
        for (int u = 0; u < C; ++u) {
            const uint32_t v = uint32_t(u * kWave) + uint32_t(lane);
            if (v0 + v < vend) st_stream(dst + v, u32x4{a[u].x, a[u].z, b[u].x, b[u].z});
        }
    } else {
        const uint32_t tl = fdiv((vend - 1u) / kWave, p.div_upt);
        const bool need = uint32_t(lane) <= tl - tf;
        const uint32_t* slot = slots + j * kSlotsPerRank + tf + (need ? uint32_t(lane) : 0u);
        uint32_t seen = need ? flag_load_relaxed(slot) : 0u;
        const uint64_t t_start = now_ticks();
        while (true) {
            const uint64_t missing = ~wave_ballot(!need || seen >= p.step) & wave_exec();
            if (missing == 0) break;
            if (now_ticks() - t_start > p.timeout_ticks) {
                const int bad_lane = __ffsll((unsigned long long)missing) - 1;
                if (lane == 0) report_timeout(p.flags, kPhaseTwoshotAg, j, tf + uint32_t(bad_lane));
                return;  // skip the chunk's copies
            }
            __builtin_amdgcn_s_sleep(1);
            if (need) seen = flag_load_relaxed(slot);
        }
        const __amdgpu_buffer_rsrc_t rs = buffer_range(p.seg[j] + v0, (vend - v0) * 16u);
        u32x4 x[C];
#pragma unroll
        for (int u = 0; u < C; ++u) x[u] = ld_coherent(rs, (uint32_t(u * kWave) + uint32_t(lane)) * 16u);
#pragma unroll
        for (int u = 0; u < C; ++u) {
            const uint32_t v = uint32_t(u * kWave) + uint32_t(lane);
            if (v0 + v < vend) st_stream(dst + v, x[u]);
        }
    }
}

// ---------------------------------------------------------------------------
// Two-shot under LL128: each reduced segment travels as an LL128 wire (128-
// byte lines of 120 data bytes and a 64-bit flag, "集合通信：NCCL 的算法、协议与
// 推理框架的定制 all-reduce", 协议 table).  The pages' LL128 rests on a 128-byte
// line being written and read whole.  Here a line is written by 8 lanes and
// read as separate 64-byte requests, so a reader that takes the data it
// loaded beside a flag could see the flag of step s with data of step s-1.
// The protocol is therefore made to hold by ordering:
//   producer  the 120 data bytes of its lines (sc1 stores), a wait until
//             those stores are complete, then each line's flag;
//   consumer  the flags of its lines first, and the data only once every
//             flag it needs is >= step.
// A flag seen >= step then means that its line's data was complete before
// the data loads were issued, also when the producer runs at the same time
// (another workgroup of the same launch, or another GPU).  The price is two
// dependent memory round trips on each side, as with the arrival slots;
// what LL128 still changes is the flag granularity (one per line, not one
// per tile).
//
// Work.  A segment of SB = m * element bytes is nlines = ceil(SB / 120)
// lines; a unit is 8 lines (one wavefront: lane l holds wire bytes
// [16 (l % 8), +16) of line l / 8, i.e. data bytes [120 line + 16 part, +16),
// at part 7 8 data bytes and then the flag; on the data side lane i < 60
// holds the unit's aligned 16-byte chunk i, the two orders exchanged through
// LDS, below).  Items: reduce-scatter units of
// segments r0..r1-1, then all-gather chunks of C units of every peer segment
// for every output in [r0, r1).  With a grid of one wavefront per item (one
// GPU's share with an explicit step id, or the reduce-scatter alone) each
// wavefront has one item; otherwise the grid is persistent (no larger than
// the device holds at once; with auto step ids the fixed grid of every auto
// launch) and items are dealt round-robin, all-gather items starting after
// the wavefronts with reduce-scatter items, as in the slot kernel.
struct TwoShot128Params {
    const uint8_t* in[kMaxRanks];
    uint8_t* segw[kMaxRanks];
    uint8_t* out[kMaxRanks];
    uint32_t* flags;
    uint64_t timeout_ticks;
    size_t seg_bytes;    // SB, a multiple of 16
    uint32_t nlines;     // lines per segment wire
    uint32_t nunits;     // 8-line units per segment
    uint32_t ag_chunks;  // all-gather chunks (C units) per segment
    uint32_t step;
    int auto_step;
    int r0, r1;
    int do_ag;
    FastDiv div_units;    // nunits
    FastDiv div_per_out;  // all-gather items per output rank: (n - 1) * ag_chunks
    FastDiv div_chunks;   // ag_chunks
};

// The flags of reduce-scatter unit u of segment r, only once the unit's data
// stores are complete.  A line's flag shares its last 32-byte sector with
// data bytes [96, 120); an 8-byte store of the flag alone is a partial
// sector write, which measured slower than whole sectors, so the lanes at
// parts 6 and 7 store that sector whole: their data again (the values the
// data pass stored, so a reader can see nothing new but the flag) and the
// flag.  ld = the lane's 16 wire bytes from the data pass.
__device__ __forceinline__ void ll128_rs_flags(const TwoShot128Params& p, uint32_t r, uint32_t u, uint32_t lstep,
                                               u32x4 ld, int lane) {
    const uint32_t line = u * 8u + uint32_t(lane) / 8u;
    const uint32_t part = uint32_t(lane) & 7u;
    const uint32_t lines_here = min(8u, p.nlines - min(p.nlines, u * 8u));
    const __amdgpu_buffer_rsrc_t rs = buffer_range(p.segw[r] + size_t(u) * 1024u, lines_here * 128u);
    if (line < p.nlines && part >= 6u)
        st_coherent(rs, uint32_t(lane) * 16u, part == 7u ? u32x4{ld.x, ld.y, lstep, 0u} : ld);
}

// The 960 data bytes of an 8-line unit are contiguous in a segment and
// 16-byte aligned (960 = 60 * 16), but a lane's part of a line starts at
// 120 line + 16 part, only 8-byte aligned.  The reduce-scatter loads and
// folds a unit as 60 aligned 16-byte chunks (lane i < 60: chunk i) and puts
// the sums in line order through a wavefront-private LDS strip; the
// all-gather puts line data back in chunk order the same way and stores
// aligned 16-byte chunks.
constexpr uint32_t kUnitBytes = 960;

// LDS-only ordering between a wavefront's strip writes and its reads (a
// fence over every address space would also wait for its global stores).
__device__ __forceinline__ void strip_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Reduce-scatter unit u of segment r: loads; if a previous unit's flags are
// pending, a wait for every earlier memory operation of the wavefront (its
// data stores among them) and those flags; the fold, which otherwise runs
// as the loads land; rank r's own output chunk; the unit's line data.  Its
// own flags are left to the caller, after a later wait.
template <typename T, int NR>
__device__ __forceinline__ u32x4 ll128_rs_data(const TwoShot128Params& p, uint8_t* strip, uint32_t r, uint32_t u,
                                               uint32_t lstep, bool pend, uint32_t pend_r, uint32_t pend_u,
                                               uint32_t pend_step, u32x4 pend_ld, int lane) {
    const uint32_t line = u * 8u + uint32_t(lane) / 8u;
    const uint32_t part = uint32_t(lane) & 7u;
    const size_t seg0 = size_t(r) * p.seg_bytes;
    const size_t ubase = size_t(u) * kUnitBytes;
    const uint32_t ub = uint32_t(min(size_t(kUnitBytes), p.seg_bytes - ubase));  // a multiple of 16
    // lanes past the unit's chunks re-read chunk 0 and contribute zeros
    const bool has_chunk = uint32_t(lane) * 16u < ub;
    const size_t src = seg0 + ubase + (has_chunk ? uint32_t(lane) * 16u : 0u);
    u32x4 x[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) x[i] = ld_stream(reinterpret_cast<const u32x4*>(p.in[i] + src));
    if (pend) {
        // covers the loads and the previous unit's data stores (issued before
        // them): that unit's flags may go now, a round trip after its data
        wait_stores();
        ll128_rs_flags(p, pend_r, pend_u, pend_step, pend_ld, lane);
    }
    Acc<T> acc;
#pragma unroll
    for (int i = 0; i < NR; ++i) acc.add(x[i]);
    u32x4 v = acc.result();
    if (!has_chunk) v = u32x4{0u, 0u, 0u, 0u};  // zero padding past the segment's end
    // rank r's own segment of its output, straight from registers (fused form)
    if (p.do_ag && has_chunk) st_stream(reinterpret_cast<u32x4*>(p.out[r] + seg0 + ubase) + lane, v);
    // chunk order -> line order
    if (lane < 60) *reinterpret_cast<u32x4*>(strip + lane * 16) = v;
    strip_sync();
    const uint32_t d = uint32_t(lane / 8) * 120u + part * 16u;
    const u32x2 lo = *reinterpret_cast<const u32x2*>(strip + d);
    const u32x2 hi = part != 7u ? *reinterpret_cast<const u32x2*>(strip + d + 8) : u32x2{0u, 0u};
    strip_sync();  // the strip's next writes after these reads
    const uint32_t lines_here = min(8u, p.nlines - min(p.nlines, u * 8u));
    const __amdgpu_buffer_rsrc_t rs = buffer_range(p.segw[r] + size_t(u) * 1024u, lines_here * 128u);
    // part 7: its 8 data bytes with the flag word at the previous step id
    // (below lstep, so no reader takes the line yet, and not below any id
    // the line carried before), one whole 16-byte store
    const u32x4 ld = part != 7u ? u32x4{lo.x, lo.y, hi.x, hi.y} : u32x4{lo.x, lo.y, lstep - 1u, 0u};
    if (line < p.nlines) st_coherent(rs, uint32_t(lane) * 16u, ld);
    return ld;
}

template <int NR, int C>
__device__ __forceinline__ void ll128_ag_chunk(const TwoShot128Params& p, uint8_t* strip, uint32_t ro, uint32_t j,
                                               uint32_t k, uint32_t want, int lane) {
    const uint32_t u0 = k * uint32_t(C);
    const uint32_t line0 = u0 * 8u;
    const uint32_t nl = min(uint32_t(8 * C), p.nlines - line0);  // lines of this chunk
    const __amdgpu_buffer_rsrc_t rs = buffer_range(p.segw[j] + size_t(line0) * 128u, nl * 128u);
    // the chunk's flags: lane l < nl polls line line0 + l
    const bool need = uint32_t(lane) < nl;
    const uint32_t foff = uint32_t(lane) * 128u + 120u;
    uint32_t seen = need ? ld_coherent8(rs, foff).x : 0u;
    const uint64_t t_start = now_ticks();
    while (true) {
        const uint64_t missing = ~wave_ballot(!need || seen >= want) & wave_exec();
        if (missing == 0) break;
        if (now_ticks() - t_start > p.timeout_ticks) {
            const int bad = __ffsll((unsigned long long)missing) - 1;
            if (lane == 0) report_timeout(p.flags, kPhaseTwoshotAg, j, line0 + uint32_t(bad));
            return;  // skip the chunk's copies
        }
        __builtin_amdgcn_s_sleep(1);
        if (need) seen = ld_coherent8(rs, foff).x;
    }
    // every flag seen: now the data (out-of-range loads read zero)
    u32x4 x[C];
#pragma unroll
    for (int c = 0; c < C; ++c) x[c] = ld_coherent(rs, uint32_t(c) * 1024u + uint32_t(lane) * 16u);
    const uint32_t part = uint32_t(lane) & 7u;
    const uint32_t d = uint32_t(lane / 8) * 120u + part * 16u;
    uint8_t* o = p.out[ro] + size_t(j) * p.seg_bytes;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const size_t ubase = size_t(u0 + uint32_t(c)) * kUnitBytes;
        if (ubase >= p.seg_bytes) break;  // wavefront-uniform
        const uint32_t ub = uint32_t(min(size_t(kUnitBytes), p.seg_bytes - ubase));
        // line order -> chunk order: the data half of part 7 only, the flag stays out
        *reinterpret_cast<u32x2*>(strip + d) = u32x2{x[c].x, x[c].y};
        if (part != 7u) *reinterpret_cast<u32x2*>(strip + d + 8) = u32x2{x[c].z, x[c].w};
        strip_sync();
        // lanes 0..59 hold the unit's chunks (fewer in a segment's last unit);
        // the others read nothing, so no lane reads past its 960-byte strip
        const bool mine = uint32_t(lane) * 16u < ub;
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (mine) v = *reinterpret_cast<const u32x4*>(strip + lane * 16);
        strip_sync();  // the strip's next writes after these reads
        if (mine) st_stream(reinterpret_cast<u32x4*>(o + ubase) + lane, v);
    }
}

template <typename T, int NR, int C, int WB>
__global__ __launch_bounds__(kWave * WB) void twoshot_ll128_kernel(TwoShot128Params p) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(blockIdx.x * WB + threadIdx.x / kWave);
    const uint32_t nwaves = gridDim.x * WB;
    const uint32_t R = uint32_t(p.r1 - p.r0);
    __shared__ __attribute__((aligned(16))) uint8_t strips[WB][kUnitBytes];
    uint8_t* strip = &strips[threadIdx.x / kWave][0];
    // auto step ids: lane l < R holds this wavefront's epoch copy of rank r0 + l
    uint32_t* epoch = p.flags + kStatusWords + NR * kSlotsPerRank + size_t(wave) * NR + p.r0;
    uint32_t epoch_lane = 0;
    if (p.auto_step && uint32_t(lane) < R) epoch_lane = flag_load_relaxed(epoch + lane);
    const uint32_t rs_items = R * p.nunits;
    // Each unit's flags are written while the next unit's loads are waited
    // for (that wait also covers the unit's data stores), the last unit's
    // after a wait of its own: every flag after its line's data, with no
    // store round trip inside the loop.
    bool pend = false;
    uint32_t pend_r = 0, pend_u = 0, pend_step = 0;
    u32x4 pend_ld = u32x4{0u, 0u, 0u, 0u};
    for (uint32_t it = wave; it < rs_items; it += nwaves) {
        const uint32_t rr = fdiv(it, p.div_units);
        const uint32_t r = uint32_t(p.r0) + rr;
        const uint32_t u = it - rr * p.nunits;
        const uint32_t lstep = p.auto_step ? __shfl(epoch_lane + 1u, int(rr)) : p.step;
        pend_ld = ll128_rs_data<T, NR>(p, strip, r, u, lstep, pend, pend_r, pend_u, pend_step, pend_ld, lane);
        pend = true;
        pend_r = r;
        pend_u = u;
        pend_step = lstep;
    }
    if (pend) {
        wait_stores();  // every data byte of the last unit's lines complete before its flags
        ll128_rs_flags(p, pend_r, pend_u, pend_step, pend_ld, lane);
    }
    if (p.do_ag) {
        const uint32_t per_out = uint32_t(NR - 1) * p.ag_chunks;
        const uint32_t items = R * per_out;
        const uint32_t rs_busy = min(rs_items, nwaves);
        const uint32_t ag_wave = wave >= rs_busy ? wave - rs_busy : wave + (nwaves - rs_busy);
        for (uint32_t it = ag_wave; it < items; it += nwaves) {
            const uint32_t oo = fdiv(it, p.div_per_out);
            const uint32_t ro = uint32_t(p.r0) + oo;
            const uint32_t rem = it - oo * per_out;
            const uint32_t jj = fdiv(rem, p.div_chunks);
            const uint32_t j = ag_source(jj, ro, true);
            const uint32_t k = rem - jj * p.ag_chunks;
            // the output rank's step id (its reduce-scatter in this launch, for
            // auto ids: every rank's epoch moves in step)
            const uint32_t want = p.auto_step ? __shfl(epoch_lane + 1u, int(oo)) : p.step;
            ll128_ag_chunk<NR, C>(p, strip, ro, j, k, want, lane);
        }
    }
    if (p.auto_step && uint32_t(lane) < R) flag_store_relaxed(epoch + lane, epoch_lane + 1u);
}

// all-gather chunk of the LL128 two-shot, 8-line units per wavefront: one
// where a wavefront has one item, eight (64 lines, one flag per lane) in the
// persistent grid, where a wavefront walks many
constexpr int kLL128ChunkShare = 1;
constexpr int kLL128ChunkPersistent = 8;

template <typename T, int NR>
hipError_t launch_ll128(const TwoShotRequest& rq, hipStream_t s) {
    DeviceInfo info;
    hipError_t e = device_info(&info);
    if (e != hipSuccess) return e;
    TwoShot128Params p{};
    for (int r = 0; r < NR; ++r) {
        p.in[r] = static_cast<const uint8_t*>(rq.in[r]);
        p.segw[r] = static_cast<uint8_t*>(rq.seg[r]);
        p.out[r] = (rq.out && r >= rq.r0 && r < rq.r1) ? static_cast<uint8_t*>(rq.out[r]) : nullptr;
    }
    p.seg_bytes = rq.numel / size_t(NR) * size_t(elem<T>::bytes);
    p.nlines = uint32_t((p.seg_bytes + 119) / 120);
    p.nunits = (p.nlines + 7u) / 8u;
    const bool sized = rq.step != 0 && (!rq.do_ag || rq.r1 - rq.r0 == 1);  // a wavefront per item
    const uint32_t chunk = sized ? kLL128ChunkShare : kLL128ChunkPersistent;
    p.ag_chunks = (p.nunits + chunk - 1) / chunk;
    p.flags = rq.flags;
    p.timeout_ticks = rq.timeout_ticks;
    p.step = rq.step;
    p.auto_step = rq.step == 0;
    p.r0 = rq.r0;
    p.r1 = rq.r1;
    p.do_ag = rq.do_ag;
    p.div_units = make_fastdiv(p.nunits);
    p.div_per_out = make_fastdiv(uint32_t(NR - 1) * p.ag_chunks);
    p.div_chunks = make_fastdiv(p.ag_chunks);
    const uint32_t R = uint32_t(rq.r1 - rq.r0);
    const uint64_t items = uint64_t(R) * p.nunits + (rq.do_ag ? uint64_t(R) * (NR - 1) * p.ag_chunks : 0u);
    if (p.auto_step) {
        // the fixed grid of every auto launch on a flag region (two 256-lane
        // workgroups per CU), so each wavefront's epoch copies see every call
        const uint32_t grid = uint32_t(info.cu_count) * 2u;
        if (grid * 4u > uint32_t(kEpochCopies)) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((twoshot_ll128_kernel<T, NR, kLL128ChunkPersistent, 4>), dim3(grid), dim3(kBlock), 0, s,
                           p);
        return hipGetLastError();
    }
    if (!rq.do_ag || R == 1) {
        // nothing in this launch waits on another wavefront of it: one
        // wavefront per item, four-wavefront workgroups for large grids
        if (items >= uint64_t(kShareWideMinWavesPerCu) * uint64_t(info.cu_count)) {
            hipLaunchKernelGGL((twoshot_ll128_kernel<T, NR, kLL128ChunkShare, 4>), dim3(uint32_t((items + 3) / 4)),
                               dim3(kBlock), 0, s, p);
        } else {
            hipLaunchKernelGGL((twoshot_ll128_kernel<T, NR, kLL128ChunkShare, 1>), dim3(uint32_t(items)), dim3(kWave),
                               0, s, p);
        }
        return hipGetLastError();
    }
    // consumers wait on producers of the same launch: a persistent grid
    static int per_cu = -1;
    static hipError_t occ_err = hipSuccess;
    static std::once_flag once;
    auto kern = twoshot_ll128_kernel<T, NR, kLL128ChunkPersistent, 4>;
    std::call_once(once, [&] { occ_err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kBlock, 0); });
    if (occ_err != hipSuccess) return occ_err;
    if (per_cu < 1) return hipErrorLaunchOutOfResources;
    const uint32_t resident = uint32_t(info.cu_count) * uint32_t(per_cu < 2 ? per_cu : 2);
    uint64_t grid = (items + 3) / 4;
    if (grid > resident) grid = resident;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(kern, dim3(uint32_t(grid)), dim3(kBlock), 0, s, p);
    return hipGetLastError();
}

// The barrier of a copy-engine all-gather: one workgroup waits until the
// arrival slot of every tile of every segment is >= the step id (the
// largest of the ranks' in [r0, r1) in auto mode, where wavefront 0's epoch
// copies stand for all copies), or reports a timeout; the copies follow in
// stream order and need no compute unit.
template <int NR>
__global__ __launch_bounds__(kBlock) void ag_wait_kernel(TwoShotParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    uint32_t want = p.step;
    if (p.auto_step) {
        want = 0;
        for (int r = p.r0; r < p.r1; ++r) {
            const uint32_t e = flag_load_relaxed(p.flags + kStatusWords + NR * kSlotsPerRank + r);
            want = e > want ? e : want;
        }
    }
    const uint32_t* slots = p.flags + kStatusWords;
    const uint32_t items = uint32_t(NR) * p.ktiles;
    for (uint32_t kb = wave * kWave; kb < items; kb += kWavesPerBlock * kWave) {
        const uint32_t k = kb + uint32_t(lane);
        const bool need = k < items;
        const uint32_t j = need ? k / p.ktiles : 0u, t = need ? k % p.ktiles : 0u;
        const uint32_t* slot = slots + j * kSlotsPerRank + t;
        const uint64_t t0 = now_ticks();
        while (true) {
            const bool ok = !need || flag_load_relaxed(slot) >= want;
            const uint64_t missing = ~wave_ballot(ok) & wave_exec();
            if (missing == 0) break;
            if (now_ticks() - t0 > p.timeout_ticks) {
                const int bad_lane = __ffsll((unsigned long long)missing) - 1;
                const uint32_t bj = __shfl(j, bad_lane);
                const uint32_t bt = __shfl(t, bad_lane);
                if (lane == 0) report_timeout(p.flags, kPhaseTwoshotAg, bj, bt);
                return;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
}

// Segment tiling shared by every two-shot launch and the copy-engine wait.
void tile_params(TwoShotParams& p, size_t seg_bytes) {
    p.mvec = uint32_t(seg_bytes / 16);
    const uint32_t per_slot = (p.mvec + kSlotsPerRank - 1) / kSlotsPerRank;  // vectors per slot at least
    p.tile = ((per_slot + kWave - 1) / kWave) * kWave;
    if (p.tile == 0) p.tile = kWave;
    p.ktiles = (p.mvec + p.tile - 1) / p.tile;
    p.div_upt = make_fastdiv(p.tile / kWave);
    p.div_ktiles = make_fastdiv(p.ktiles);
}

template <typename T, int NR, bool kLL>
hipError_t launch_k(const TwoShotRequest& rq, hipStream_t s) {
    // one unit in flight per wavefront in phase 1 (NR loads per lane), four in
    // phase 2: measured best for decode-sized messages, equal within noise
    // at 64 MiB per rank
    constexpr int U = 1;
    DeviceInfo info;
    hipError_t e = device_info(&info);
    if (e != hipSuccess) return e;

    TwoShotParams p{};
    for (int r = 0; r < NR; ++r) {
        p.in[r] = rq.in ? static_cast<const u32x4*>(rq.in[r]) : nullptr;
        p.seg[r] = static_cast<u32x4*>(rq.seg[r]);
        p.out[r] = (rq.out && r >= rq.r0 && r < rq.r1) ? static_cast<u32x4*>(rq.out[r]) : nullptr;
    }
    tile_params(p, rq.numel / size_t(NR) * size_t(elem<T>::bytes));
    p.flags = rq.flags;
    p.timeout_ticks = rq.timeout_ticks;
    p.step = rq.step;
    p.auto_step = rq.step == 0;
    p.r0 = rq.r0;
    p.r1 = rq.r1;
    p.do_rs = rq.do_rs;
    p.do_ag = rq.do_ag;
    p.div_per_out = make_fastdiv(uint32_t(rq.do_rs ? NR - 1 : NR) * p.ktiles);

    auto kern = twoshot_kernel<T, NR, U, kLL>;
    const uint32_t R = uint32_t(rq.r1 - rq.r0);
    {
        if (!p.auto_step && R == 1 && rq.do_rs && rq.do_ag) {
            // one GPU's share: a grid of one wavefront per reduce-scatter
            // tile plus one per all-gather chunk
            p.ag_chunks = (p.mvec + uint32_t(kShareChunk * kWave) - 1) / uint32_t(kShareChunk * kWave);
            p.div_chunks = make_fastdiv(p.ag_chunks);
            const uint64_t waves = uint64_t(p.ktiles) + uint64_t(NR - 1) * p.ag_chunks;
            constexpr int RU = share_rs_unroll<NR>();
            if (waves >= uint64_t(kShareWideMinWavesPerCu) * uint64_t(info.cu_count)) {
                hipLaunchKernelGGL((twoshot_share_kernel<T, NR, kShareChunk, 4, RU, kLL>), dim3(uint32_t((waves + 3) / 4)),
                                   dim3(kWave * 4), 0, s, p);
            } else {
                hipLaunchKernelGGL((twoshot_share_kernel<T, NR, kShareChunk, 1, RU, kLL>), dim3(uint32_t(waves)),
                                   dim3(kWave), 0, s, p);
            }
            return hipGetLastError();
        }
    }
    if (p.auto_step) {
        // every auto launch on a flag region uses the same grid, two
        // workgroups per CU (resident at once: the occupancy of every
        // instantiation is at least that), so that each wavefront's epoch
        // copies see every call
        const uint32_t grid = uint32_t(info.cu_count) * 2u;
        if (grid * uint32_t(kWavesPerBlock) > uint32_t(kEpochCopies)) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(kern, dim3(grid), dim3(kBlock), 0, s, p);
        return hipGetLastError();
    }
    if (rq.do_rs && rq.do_ag) {
        // Persistent grid for the fused form: at most as many workgroups as
        // the device holds at once (occupancy of this kernel, capped at two
        // per CU), so every producer is resident while consumers poll.  The
        // occupancy is a property of the compiled kernel: query it once.
        static int per_cu = -1;
        static hipError_t occ_err = hipSuccess;
        static std::once_flag once;
        std::call_once(once, [&] { occ_err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kBlock, 0); });
        if (occ_err != hipSuccess) return occ_err;
        if (per_cu < 1) return hipErrorLaunchOutOfResources;
        const uint32_t resident = uint32_t(info.cu_count) * uint32_t(per_cu < 2 ? per_cu : 2);
        // one wavefront per item (phase 1 plus phase 2) if the device holds that many
        uint32_t grid = (R * uint32_t(NR) * p.ktiles + kWavesPerBlock - 1) / kWavesPerBlock;
        if (grid > resident) grid = resident;
        if (grid < 1) grid = 1;
        hipLaunchKernelGGL(kern, dim3(grid), dim3(kBlock), 0, s, p);
        return hipGetLastError();
    }
    // Split launches: size the grid to the work, at most two blocks per CU.
    const uint32_t items = rq.do_rs ? R * p.ktiles : R * uint32_t(NR) * p.ktiles;
    uint32_t grid = (items + kWavesPerBlock - 1) / kWavesPerBlock;
    const uint32_t cap = uint32_t(info.cu_count) * 2u;
    if (grid > cap) grid = cap;
    if (grid == 0) grid = 1;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kBlock), 0, s, p);
    return hipGetLastError();
}

template <typename T, int NR>
hipError_t launch_t(const TwoShotRequest& rq, hipStream_t s) {
    if (rq.ll128) return launch_ll128<T, NR>(rq, s);
    return rq.ll ? launch_k<T, NR, true>(rq, s) : launch_k<T, NR, false>(rq, s);
}

}  // namespace

hipError_t launch_twoshot_ag_copy(const TwoShotRequest& rq, hipStream_t s) {
    const size_t es = rq.dtype == 0 ? 4 : 2;
    const size_t m_bytes = rq.numel / size_t(rq.n) * es;
    TwoShotParams p{};
    tile_params(p, m_bytes);
    p.flags = rq.flags;
    p.timeout_ticks = rq.timeout_ticks;
    p.step = rq.step;
    p.auto_step = rq.step == 0;
    p.r0 = rq.r0;
    p.r1 = rq.r1;
    hipError_t e = dispatch_ranks(rq.n, [&](auto nr) {
        constexpr int NR = decltype(nr)::value;
        hipLaunchKernelGGL(ag_wait_kernel<NR>, dim3(1), dim3(kBlock), 0, s, p);
        return hipGetLastError();
    });
    if (e != hipSuccess) return e;
    // the all-gather proper: n segment copies per output on the copy engines
    for (int r = rq.r0; r < rq.r1; ++r)
        for (int j = 0; j < rq.n; ++j) {
            e = hipMemcpyAsync(static_cast<char*>(rq.out[r]) + size_t(j) * m_bytes, rq.seg[j], m_bytes,
                               hipMemcpyDeviceToDeviceNoCU, s);
            if (e != hipSuccess) return e;
        }
    return hipSuccess;
}

hipError_t launch_twoshot(const TwoShotRequest& rq, hipStream_t s) {
    return dispatch_ranks(rq.n, [&](auto nr) {
        constexpr int NR = decltype(nr)::value;
        return rq.dtype == 0 ? launch_t<float, NR>(rq, s) : launch_t<bf16_t, NR>(rq, s);
    });
}

}  // namespace ar
