// Internal launch interface between the C ABI (ar_api.cpp) and the kernel
// files.  Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace ar {

// Flag region layout for n ranks (32-bit words): word 0 status, word 1
// detail, words 2..31 unused (one 128-byte line), then kSlotsPerRank arrival
// slots per rank, then kEpochCopies x n epoch copies: wavefront w of an
// auto-step two-shot launch keeps rank r's copy at word w * n + r of that
// area, so one wavefront's copies share a cache line.
constexpr int kMaxRanks = 16;
constexpr int kSlotsPerRank = 1024;
constexpr int kEpochCopies = 4096;
constexpr int kStatusWords = 32;
constexpr uint32_t kTimeoutCode = 5;  // AR_ERR_TIMEOUT
// Phase of a reported timeout (the status word's bits 8..15), one per kind
// of bounded wait: a two-shot all-gather's slot or done flag, an LL line,
// an LL128 line, a fused RMSNorm row's sibling partial sums.
constexpr uint32_t kPhaseTwoshotAg = 1;  // AR_PHASE_TWOSHOT_AG
constexpr uint32_t kPhaseLl = 2;         // AR_PHASE_LL
constexpr uint32_t kPhaseLl128 = 3;      // AR_PHASE_LL128
constexpr uint32_t kPhaseRmsnorm = 4;    // AR_PHASE_RMSNORM

struct DeviceInfo {
    int cu_count;
    int wallclock_khz;
    int coop_supported;
};

// Cached per-device properties (queried once per device).
hipError_t device_info(DeviceInfo* out);

hipError_t launch_oneshot(const void* const* in, int n, void* out, size_t numel, int dtype,
                          hipStream_t s);

hipError_t launch_reduce_bcast(const void* const* in, int n, void* const* out, size_t numel, int dtype, int r0,
                               int r1, hipStream_t s);

hipError_t launch_push(const void* const* src, int nsrc, void* const* dst, int ndst, size_t nbytes,
                       hipStream_t s);

struct TwoShotRequest {
    const void* const* in;   // may be null when !do_rs
    void* const* seg;
    void* const* out;        // may be null when !do_ag
    int n;
    size_t numel;
    int dtype;
    int r0, r1;
    uint32_t* flags;
    uint32_t step;
    bool do_rs, do_ag;
    uint64_t timeout_ticks;
    bool ll;  // segments are LL wires (4 data bytes + the step id per line); no slots
    bool ll128 = false;  // segments are LL128 wires (120 data bytes + a 64-bit step id per line)
};
hipError_t launch_twoshot(const TwoShotRequest& rq, hipStream_t s);
// All-gather on the copy engines: a one-workgroup slot wait, then n
// hipMemcpyAsync copies per output rank.
hipError_t launch_twoshot_ag_copy(const TwoShotRequest& rq, hipStream_t s);

hipError_t launch_ll_pack(const void* const* src, void* const* wire, int count, size_t nbytes,
                          int proto, uint32_t step, hipStream_t s);

hipError_t launch_ll_reduce(const void* const* wire, int n, void* out, size_t numel, int dtype,
                            int proto, uint32_t step, uint32_t* flags, uint64_t timeout_ticks,
                            hipStream_t s);

// One GPU's LL / LL128 step in one launch: pack rank me's message src into
// wire[me] and reduce all n messages into out (rank me's term from src).
hipError_t launch_ll_allreduce(const void* src, const void* const* wire, int n, int me, void* out, size_t numel,
                               int dtype, int proto, uint32_t step, uint32_t* flags, uint64_t timeout_ticks,
                               hipStream_t s);

hipError_t launch_flag_reset(uint32_t* flags, size_t words, hipStream_t s);

// One-shot all-reduce + residual add + RMSNorm over rows of `hidden`
// elements (hidden * element size a multiple of 16, at most 4096 16-byte
// vectors per row).  ws (may be null): the workspace of the cooperative
// few-rows path, kRmsWorkspaceBytes, zeroed before first use.
constexpr size_t kRmsMaxRowVecs = 4096;
constexpr uint32_t kCoopGrid = 1024;
constexpr size_t kRmsWorkspaceBytes = (size_t(kStatusWords) + kCoopGrid + 2 * size_t(kCoopGrid)) * 4;
hipError_t launch_oneshot_rmsnorm(const void* const* in, int n, const void* residual, const void* weight,
                                  void* residual_out, void* out, size_t rows, size_t hidden, float eps, int dtype,
                                  uint32_t* ws, uint64_t timeout_ticks, hipStream_t s);
// Its two-shot form: rank r's reduce-scatter owns rows [r G, (r+1) G),
// G = rows / n, and writes them (out rows, then residual_out rows) to seg[r]
// with an arrival slot per tile; out == null: the reduce-scatter of ranks
// [r0, r1) alone; else one rank's share (r1 == r0 + 1), the all-gather of
// the peers' rows included.
size_t twoshot_rmsnorm_segment_bytes(int n, size_t rows, size_t hidden, int dtype);
hipError_t launch_twoshot_rmsnorm(const void* const* in, int n, const void* const* residual, const void* weight,
                                  void* const* seg, void* const* residual_out, void* const* out, size_t rows,
                                  size_t hidden, float eps, int dtype, int r0, int r1, uint32_t* flags,
                                  uint32_t step, uint64_t timeout_ticks, hipStream_t s);

// Allocation-free two-shot: a device array holding the arrival slots of up to
// kMaxRanks ranks (the flag region without its epoch area, padded to 256
// bytes) followed by up to kNoAllocMaxBytes of segments (the n segments of
// one message of at most that many bytes per rank).
constexpr size_t kNoAllocMaxBytes = size_t(64) << 20;
constexpr size_t kNoAllocFlagBytes = ((size_t(kStatusWords) + size_t(kMaxRanks) * kSlotsPerRank) * 4 + 255) / 256 * 256;
constexpr size_t kNoAllocScratchBytes = kNoAllocFlagBytes + kNoAllocMaxBytes;
// Device address of this device's scratch array (looked up once per device).
hipError_t noalloc_scratch(void** base);

// Call f(std::integral_constant<int, N>{}) for the rank count n in [2, 16].
template <typename F>
auto dispatch_ranks(int n, F&& f) {
    switch (n) {
        case 2: return f(std::integral_constant<int, 2>{});
        case 3: return f(std::integral_constant<int, 3>{});
        case 4: return f(std::integral_constant<int, 4>{});
        case 5: return f(std::integral_constant<int, 5>{});
        case 6: return f(std::integral_constant<int, 6>{});
        case 7: return f(std::integral_constant<int, 7>{});
        case 8: return f(std::integral_constant<int, 8>{});
        case 9: return f(std::integral_constant<int, 9>{});
        case 10: return f(std::integral_constant<int, 10>{});
        case 11: return f(std::integral_constant<int, 11>{});
        case 12: return f(std::integral_constant<int, 12>{});
        case 13: return f(std::integral_constant<int, 13>{});
        case 14: return f(std::integral_constant<int, 14>{});
        case 15: return f(std::integral_constant<int, 15>{});
        default: return f(std::integral_constant<int, 16>{});
    }
}

}  // namespace ar
