// C ABI of the library (declared in include/ar.h): synchronous argument
// checks, then the launch.  Every check happens before anything is enqueued,
// so an error return means the stream is untouched.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <atomic>
#include <mutex>
#include <vector>

#include "ar.h"
#include "ar_launch.hpp"

static_assert(ar::kNoAllocMaxBytes == AR_NOALLOC_MAX_BYTES, "the header states the scratch limit");
static_assert(ar::kTimeoutCode == AR_ERR_TIMEOUT && ar::kPhaseTwoshotAg == AR_PHASE_TWOSHOT_AG &&
                  ar::kPhaseLl == AR_PHASE_LL && ar::kPhaseLl128 == AR_PHASE_LL128 &&
                  ar::kPhaseRmsnorm == AR_PHASE_RMSNORM,
              "the kernels report the header's status codes");

namespace ar {

namespace {

constexpr uint64_t kDefaultTimeoutNs = 1000000000ull;  // 1 s
std::atomic<uint64_t> g_timeout_ns{kDefaultTimeoutNs};

constexpr int kMaxDevices = 64;
std::mutex g_info_mu;
DeviceInfo g_info[kMaxDevices];
bool g_info_ok[kMaxDevices] = {};

// Largest message accepted per rank (16 GiB).  A dispatch holds fewer than
// 2^32 work-items, and the finest-grained launches take one work-item per
// 8 bytes of the message (the one-shot's 8-byte lanes, the reduce-broadcast's
// 8-byte halves, the LL reduction's pairs of lines), so 2^34 bytes keeps every
// grid at 2^31 work-items or fewer; 16-byte vector indices then fit in 31 bits.
constexpr size_t kMaxBytes = size_t(1) << 34;
constexpr size_t kStatusBytes = size_t(kStatusWords) * 4;

size_t elem_bytes(int dtype) { return dtype == AR_F32 ? 4 : 2; }

#include "select_table.inc"

// Semaphore synchronisations per call charged by the cost model, in ar_algo
// order: start and end for the one-shot, the push and the reduce-broadcast;
// two more around the two-shot's barrier; none for LL / LL128, whose
// receivers learn of arrival from the flags in the lines; start and end for
// the two-shot under LL and under LL128 (they read the peers' inputs; the
// barrier between their phases is in the lines).
constexpr double kSemaphoreSyncs[] = {2.0, 4.0, 0.0, 0.0, 2.0, 2.0, 2.0, 2.0};
static_assert(kSelNumAlgos <= int(sizeof(kSemaphoreSyncs) / sizeof(kSemaphoreSyncs[0])), "one count per algorithm");

// Measured one-GPU time of algo at `bytes` per rank: piecewise linear in the
// size between grid points, flat below the first (launch-bound), and
// extended with the last segment's slope above the last (bandwidth-bound).
double share_us(int algo, int n, double bytes) {
    const float* t = kSelUs[n - 2][algo];
    if (bytes <= double(kSelSizes[0])) return t[0];
    int k = 1;
    while (k < kSelNumSizes - 1 && bytes > double(kSelSizes[k])) ++k;
    const double x0 = double(kSelSizes[k - 1]), x1 = double(kSelSizes[k]);
    return t[k - 1] + (double(t[k]) - double(t[k - 1])) * (bytes - x0) / (x1 - x0);
}
bool dtype_ok(int dtype) { return dtype == AR_F32 || dtype == AR_BF16; }
bool ranks_ok(int n) { return n >= 2 && n <= AR_MAX_RANKS; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
    uintptr_t lo, hi;
    bool written;
};

Span span(const void* p, size_t bytes, bool written) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Span{lo, lo + bytes, written};
}

// A written span may not overlap any other span; read spans may overlap each
// other (one buffer may stand for several emulated ranks).  Sorted by start,
// a span can only overlap the spans that start before it ends.
bool spans_ok(std::vector<Span> v) {
    std::sort(v.begin(), v.end(), [](const Span& x, const Span& y) { return x.lo < y.lo; });
    for (size_t a = 0; a < v.size(); ++a) {
        if (v[a].lo == v[a].hi) continue;
        for (size_t b = a + 1; b < v.size() && v[b].lo < v[a].hi; ++b)
            if (v[b].lo != v[b].hi && (v[a].written || v[b].written)) return false;
    }
    return true;
}

uint64_t timeout_ticks() {
    DeviceInfo info;
    if (device_info(&info) != hipSuccess || info.wallclock_khz <= 0) return 100000000ull;
    const uint64_t ns = g_timeout_ns.load();
    const uint64_t khz = uint64_t(info.wallclock_khz);
    const uint64_t ticks = ns / 1000000ull * khz + (ns % 1000000ull) * khz / 1000000ull;
    return ticks == 0 ? 1 : ticks;
}

int hip_status(hipError_t e) { return e == hipSuccess ? AR_OK : AR_ERR_HIP; }

size_t wire_bytes(int proto, size_t nbytes) {
    if (proto == AR_PROTO_LL) return 8 * ((nbytes + 3) / 4);
    if (proto == AR_PROTO_LL128) return 128 * ((nbytes + 119) / 120);
    return 0;
}

// Shared checks of the two-shot entry points.
// seg_proto: the segment buffers hold the reduced data (-1) or an LL /
// LL128 wire of it (AR_PROTO_LL, AR_PROTO_LL128).
int twoshot_check(const void* const* in, const void* const* seg, const void* const* out, int n,
                  size_t numel, int dtype, int r0, int r1, const uint32_t* flags, uint32_t step,
                  int seg_proto = -1) {
    (void)step;  // 0 = the step id kept in the flag region (auto)
    if (!ranks_ok(n) || !dtype_ok(dtype) || numel == 0 || !seg || !flags) return AR_ERR_ARG;
    if (r0 < 0 || r1 > n || r0 >= r1) return AR_ERR_ARG;
    const size_t es = elem_bytes(dtype);
    if (numel > kMaxBytes / es) return AR_ERR_ARG;
    for (int i = 0; i < n; ++i) {
        if (!seg[i] || (in && !in[i])) return AR_ERR_ARG;
        if (!aligned16(seg[i]) || (in && !aligned16(in[i]))) return AR_ERR_ALIGN;
    }
    if (out)
        for (int r = r0; r < r1; ++r) {
            if (!out[r]) return AR_ERR_ARG;
            if (!aligned16(out[r])) return AR_ERR_ALIGN;
        }
    if (!aligned16(flags)) return AR_ERR_ALIGN;
    if (numel % size_t(n) != 0 || (numel / size_t(n) * es) % 16 != 0) return AR_ERR_DIVISIBLE;

    const size_t S = numel * es, m_bytes = S / size_t(n);
    std::vector<Span> v;
    v.push_back(span(flags, ar_flag_bytes(n), true));
    if (in)
        for (int i = 0; i < n; ++i) v.push_back(span(in[i], S, false));
    for (int j = 0; j < n; ++j) {
        // with an input present (reduce-scatter), seg[r0..r1) are written
        const bool written = in && j >= r0 && j < r1;
        v.push_back(span(seg[j], seg_proto < 0 ? m_bytes : wire_bytes(seg_proto, m_bytes), written));
    }
    if (out)
        for (int r = r0; r < r1; ++r) v.push_back(span(out[r], S, true));
    if (!spans_ok(v)) return AR_ERR_ALIAS;
    return AR_OK;
}

int ll_reduce_common(const void* const* wire, int n, void* out, size_t numel, int dtype,
                     uint32_t step, uint32_t* flags, int proto, void* stream) {
    if (!ranks_ok(n) || !dtype_ok(dtype) || numel == 0 || !wire || !out || !flags || step == 0)
        return AR_ERR_ARG;
    const size_t es = elem_bytes(dtype);
    if (numel > kMaxBytes / es) return AR_ERR_ARG;
    for (int i = 0; i < n; ++i) {
        if (!wire[i]) return AR_ERR_ARG;
        if (!aligned16(wire[i])) return AR_ERR_ALIGN;
    }
    if (!aligned16(out) || !aligned16(flags)) return AR_ERR_ALIGN;
    const size_t S = numel * es, W = wire_bytes(proto, S);
    std::vector<Span> v;
    v.push_back(span(out, S, true));
    v.push_back(span(flags, kStatusBytes, true));
    for (int i = 0; i < n; ++i) v.push_back(span(wire[i], W, false));
    if (!spans_ok(v)) return AR_ERR_ALIAS;
    return hip_status(launch_ll_reduce(wire, n, out, numel, dtype, proto, step, flags, timeout_ticks(),
                                       static_cast<hipStream_t>(stream)));
}

}  // namespace

hipError_t device_info(DeviceInfo* out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_info_mu);
    if (!g_info_ok[dev]) {
        DeviceInfo d{};
        if ((e = hipDeviceGetAttribute(&d.cu_count, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
            return e;
        if ((e = hipDeviceGetAttribute(&d.wallclock_khz, hipDeviceAttributeWallClockRate, dev)) != hipSuccess)
            return e;
        if ((e = hipDeviceGetAttribute(&d.coop_supported, hipDeviceAttributeCooperativeLaunch, dev)) !=
            hipSuccess)
            return e;
        g_info[dev] = d;
        g_info_ok[dev] = true;
    }
    *out = g_info[dev];
    return hipSuccess;
}

}  // namespace ar

using namespace ar;

extern "C" {

size_t ar_flag_bytes(int n) {
    if (!ranks_ok(n)) return 0;
    return (size_t(kStatusWords) + size_t(n) * (kSlotsPerRank + kEpochCopies)) * 4;
}

size_t ar_ll_wire_bytes(int proto, size_t nbytes) { return wire_bytes(proto, nbytes); }

void ar_set_poll_timeout_ns(uint64_t ns) { g_timeout_ns.store(ns == 0 ? kDefaultTimeoutNs : ns); }

uint64_t ar_get_poll_timeout_ns(void) { return g_timeout_ns.load(); }

const char* ar_status_string(int status) {
    switch (status & 0xFF) {
        case AR_OK: return "ok";
        case AR_ERR_ARG: return "invalid argument";
        case AR_ERR_ALIGN: return "pointer not 16-byte aligned";
        case AR_ERR_DIVISIBLE: return "two-shot size not divisible into 16-byte segments";
        case AR_ERR_ALIAS: return "written buffer overlaps another buffer";
        case AR_ERR_TIMEOUT: return "flag wait timed out";
        case AR_ERR_HIP: return "HIP runtime error";
        case AR_ERR_SIZE: return "message larger than the allocation-free call's scratch memory";
        default: return "unknown status";
    }
}

int ar_oneshot(const void* const* in, int n, void* out, size_t numel, int dtype, void* stream) {
    if (!in || !out || !ranks_ok(n) || !dtype_ok(dtype) || numel == 0) return AR_ERR_ARG;
    const size_t es = elem_bytes(dtype);
    if (numel > kMaxBytes / es) return AR_ERR_ARG;
    for (int i = 0; i < n; ++i) {
        if (!in[i]) return AR_ERR_ARG;
        if (!aligned16(in[i])) return AR_ERR_ALIGN;
    }
    if (!aligned16(out)) return AR_ERR_ALIGN;
    const size_t S = numel * es;
    std::vector<Span> v;
    v.push_back(span(out, S, true));
    for (int i = 0; i < n; ++i) v.push_back(span(in[i], S, false));
    if (!spans_ok(v)) return AR_ERR_ALIAS;
    return hip_status(launch_oneshot(in, n, out, numel, dtype, static_cast<hipStream_t>(stream)));
}

size_t ar_rmsnorm_workspace_bytes(void) { return kRmsWorkspaceBytes; }

int ar_oneshot_rmsnorm(const void* const* in, int n, const void* residual, const void* weight, void* residual_out,
                       void* out, size_t rows, size_t hidden, float eps, int dtype, uint32_t* workspace,
                       void* stream) {
    if (!in || !residual || !weight || !residual_out || !out || !ranks_ok(n) || !dtype_ok(dtype) || rows == 0 ||
        hidden == 0)
        return AR_ERR_ARG;
    if (!(eps >= 0.0f && eps <= FLT_MAX)) return AR_ERR_ARG;  // negative, NaN or infinite
    const size_t es = elem_bytes(dtype);
    if (hidden > kRmsMaxRowVecs * 16 / es || rows > kMaxBytes / es / hidden) return AR_ERR_ARG;
    for (int i = 0; i < n; ++i) {
        if (!in[i]) return AR_ERR_ARG;
        if (!aligned16(in[i])) return AR_ERR_ALIGN;
    }
    if (!aligned16(residual) || !aligned16(weight) || !aligned16(residual_out) || !aligned16(out) ||
        !aligned16(workspace))
        return AR_ERR_ALIGN;
    if ((hidden * es) % 16 != 0) return AR_ERR_DIVISIBLE;
    const size_t S = rows * hidden * es;
    std::vector<Span> v;
    v.push_back(span(out, S, true));
    // residual_out may be residual itself (each element is read before the
    // same lane writes it); any other overlap is refused
    if (residual_out != residual) {
        v.push_back(span(residual_out, S, true));
        v.push_back(span(residual, S, false));
    } else {
        v.push_back(span(residual_out, S, true));
    }
    v.push_back(span(weight, hidden * es, false));
    for (int i = 0; i < n; ++i) v.push_back(span(in[i], S, false));
    if (workspace) v.push_back(span(workspace, kRmsWorkspaceBytes, true));
    if (!spans_ok(v)) return AR_ERR_ALIAS;
    return hip_status(launch_oneshot_rmsnorm(in, n, residual, weight, residual_out, out, rows, hidden, eps, dtype,
                                             workspace, timeout_ticks(), static_cast<hipStream_t>(stream)));
}

size_t ar_rmsnorm_segment_bytes(int n, size_t rows, size_t hidden, int dtype) {
    if (!ranks_ok(n) || !dtype_ok(dtype) || rows % size_t(n) != 0) return 0;
    return twoshot_rmsnorm_segment_bytes(n, rows, hidden, dtype);
}

int ar_twoshot_rmsnorm(const void* const* in, int n, const void* const* residual, const void* weight,
                       void* const* seg, void* const* residual_out, void* const* out, size_t rows, size_t hidden,
                       float eps, int dtype, int r0, int r1, uint32_t* flags, uint32_t step, void* stream) {
    if (!in || !residual || !weight || !seg || !flags || !ranks_ok(n) || !dtype_ok(dtype) || rows == 0 ||
        hidden == 0)
        return AR_ERR_ARG;
    if (r0 < 0 || r1 > n || r0 >= r1) return AR_ERR_ARG;
    const bool fused = out != nullptr;
    if (fused != (residual_out != nullptr)) return AR_ERR_ARG;
    if (fused && r1 != r0 + 1) return AR_ERR_ARG;  // the all-gather: one rank's share per launch
    if (!(eps >= 0.0f && eps <= FLT_MAX)) return AR_ERR_ARG;
    const size_t es = elem_bytes(dtype);
    if (hidden > kRmsMaxRowVecs * 16 / es || rows > kMaxBytes / es / hidden) return AR_ERR_ARG;
    for (int i = 0; i < n; ++i) {
        if (!in[i] || !seg[i]) return AR_ERR_ARG;
        if (!aligned16(in[i]) || !aligned16(seg[i])) return AR_ERR_ALIGN;
    }
    for (int r = r0; r < r1; ++r) {
        if (!residual[r] || (fused && (!residual_out[r] || !out[r]))) return AR_ERR_ARG;
        if (!aligned16(residual[r]) || (fused && (!aligned16(residual_out[r]) || !aligned16(out[r]))))
            return AR_ERR_ALIGN;
    }
    if (!aligned16(weight) || !aligned16(flags)) return AR_ERR_ALIGN;
    if ((hidden * es) % 16 != 0 || rows % size_t(n) != 0) return AR_ERR_DIVISIBLE;
    const size_t S = rows * hidden * es, seg_bytes = twoshot_rmsnorm_segment_bytes(n, rows, hidden, dtype);
    std::vector<Span> v;
    v.push_back(span(flags, ar_flag_bytes(n), true));
    v.push_back(span(weight, hidden * es, false));
    for (int i = 0; i < n; ++i) {
        v.push_back(span(in[i], S, false));
        const bool mine = i >= r0 && i < r1;
        if (mine || fused) v.push_back(span(seg[i], seg_bytes, mine));
    }
    for (int r = r0; r < r1; ++r) {
        v.push_back(span(residual[r], S, false));
        if (fused) {
            v.push_back(span(residual_out[r], S, true));
            v.push_back(span(out[r], S, true));
        }
    }
    if (!spans_ok(v)) return AR_ERR_ALIAS;
    return hip_status(launch_twoshot_rmsnorm(in, n, residual, weight, seg, residual_out, out, rows, hidden, eps,
                                             dtype, r0, r1, flags, step, timeout_ticks(),
                                             static_cast<hipStream_t>(stream)));
}

int ar_reduce_bcast(const void* const* in, int n, void* const* out, size_t numel, int dtype, int r0, int r1,
                    void* stream) {
    if (!in || !out || !ranks_ok(n) || !dtype_ok(dtype) || numel == 0) return AR_ERR_ARG;
    if (r0 < 0 || r1 > n || r0 >= r1) return AR_ERR_ARG;
    const size_t es = elem_bytes(dtype);
    if (numel > kMaxBytes / es) return AR_ERR_ARG;
    for (int i = 0; i < n; ++i) {
        if (!in[i] || !out[i]) return AR_ERR_ARG;
        if (!aligned16(in[i]) || !aligned16(out[i])) return AR_ERR_ALIGN;
    }
    const size_t S = numel * es;
    std::vector<Span> v;
    for (int i = 0; i < n; ++i) v.push_back(span(out[i], S, true));
    for (int i = 0; i < n; ++i) v.push_back(span(in[i], S, false));
    if (!spans_ok(v)) return AR_ERR_ALIAS;
    return hip_status(launch_reduce_bcast(in, n, out, numel, dtype, r0, r1, static_cast<hipStream_t>(stream)));
}

int ar_push(const void* const* src, int nsrc, void* const* dst, int ndst, size_t numel, int dtype, void* stream) {
    if (!src || !dst || nsrc < 1 || nsrc > AR_MAX_RANKS || ndst < 1 || ndst > AR_MAX_RANKS || !dtype_ok(dtype) ||
        numel == 0)
        return AR_ERR_ARG;
    const size_t es = elem_bytes(dtype);
    if (numel > kMaxBytes / es) return AR_ERR_ARG;
    const size_t nd = size_t(nsrc) * size_t(ndst);
    for (int i = 0; i < nsrc; ++i) {
        if (!src[i]) return AR_ERR_ARG;
        if (!aligned16(src[i])) return AR_ERR_ALIGN;
    }
    for (size_t j = 0; j < nd; ++j) {
        if (!dst[j]) return AR_ERR_ARG;
        if (!aligned16(dst[j])) return AR_ERR_ALIGN;
    }
    const size_t S = numel * es;
    std::vector<Span> v;
    for (size_t j = 0; j < nd; ++j) v.push_back(span(dst[j], S, true));
    for (int i = 0; i < nsrc; ++i) v.push_back(span(src[i], S, false));
    if (!spans_ok(v)) return AR_ERR_ALIAS;
    return hip_status(launch_push(src, nsrc, dst, ndst, S, static_cast<hipStream_t>(stream)));
}

int ar_twoshot_rs(const void* const* in, int n, void* const* seg, size_t numel, int dtype, int r0, int r1,
                  uint32_t* flags, uint32_t step, void* const* out, void* stream) {
    if (!in) return AR_ERR_ARG;
    const int st = twoshot_check(in, seg, out, n, numel, dtype, r0, r1, flags, step);
    if (st != AR_OK) return st;
    TwoShotRequest rq{in, seg, out, n, numel, dtype, r0, r1, flags, step, true, out != nullptr,
                      timeout_ticks()};
    return hip_status(launch_twoshot(rq, static_cast<hipStream_t>(stream)));
}

int ar_twoshot_ag(const void* const* seg, int n, void* const* out, size_t numel, int dtype, int r0, int r1,
                  uint32_t* flags, uint32_t step, void* stream) {
    if (!out) return AR_ERR_ARG;
    const int st = twoshot_check(nullptr, seg, out, n, numel, dtype, r0, r1, flags, step);
    if (st != AR_OK) return st;
    TwoShotRequest rq{nullptr, const_cast<void* const*>(seg), out, n, numel, dtype, r0, r1, flags, step,
                      false, true, timeout_ticks()};
    return hip_status(launch_twoshot(rq, static_cast<hipStream_t>(stream)));
}

int ar_ll_pack(const void* const* src, void* const* wire, int count, size_t numel, int dtype, int proto,
               uint32_t step, void* stream) {
    // step 0: auto (each line's previous flag + 1)
    if (!src || !wire || count < 1 || count > AR_MAX_RANKS || numel == 0 || !dtype_ok(dtype)) return AR_ERR_ARG;
    if (proto != AR_PROTO_LL && proto != AR_PROTO_LL128) return AR_ERR_ARG;
    const size_t es = elem_bytes(dtype);
    if (numel > kMaxBytes / es) return AR_ERR_ARG;
    for (int i = 0; i < count; ++i) {
        if (!src[i] || !wire[i]) return AR_ERR_ARG;
        if (!aligned16(src[i]) || !aligned16(wire[i])) return AR_ERR_ALIGN;
    }
    const size_t S = numel * es, W = wire_bytes(proto, S);
    std::vector<Span> v;
    for (int i = 0; i < count; ++i) {
        v.push_back(span(src[i], S, false));
        v.push_back(span(wire[i], W, true));
    }
    if (!spans_ok(v)) return AR_ERR_ALIAS;
    return hip_status(launch_ll_pack(src, wire, count, S, proto, step, static_cast<hipStream_t>(stream)));
}

int ar_ll_reduce_unpack(const void* const* wire, int n, void* out, size_t numel, int dtype, uint32_t step,
                        uint32_t* flags, void* stream) {
    return ll_reduce_common(wire, n, out, numel, dtype, step, flags, AR_PROTO_LL, stream);
}

int ar_ll128_reduce_unpack(const void* const* wire, int n, void* out, size_t numel, int dtype, uint32_t step,
                           uint32_t* flags, void* stream) {
    return ll_reduce_common(wire, n, out, numel, dtype, step, flags, AR_PROTO_LL128, stream);
}

int ar_twoshot_ll(const void* const* in, int n, void* const* segw, size_t numel, int dtype, int r0, int r1,
                  uint32_t* flags, uint32_t step, void* const* out, void* stream) {
    if (!in) return AR_ERR_ARG;  // step 0: auto ids, as ar_twoshot_rs
    const int st = twoshot_check(in, segw, out, n, numel, dtype, r0, r1, flags, step, AR_PROTO_LL);
    if (st != AR_OK) return st;
    TwoShotRequest rq{in, segw, out, n, numel, dtype, r0, r1, flags, step, true, out != nullptr,
                      timeout_ticks(), true};
    return hip_status(launch_twoshot(rq, static_cast<hipStream_t>(stream)));
}

int ar_twoshot_ll128(const void* const* in, int n, void* const* segw, size_t numel, int dtype, int r0, int r1,
                     uint32_t* flags, uint32_t step, void* const* out, void* stream) {
    if (!in) return AR_ERR_ARG;  // step 0: auto ids, as ar_twoshot_rs
    const int st = twoshot_check(in, segw, out, n, numel, dtype, r0, r1, flags, step, AR_PROTO_LL128);
    if (st != AR_OK) return st;
    TwoShotRequest rq{in, segw, out, n, numel, dtype, r0, r1, flags, step, true, out != nullptr,
                      timeout_ticks(), false, true};
    return hip_status(launch_twoshot(rq, static_cast<hipStream_t>(stream)));
}

int ar_ll_allreduce(const void* src, void* const* wire, int n, int me, void* out, size_t numel, int dtype,
                    int proto, uint32_t step, uint32_t* flags, void* stream) {
    // step 0: auto (one past the previous flag of rank me's line, line by line)
    if (!ranks_ok(n) || me < 0 || me >= n || !dtype_ok(dtype) || numel == 0 || !src || !wire || !out || !flags)
        return AR_ERR_ARG;
    if (proto != AR_PROTO_LL && proto != AR_PROTO_LL128) return AR_ERR_ARG;
    const size_t es = elem_bytes(dtype);
    if (numel > kMaxBytes / es) return AR_ERR_ARG;
    for (int i = 0; i < n; ++i) {
        if (!wire[i]) return AR_ERR_ARG;
        if (!aligned16(wire[i])) return AR_ERR_ALIGN;
    }
    if (!aligned16(src) || !aligned16(out) || !aligned16(flags)) return AR_ERR_ALIGN;
    const size_t S = numel * es, W = wire_bytes(proto, S);
    std::vector<Span> v;
    v.push_back(span(src, S, false));
    v.push_back(span(out, S, true));
    v.push_back(span(flags, kStatusBytes, true));
    for (int i = 0; i < n; ++i) v.push_back(span(wire[i], W, i == me));
    if (!spans_ok(v)) return AR_ERR_ALIAS;
    return hip_status(launch_ll_allreduce(src, wire, n, me, out, numel, dtype, proto, step, flags, timeout_ticks(),
                                          static_cast<hipStream_t>(stream)));
}

double ar_algo_cost_us(int algo, int n, size_t numel, int dtype, double sync_us) {
    if (algo < AR_ALGO_ONESHOT || algo >= kSelNumAlgos || !ranks_ok(n) || !dtype_ok(dtype) || numel == 0 ||
        !(sync_us >= 0.0))
        return -1.0;
    const size_t es = elem_bytes(dtype);
    if ((algo == AR_ALGO_TWOSHOT || algo == AR_ALGO_TWOSHOT_LL || algo == AR_ALGO_TWOSHOT_LL128) &&
        !(numel % size_t(n) == 0 && (numel / size_t(n) * es) % 16 == 0))
        return -1.0;
    return share_us(algo, n, double(numel) * double(es)) + kSemaphoreSyncs[algo] * sync_us;
}

int ar_select_algo(int n, size_t numel, int dtype, double sync_us) {
    if (!ranks_ok(n) || !dtype_ok(dtype) || numel == 0 || !(sync_us >= 0.0)) return -AR_ERR_ARG;
    int best = AR_ALGO_ONESHOT;
    double best_us = ar_algo_cost_us(best, n, numel, dtype, sync_us);
    for (int a = AR_ALGO_TWOSHOT; a < kSelNumAlgos; ++a) {
        const double t = ar_algo_cost_us(a, n, numel, dtype, sync_us);
        if (t >= 0.0 && t < best_us) best = a, best_us = t;
    }
    return best;
}

int ar_twoshot_ag_copy(const void* const* seg, int n, void* const* out, size_t numel, int dtype, int r0, int r1,
                       uint32_t* flags, uint32_t step, void* stream) {
    if (!out) return AR_ERR_ARG;
    const int st = twoshot_check(nullptr, seg, out, n, numel, dtype, r0, r1, flags, step);
    if (st != AR_OK) return st;
    TwoShotRequest rq{nullptr, const_cast<void* const*>(seg), out, n, numel, dtype, r0, r1, flags, step,
                      false, true, timeout_ticks()};
    return hip_status(launch_twoshot_ag_copy(rq, static_cast<hipStream_t>(stream)));
}

int ar_twoshot_noalloc(const void* const* in, int n, void* const* out, size_t numel, int dtype, void* stream) {
    if (!in || !out || !ranks_ok(n) || !dtype_ok(dtype) || numel == 0) return AR_ERR_ARG;
    const size_t es = elem_bytes(dtype);
    if (numel > kNoAllocMaxBytes / es) return AR_ERR_SIZE;
    for (int i = 0; i < n; ++i) {
        if (!in[i] || !out[i]) return AR_ERR_ARG;
        if (!aligned16(in[i]) || !aligned16(out[i])) return AR_ERR_ALIGN;
    }
    if (numel % size_t(n) != 0 || (numel / size_t(n) * es) % 16 != 0) return AR_ERR_DIVISIBLE;
    const size_t S = numel * es, m_bytes = S / size_t(n);
    std::vector<Span> v;
    for (int i = 0; i < n; ++i) v.push_back(span(in[i], S, false));
    for (int r = 0; r < n; ++r) v.push_back(span(out[r], S, true));
    if (!spans_ok(v)) return AR_ERR_ALIAS;
    void* base = nullptr;
    if (noalloc_scratch(&base) != hipSuccess) return AR_ERR_HIP;
    uint32_t* flags = static_cast<uint32_t*>(base);
    void* seg[AR_MAX_RANKS];
    for (int j = 0; j < n; ++j) seg[j] = static_cast<unsigned char*>(base) + kNoAllocFlagBytes + size_t(j) * m_bytes;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // every call starts from zeroed slots and uses step 1: nothing a previous
    // call left (another n, a timeout) can let a wait pass early
    hipError_t e = launch_flag_reset(flags, size_t(kStatusWords) + size_t(n) * kSlotsPerRank, s);
    if (e != hipSuccess) return AR_ERR_HIP;
    TwoShotRequest rq{in, seg, out, n, numel, dtype, 0, n, flags, 1u, true, true, timeout_ticks()};
    return hip_status(launch_twoshot(rq, s));
}

int ar_flag_barrier_reset(uint32_t* flags, int n, void* stream) {
    if (!flags || !ranks_ok(n)) return AR_ERR_ARG;
    if (!aligned16(flags)) return AR_ERR_ALIGN;
    return hip_status(launch_flag_reset(flags, ar_flag_bytes(n) / 4, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
