// LL and LL128 flag-packed protocols for gfx950 ("集合通信：NCCL 的算法、协议与
// 推理框架的定制 all-reduce", 协议 table): the sender packs its message into
// lines that carry their own flag (the step id); the receiver polls the flags,
// takes the data out and reduces the n messages exactly as the one-shot path.
//
// LL line  : 8 bytes  = 4 data bytes, then a 32-bit flag.
// LL128 line: 128 bytes = 120 data bytes, then a 64-bit flag.
// Data bytes past the message in the last line are zero.
//
// LL receiver: up to 16 MiB per rank a lane owns one line of every rank (one
// 8-byte load per rank) and produces 4 output bytes; above, 16 wire bytes of
// every rank (2 lines, one 16-byte load per rank) and 8 output bytes.
// LL128 receiver: a wavefront owns 1 KiB of wire per rank = 8 lines; lane l
// holds 16 bytes at part l % 8 of line l / 8, and the lane at part 7 holds 8
// data bytes plus the flag.  Readiness of the whole wavefront is one ballot.
// If a line is behind, the slow path re-reads with agent-coherent 64-bit
// atomic loads until every flag is >= step or the wall-clock budget runs out.
//
// Send and receive in one launch (one GPU's LL step): the one-line LL
// receiver and the LL128 receiver also take rank me's message.  Each lane
// reads the message bytes its line position carries, writes rank me's line
// (data and flag) to rank me's wire for the peers, and uses those bytes as
// rank me's term of the fold, in rank order; rank me's wire is not read.
#include "ar_device.hpp"
#include "ar_launch.hpp"

namespace ar {
namespace {

constexpr int kBlock = 256;
// LL receiver: one wavefront per workgroup (measured 5% faster than four at
// 128 KiB, 8 MiB and 64 MiB per rank, 5% slower at 1 MiB).
constexpr int kBlockLL = kWave;
// Messages up to this many bytes per rank take the one-line LL receiver.
constexpr size_t kOneLineMaxBytes = size_t(16) << 20;
// LL128 receiver: one wavefront per workgroup (measured faster than four at
// every size from 128 KiB to 8 MiB per rank: more, smaller workgroups spread
// the few waves of a small message over more CUs).
constexpr int kBlock128 = kWave;
constexpr int kWavesPerBlock128 = 1;

// ------------------------------------------------------------------ pack --
struct PackParams {
    const uint8_t* src[kMaxRanks];
    uint8_t* wire[kMaxRanks];
    size_t nbytes;
    uint32_t step;
};

// LL pack: lane c takes message bytes [8c, 8c+8) and writes the 16 wire
// bytes of lines 2c and 2c+1, so each load instruction of a wavefront reads
// 512 contiguous bytes and each store writes 1 KiB of whole lines.  A lane
// handles kPackUnroll chunks kBlock apart.  blockIdx.y selects the message.
// The lane whose chunk runs past the end reads byte by byte, zero-fills,
// and writes only the lines that exist.
template <int kPackUnroll>
__global__ __launch_bounds__(kBlock) void ll_pack_kernel(PackParams p) {
    const uint8_t* src = p.src[blockIdx.y];
    u32x4* wire = reinterpret_cast<u32x4*>(p.wire[blockIdx.y]);
    const size_t full = p.nbytes / 8;          // whole 8-byte chunks
    const size_t lines = (p.nbytes + 3) / 4;   // = words
    const size_t c0 = size_t(blockIdx.x) * (kBlock * kPackUnroll) + threadIdx.x;
    u32x2 v[kPackUnroll];
    u32x4 old[kPackUnroll];  // auto step ids: the two lines as the last call left them
#pragma unroll
    for (int u = 0; u < kPackUnroll; ++u) {
        const size_t c = c0 + size_t(u) * kBlock;
        if (c < full) {
            v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src) + c);
            if (p.step == 0) old[u] = __builtin_nontemporal_load(wire + c);
        }
    }
#pragma unroll
    for (int u = 0; u < kPackUnroll; ++u) {
        const size_t c = c0 + size_t(u) * kBlock;
        if (c < full) {
            const uint32_t s0 = p.step != 0 ? p.step : old[u].y + 1u;
            const uint32_t s1 = p.step != 0 ? p.step : old[u].w + 1u;
            st_stream(wire + c, u32x4{v[u].x, s0, v[u].y, s1});
        } else if (2 * c < lines) {
            uint32_t w[2] = {0u, 0u};
            for (size_t b = 8 * c; b < p.nbytes; ++b) w[(b >> 2) & 1] |= uint32_t(src[b]) << (8 * (b & 3));
            u32x2* ln = reinterpret_cast<u32x2*>(p.wire[blockIdx.y]);
            ln[2 * c] = u32x2{w[0], p.step != 0 ? p.step : ln[2 * c].y + 1u};
            if (2 * c + 1 < lines) ln[2 * c + 1] = u32x2{w[1], p.step != 0 ? p.step : ln[2 * c + 1].y + 1u};
        }
    }
}

// LL128 pack: 8 lanes per line, lane part q writes wire bytes [16q, 16q+16)
// of its line; parts 0..6 carry data bytes [120L+16q, +16), part 7 carries
// data bytes [120L+112, +8) and the 64-bit flag.
__global__ __launch_bounds__(kBlock) void ll128_pack_kernel(PackParams p, size_t nlines) {
    const uint8_t* src = p.src[blockIdx.y];
    u32x4* wire = reinterpret_cast<u32x4*>(p.wire[blockIdx.y]);
    const size_t g = size_t(blockIdx.x) * kBlock + threadIdx.x;
    const size_t line = g / 8;
    const uint32_t part = uint32_t(g % 8);
    if (line >= nlines) return;
    const size_t off = line * 120 + size_t(part) * 16;
    const uint32_t data_bytes = part == 7 ? 8u : 16u;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (off + data_bytes <= p.nbytes) {
        // 8-byte aligned (120 L + 16 q is a multiple of 8)
        const u32x2* s = reinterpret_cast<const u32x2*>(src + off);
        const u32x2 a = s[0];
        w[0] = a.x; w[1] = a.y;
        if (part != 7) { const u32x2 b = s[1]; w[2] = b.x; w[3] = b.y; }
    } else {
        for (size_t b = off; b < p.nbytes && b < off + data_bytes; ++b)
            w[((b - off) >> 2) & 3] |= uint32_t(src[b]) << (8 * (b & 3));
    }
    if (part == 7) {  // 64-bit flag = step, little endian; auto: the line's last flag + 1
        w[2] = p.step != 0 ? p.step : reinterpret_cast<const uint32_t*>(p.wire[blockIdx.y])[line * 32 + 30] + 1u;
        w[3] = 0u;
    }
    st_stream(wire + line * 8 + part, u32x4{w[0], w[1], w[2], w[3]});
}

// ---------------------------------------------------------------- reduce --
struct ReduceParams {
    const uint8_t* wire[kMaxRanks];
    uint8_t* out;
    uint32_t* flags;
    uint64_t timeout_ticks;
    size_t nbytes;
    size_t nlines;  // lines per rank
    uint32_t step;
    // send and receive in one launch: rank me's message and wire
    int me;
    const uint8_t* src;
    uint8_t* own_wire;
};

// Bounded wait for the lines [2c, 2c + nl) of every rank (nl = 1 or 2) to
// reach step ids s0 (line 2c) and s1 (line 2c + 1), re-read with
// agent-coherent atomic 64-bit loads into x (data in .x/.z, flags in .y/.w).
// Lanes with nl == 0 just take part in the ballots.  Returns false on
// timeout (reported).
template <int NR>
__device__ bool ll_slow_wait(const ReduceParams& p, size_t c, uint32_t nl, u32x4 (&x)[NR], int lane, uint32_t s0,
                             uint32_t s1) {
    const uint64_t t0 = now_ticks();
    while (true) {
        bool ok = true;
        int bad_r = 0;
        uint32_t bad_l = 0;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const uint64_t* w = reinterpret_cast<const uint64_t*>(p.wire[r]) + 2 * c;
            if (nl > 0 && x[r].y < s0) {
                const uint64_t a = line_load_relaxed(w);
                x[r].x = uint32_t(a);
                x[r].y = uint32_t(a >> 32);
                if (x[r].y < s0 && ok) { ok = false; bad_r = r; bad_l = 0; }
            }
            if (nl > 1 && x[r].w < s1) {
                const uint64_t b = line_load_relaxed(w + 1);
                x[r].z = uint32_t(b);
                x[r].w = uint32_t(b >> 32);
                if (x[r].w < s1 && ok) { ok = false; bad_r = r; bad_l = 1; }
            }
        }
        const uint64_t missing = ~wave_ballot(ok) & wave_exec();
        if (missing == 0) return true;
        if (now_ticks() - t0 > p.timeout_ticks) {
            const int bl = __ffsll((unsigned long long)missing) - 1;
            if (lane == bl) report_timeout(p.flags, kPhaseLl, uint32_t(bad_r), uint32_t(2 * c + bad_l));
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

template <typename T>
__device__ __forceinline__ void store_out_bytes(uint8_t* out, size_t off, size_t nbytes, const uint32_t* words) {
    for (size_t b = off; b < nbytes; b += elem<T>::bytes) {
        const uint32_t word = words[(b - off) >> 2];
        if (elem<T>::bytes == 4) *reinterpret_cast<uint32_t*>(out + b) = word;
        else *reinterpret_cast<uint16_t*>(out + b) = uint16_t(word >> (8 * (b & 2)));
    }
}

// LL receiver.  Lane chunk c = lines 2c and 2c+1 of every rank (one 16-byte
// load per rank; a wavefront's load instruction reads 1 KiB of whole lines)
// and output bytes [8c, 8c+8).  A lane handles U chunks kBlockLL apart.  The
// main path is branch-free: lanes past the last two-line chunk load a valid
// clamped chunk and discard it, so all U * n loads issue back to back.  A
// final single line (odd line count) is finished by one lane on its own.
//
// kFused (one chunk per lane): rank me's term is bytes [8c, 8c+8) of its
// message, loaded with the peers' lines by every wavefront whose 64 chunks
// all exist and word by word in the last one (a lone bf16 in the chunk's
// second line is zero-extended); lines 2c and 2c+1 of rank me's wire are
// written from it, each with its step id, before the wavefront waits on any
// peer, or last when nothing has to be waited for.  The odd last line is
// sent the same way by its lane.
template <typename T, int NR, int U, bool kFused>
__global__ __launch_bounds__(kBlockLL) void ll_reduce_kernel(ReduceParams p) {
    static_assert(!kFused || U == 1, "send and receive take one chunk per lane");
    const int lane = threadIdx.x & (kWave - 1);
    const size_t nfull = p.nlines / 2;  // chunks that hold two lines
    const size_t c0 = size_t(blockIdx.x) * (kBlockLL * U) + threadIdx.x;
    const u32x4* w[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) w[r] = reinterpret_cast<const u32x4*>(p.wire[r]);
    // A last chunk with a single line (odd line count): chunk nfull, finished
    // by the one lane of the grid that owns that chunk index.
    const size_t rel = nfull - size_t(blockIdx.x) * (kBlockLL * U);
    const bool odd_owner = (p.nlines & 1) && nfull >= size_t(blockIdx.x) * (kBlockLL * U) &&
                           rel < size_t(kBlockLL) * U && rel % kBlockLL == threadIdx.x;
    // kFused: that lane sends rank me's last line (message bytes
    // [8 nfull, nbytes), 2 or 4) first, before its wavefront waits on anything
    uint32_t odd_own = 0u, odd_step = p.step;
    if constexpr (kFused) {
        if (odd_owner) {
            odd_own = 8 * nfull + 4 <= p.nbytes ? reinterpret_cast<const uint32_t*>(p.src)[2 * nfull]
                                                : uint32_t(reinterpret_cast<const uint16_t*>(p.src)[4 * nfull]);
            u32x2* ln = reinterpret_cast<u32x2*>(p.own_wire) + 2 * nfull;
            if (p.step == 0) odd_step = ln->y + 1u;
            *ln = u32x2{odd_own, odd_step};
        }
    }

    if (nfull > 0) {
        u32x4 x[U][NR];
        bool act[U];
        // kFused: rank me's 8 message bytes and (auto step ids, step 0) its
        // two lines as the last call left them
        const bool own_whole = kFused && (size_t(blockIdx.x) + 1) * kBlockLL * 8 <= p.nbytes;  // wavefront-uniform
        u32x2 own = u32x2{0u, 0u};
        u32x4 own_old = u32x4{0u, 0u, 0u, 0u};
        if constexpr (kFused) {
            const size_t cc = c0 < nfull ? c0 : nfull - 1;
            if (own_whole) own = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p.src) + c0);
            if (p.step == 0) own_old = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.own_wire) + cc);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t c = c0 + size_t(u) * kBlockLL;
            act[u] = c < nfull;
            const size_t cc = act[u] ? c : nfull - 1;
            // kFused: rank me's slot too (it holds a peer's wire; the term is
            // replaced below) -- skipping it, the compiler waited between loads
#pragma unroll
            for (int r = 0; r < NR; ++r) x[u][r] = ld_stream(w[r] + cc);
        }
        // Keep every load ahead of the first use: left alone, the scheduler
        // sometimes hoists a flag compare between the loads, and the wait it
        // needs then serialises two memory round trips.
        __builtin_amdgcn_sched_barrier(0);
        // the step ids of lines 2c and 2c+1: the call's, or (auto) one past
        // the last flag of each of rank me's two lines
        uint32_t s0 = p.step, s1 = p.step;
        bool own_late = false;
        if constexpr (kFused) {
            if (!own_whole && act[0]) {
                // the last wavefront: line 2c is whole (the chunk has two
                // lines); line 2c+1 may hold a lone bf16
                own.x = reinterpret_cast<const uint32_t*>(p.src)[2 * c0];
                own.y = 8 * c0 + 8 <= p.nbytes ? reinterpret_cast<const uint32_t*>(p.src)[2 * c0 + 1]
                                               : uint32_t(reinterpret_cast<const uint16_t*>(p.src)[4 * c0 + 2]);
            }
            if (p.step == 0) { s0 = own_old.y + 1u; s1 = own_old.w + 1u; }
            // rank me's lines carry their step ids: the readiness checks pass them
#pragma unroll
            for (int r = 0; r < NR; ++r)
                if (r == p.me) x[0][r] = u32x4{own.x, s0, own.y, s1};
        }
        // Readiness without short-circuit branches: the smallest flag a lane
        // holds, folded with min as the loads land.
        bool ok = true;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (kFused) {
                uint32_t f0 = 0xFFFFFFFFu, f1 = 0xFFFFFFFFu;
#pragma unroll
                for (int r = 0; r < NR; ++r) { f0 = min(f0, x[u][r].y); f1 = min(f1, x[u][r].w); }
                ok &= !act[u] | ((f0 >= s0) & (f1 >= s1));
            } else {
                uint32_t fmin = 0xFFFFFFFFu;
#pragma unroll
                for (int r = 0; r < NR; ++r) fmin = min(fmin, min(x[u][r].y, x[u][r].w));
                ok &= !act[u] | (fmin >= p.step);
            }
        }
        if (wave_ballot(!ok) != 0) {
            // kFused: rank me's lines go out before any wait on a peer
            if (kFused && act[0]) st_stream(reinterpret_cast<u32x4*>(p.own_wire) + c0, u32x4{own.x, s0, own.y, s1});
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (!ll_slow_wait<NR>(p, c0 + size_t(u) * kBlockLL, act[u] ? 2u : 0u, x[u], lane, s0, s1)) return;
            if constexpr (kFused) wait_stores();  // nothing of this path left to wait for where the paths join
        } else if (kFused && act[0]) {
            own_late = true;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t c = c0 + size_t(u) * kBlockLL;
            Acc8<T> acc;
#pragma unroll
            for (int r = 0; r < NR; ++r) acc.add(x[u][r].x, x[u][r].z);
            const u32x2 res = acc.result();
            if (act[u]) {
                if (8 * c + 8 <= p.nbytes) {
                    __builtin_nontemporal_store(res, reinterpret_cast<u32x2*>(p.out) + c);
                } else {
                    const uint32_t rw[2] = {res.x, res.y};
                    store_out_bytes<T>(p.out, 8 * c, p.nbytes, rw);
                }
            }
        }
        if (kFused && own_late) st_stream(reinterpret_cast<u32x4*>(p.own_wire) + c0, u32x4{own.x, s0, own.y, s1});
    }
    if (odd_owner) {
        u32x4 x[NR];
        const uint32_t step = odd_step;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const u32x2 a = reinterpret_cast<const u32x2*>(p.wire[r])[2 * nfull];
            x[r] = u32x4{a.x, a.y, 0u, 0xFFFFFFFFu};
        }
        if constexpr (kFused) {
#pragma unroll
            for (int r = 0; r < NR; ++r)
                if (r == p.me) x[r] = u32x4{odd_own, step, 0u, 0xFFFFFFFFu};
        }
        bool ok = true;
#pragma unroll
        for (int r = 0; r < NR; ++r) ok = ok && x[r].y >= step;
        if (!ok) {
            // single lane: poll alone (its own wave's ballot sees only it)
            const uint64_t t0 = now_ticks();
            while (!ok) {
                ok = true;
                int bad_r = 0;
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    if (x[r].y < step) {
                        const uint64_t a =
                            line_load_relaxed(reinterpret_cast<const uint64_t*>(p.wire[r]) + 2 * nfull);
                        x[r].x = uint32_t(a);
                        x[r].y = uint32_t(a >> 32);
                        if (x[r].y < step && ok) { ok = false; bad_r = r; }
                    }
                }
                if (!ok && now_ticks() - t0 > p.timeout_ticks) {
                    report_timeout(p.flags, kPhaseLl, uint32_t(bad_r), uint32_t(2 * nfull));
                    return;
                }
                if (!ok) __builtin_amdgcn_s_sleep(1);
            }
        }
        Acc8<T> acc;
#pragma unroll
        for (int r = 0; r < NR; ++r) acc.add(x[r].x, 0u);
        const u32x2 res = acc.result();
        const uint32_t rw[2] = {res.x, res.y};
        store_out_bytes<T>(p.out, 8 * nfull, p.nbytes, rw);
    }
}

// LL receiver, one line per lane: lane c owns line c of every rank (one
// 8-byte load per rank: 4 data bytes and the flag) and output bytes
// [4c, 4c+4).  Half the elements per lane of the two-line kernel and twice
// the wavefronts; measured faster up to 16 MiB per rank (n = 16 at 1 MiB:
// 8.6 -> 7.4 us; n = 8 at 1-8 MiB: 3-4%), slower above (n = 16 at 64 MiB:
// 342 -> 363 us), where the two-line kernel runs.
//
// kFused: rank me's term is word c of its message (message bytes [4c, 4c+4);
// a final lone bf16 is zero-extended), loaded with the peers' lines by every
// wavefront whose 64 words all exist and one by one in the last wavefront;
// line c of rank me's wire is written from it, with the flag, before the
// wavefront waits on any peer.
template <typename T, int NR, bool kFused>
__global__ __launch_bounds__(kBlockLL) void ll_reduce1_kernel(ReduceParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const size_t c = size_t(blockIdx.x) * kBlockLL + threadIdx.x;
    const bool act = c < p.nlines;
    const size_t cc = act ? c : p.nlines - 1;
    const size_t words = p.nbytes / 4;  // whole 4-byte words of the message
    const bool own_whole = kFused && (size_t(blockIdx.x) + 1) * kBlockLL <= words;  // wavefront-uniform
    uint32_t own = 0;
    bool own_late = false;
    if (kFused && own_whole) own = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p.src) + c);
    // auto step ids (step 0): rank me's line c as the last call left it
    u32x2 own_old = u32x2{0u, 0u};
    if (kFused && p.step == 0) own_old = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p.own_wire) + cc);
    // the last wavefront's word of rank me, ahead of the peers' loads, so
    // that the wait for it where the paths join leaves those in flight
    if constexpr (kFused) {
        if (!own_whole && act)
            own = c < words ? reinterpret_cast<const uint32_t*>(p.src)[c]
                            : uint32_t(reinterpret_cast<const uint16_t*>(p.src)[2 * c]);
    }
    // every slot, rank me's too (in the send-and-receive form it holds a
    // peer's wire, and its term is replaced below): a branch around one load
    // makes the merge of the paths wait for every load
    u32x2 x[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) x[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p.wire[r]) + cc);
    __builtin_amdgcn_sched_barrier(0);  // every load ahead of the first use
    // the step id of this lane's line: the call's, or (auto) one past the
    // last flag of rank me's line, every call advancing every line by one
    const uint32_t step = kFused && p.step == 0 ? own_old.y + 1u : p.step;
    if constexpr (kFused) {
        // rank me's line carries the step: the readiness checks pass it
#pragma unroll
        for (int r = 0; r < NR; ++r)
            if (r == p.me) x[r] = u32x2{own, step};
    }
    // The fold runs as the loads land, ahead of the flag check, and is done
    // again on the slow path.
    auto fold = [&]() -> uint32_t {
        if (elem<T>::bytes == 4) {
            float a = 0.0f;
#pragma unroll
            for (int r = 0; r < NR; ++r) a = a + __uint_as_float(x[r].x);
            return __float_as_uint(a);
        } else {
            float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
            for (int r = 0; r < NR; ++r) { a0 = a0 + bf16_lo(x[r].x); a1 = a1 + bf16_hi(x[r].x); }
            return pack_bf16x2(a0, a1);
        }
    };
    uint32_t word = fold();
    uint32_t fmin = 0xFFFFFFFFu;
#pragma unroll
    for (int r = 0; r < NR; ++r) fmin = min(fmin, x[r].y);
    bool ok = !act | (fmin >= step);
    // kFused: rank me's line for its peers goes out before any wait on a peer
    // (slow path) or, when every line is already there, last, after the
    // output (a store issued earlier is waited for by the compiler's later
    // waits: stores and loads count in one counter).
    if (wave_ballot(!ok) != 0) {
        if (kFused && act) __builtin_nontemporal_store(u32x2{own, step}, reinterpret_cast<u32x2*>(p.own_wire) + c);
        const uint64_t t0 = now_ticks();
        while (true) {
            bool good = true;
            int bad_r = 0;
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                if (act && x[r].y < step) {
                    const uint64_t a = line_load_relaxed(reinterpret_cast<const uint64_t*>(p.wire[r]) + c);
                    x[r].x = uint32_t(a);
                    x[r].y = uint32_t(a >> 32);
                    if (x[r].y < step && good) { good = false; bad_r = r; }
                }
            }
            const uint64_t missing = ~wave_ballot(good) & wave_exec();
            if (missing == 0) break;
            if (now_ticks() - t0 > p.timeout_ticks) {
                const int bl = __ffsll((unsigned long long)missing) - 1;
                if (lane == bl) report_timeout(p.flags, kPhaseLl, uint32_t(bad_r), uint32_t(c));
                return;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        wait_stores();  // nothing of this path left to wait for where the paths join
        word = fold();
    } else if (kFused && act) {
        own_late = true;
    }
    if (!act) return;
    if (4 * c + 4 <= p.nbytes) {
        __builtin_nontemporal_store(word, reinterpret_cast<uint32_t*>(p.out) + c);
    } else {
        const uint32_t rw[1] = {word};
        store_out_bytes<T>(p.out, 4 * c, p.nbytes, rw);
    }
    if (kFused && own_late) __builtin_nontemporal_store(u32x2{own, step}, reinterpret_cast<u32x2*>(p.own_wire) + c);
}

// kFused: rank me's term at a lane is the message bytes its line position
// carries ([120 line + 16 part, +16), 8 bytes at part 7, zero past the
// message), loaded with the peers' lines by every wavefront whose 8 lines
// are whole and word by word in the last one; rank me's wire gets the line
// (part 7 adds the flag) from it.  Rank me's slot of the wire table holds a
// peer's wire: every slot is loaded unconditionally (a branch around one
// load left that register undefined on one path, and the copies merging the
// paths waited for every load), and the fold takes rank me's term instead.
template <typename T, int NR, int U, bool kFused>
__global__ __launch_bounds__(kBlock128) void ll128_reduce_kernel(ReduceParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t part = uint32_t(lane) & 7u;
    const size_t wave = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerBlock128 + threadIdx.x / kWave);
    u32x4 x[U][NR];
    size_t line[U];
    bool valid[U];
    const u32x4* w[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) w[r] = reinterpret_cast<const u32x4*>(p.wire[r]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        line[u] = (wave * U + u) * 8 + size_t(lane) / 8;
        valid[u] = line[u] < p.nlines;
    }
    uint32_t own[U][4] = {};
    u32x4 mine[U];
    bool own_whole[U];
    // the step id of each unit's line: the call's, or (auto, step 0) one past
    // the last flag of rank me's line, read by the line's lanes with the loads
    uint32_t step[U];
#pragma unroll
    for (int u = 0; u < U; ++u) step[u] = p.step;
    // kFused: rank me's bytes first, so that the fold, which runs as the loads
    // land, is not held up by the last load for rank me's term
    if constexpr (kFused) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (p.step == 0) {
                const size_t ll = valid[u] ? line[u] : p.nlines - 1;
                step[u] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p.own_wire) + ll * 32 + 30);
            }
            // wavefront-uniform: every data byte of the unit's 8 lines exists
            own_whole[u] = ((wave * U + u) * 8 + 8) * 120 <= p.nbytes;
            if (own_whole[u]) {
                // 8-byte aligned (120 line + 16 part); part 7 reads its 8 bytes twice
                const u32x2* sp = reinterpret_cast<const u32x2*>(p.src + line[u] * 120 + size_t(part) * 16);
                const u32x2 a = __builtin_nontemporal_load(sp);
                const u32x2 b = __builtin_nontemporal_load(sp + (part != 7u ? 1 : 0));
                own[u][0] = a.x; own[u][1] = a.y; own[u][2] = b.x; own[u][3] = b.y;
            }
        }
    }
    if constexpr (kFused) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (!own_whole[u] && valid[u]) {
                // the last wavefront: each word on its own, independent loads
                // (4-byte aligned: 120 line + 16 part is a multiple of 8); a
                // final lone bf16 is zero-extended, bytes past it stay zero.
                // Issued before the peers' loads: a wait for these where the
                // paths join then leaves the peers' loads in flight
                const size_t off = line[u] * 120 + size_t(part) * 16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const size_t b = off + 4 * size_t(i);
                    if (i < (part == 7u ? 2 : 4)) {
                        if (b + 4 <= p.nbytes) own[u][i] = *reinterpret_cast<const uint32_t*>(p.src + b);
                        else if (b + 2 <= p.nbytes) own[u][i] = *reinterpret_cast<const uint16_t*>(p.src + b);
                    }
                }
            }
        }
    }
    // Branch-free loads: lines past the end read the last line instead and
    // are discarded.
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const size_t ll = valid[u] ? line[u] : p.nlines - 1;
#pragma unroll
        for (int r = 0; r < NR; ++r) x[u][r] = ld_stream(w[r] + ll * 8 + part);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load ahead of the first use
    if constexpr (kFused) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (p.step == 0) step[u] += 1u;
            if (part == 7u) { own[u][2] = step[u]; own[u][3] = 0u; }  // 64-bit flag = step
            mine[u] = u32x4{own[u][0], own[u][1], own[u][2], own[u][3]};
        }
    }
    // The fold runs as the loads land, ahead of the flag check, and is done
    // again on the slow path.  Every lane adds all 16 bytes, so the wavefront
    // does not split: at part 7 the upper 8 are the flag, and the result words
    // they give are never stored.
    u32x4 res[U];
    auto fold = [&]() {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            Acc<T> acc;
#pragma unroll
            for (int r = 0; r < NR; ++r) acc.add(kFused && r == p.me ? mine[u] : x[u][r]);
            res[u] = acc.result();
        }
    };
    fold();
    // rank me's line for the peers once every load has landed: a store among
    // loads still in flight would make each later load wait a wait for the
    // store too (one counter), so it is kept below the fold
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kFused) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (valid[u]) st_stream(reinterpret_cast<u32x4*>(p.own_wire) + line[u] * 8 + part, mine[u]);
    }
    // Readiness without short-circuit branches: the lane at part 7 folds the
    // low flag words with min, a nonzero high word counting as ready.
    bool ok = true;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        uint32_t fmin = 0xFFFFFFFFu;
#pragma unroll
        for (int r = 0; r < NR; ++r) fmin = min(fmin, x[u][r].w != 0u ? 0xFFFFFFFFu : x[u][r].z);
        ok &= !valid[u] | (part != 7u) | (fmin >= step[u]);
    }
    if (wave_ballot(!ok) != 0) {
        // Slow path: poll the flags with coherent 64-bit loads, then re-read
        // the data of every line after an acquire fence and fold again.
        const uint64_t t0 = now_ticks();
        while (true) {
            bool ready = true;
            int bad_r = 0;
            size_t bad_line = 0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    if (valid[u] && part == 7u) {
                        const uint64_t f = line_load_relaxed(
                            reinterpret_cast<const uint64_t*>(p.wire[r] + line[u] * 128 + 120));
                        if (f < uint64_t(step[u]) && ready) { ready = false; bad_r = r; bad_line = line[u]; }
                    }
                }
            }
            const uint64_t missing = ~wave_ballot(ready) & wave_exec();
            if (missing == 0) break;
            if (now_ticks() - t0 > p.timeout_ticks) {
                const int bl = __ffsll((unsigned long long)missing) - 1;
                const int rr = __shfl(bad_r, bl);
                const uint32_t ll = uint32_t(__shfl(uint32_t(bad_line), bl));
                if (lane == bl) report_timeout(p.flags, kPhaseLl128, uint32_t(rr), ll);
                return;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        fence_acquire_agent();
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (valid[u])
#pragma unroll
                for (int r = 0; r < NR; ++r)
                    x[u][r] = ld_plain(reinterpret_cast<const u32x4*>(p.wire[r]) + line[u] * 8 + part);
        // Wait for the re-reads here, so that where the two paths join the
        // compiler has no load of this path to wait for; its wait would also
        // cover rank me's line store (stores count in the same counter), a
        // memory round trip.
        wait_stores();
        fold();
    }
    // Repack through LDS: the 8 lines of a wavefront unit hold 960
    // contiguous output bytes (16-byte aligned, as 960 = 60 * 16), but a
    // lane's piece starts at 120 * line + 16 * part, only 8-byte aligned.
    // Write the pieces to a wavefront-private LDS strip, then let lanes 0..59
    // store 16 aligned bytes each.
    __shared__ __attribute__((aligned(16))) uint8_t strip[kWavesPerBlock128][U][960];
    uint8_t* my = &strip[threadIdx.x / kWave][0][0];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        u32x2* d = reinterpret_cast<u32x2*>(my + u * 960 + (lane / 8) * 120 + part * 16);
        d[0] = u32x2{res[u].x, res[u].y};
        if (part != 7u) d[1] = u32x2{res[u].z, res[u].w};
    }
    // LDS-only fences: a workgroup fence over every address space would also
    // wait for this wavefront's outstanding global stores (rank me's line in
    // the send-and-receive form), a memory round trip the strip does not need.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    if (lane < 60) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t off = (wave * U + u) * 960 + size_t(lane) * 16;
            const u32x4 v = *reinterpret_cast<const u32x4*>(my + u * 960 + lane * 16);
            if (off + 16 <= p.nbytes) {
                st_stream(reinterpret_cast<u32x4*>(p.out + off), v);
            } else if (off < p.nbytes) {
                const uint32_t rw[4] = {v.x, v.y, v.z, v.w};
                for (size_t b = off; b < p.nbytes; b += elem<T>::bytes) {
                    const uint32_t word = rw[(b - off) >> 2];
                    if (elem<T>::bytes == 4) *reinterpret_cast<uint32_t*>(p.out + b) = word;
                    else *reinterpret_cast<uint16_t*>(p.out + b) = uint16_t(word >> (8 * (b & 2)));
                }
            }
        }
    }
}

template <typename T, int NR>
hipError_t launch_reduce_t(const ReduceParams& p, int proto, hipStream_t s) {
    if (proto == 0 && p.nbytes <= kOneLineMaxBytes) {
        const size_t grid = (p.nlines + kBlockLL - 1) / kBlockLL;
        hipLaunchKernelGGL((ll_reduce1_kernel<T, NR, false>), dim3(uint32_t(grid)), dim3(kBlockLL), 0, s, p);
    } else if (proto == 0) {
        // One 16-byte load (two lines) per lane per rank: measured faster
        // than two from 128 KiB to 8 MiB per rank (more workgroups in flight)
        // and equal within a few percent at 64 MiB.
        constexpr int U = 1;
        const size_t chunks = (p.nlines + 1) / 2;
        const size_t grid = (chunks + kBlockLL * U - 1) / (kBlockLL * U);
        hipLaunchKernelGGL((ll_reduce_kernel<T, NR, U, false>), dim3(uint32_t(grid)), dim3(kBlockLL), 0, s, p);
    } else {
        // One 8-line unit per wavefront: measured faster than two for every
        // size, and the two-unit fp32 instantiation stalls badly.
        constexpr int U = 1;
        const size_t wave_units = (p.nlines + 7) / 8;
        const size_t waves = (wave_units + U - 1) / U;
        const size_t grid = (waves + kWavesPerBlock128 - 1) / kWavesPerBlock128;
        hipLaunchKernelGGL((ll128_reduce_kernel<T, NR, U, false>), dim3(uint32_t(grid)), dim3(kBlock128), 0, s, p);
    }
    return hipGetLastError();
}

// Send and receive in one launch, LL with the receivers' line split: one
// line per lane up to 16 MiB per rank, two above.
template <typename T, int NR>
hipError_t launch_fused_t(const ReduceParams& p, int proto, hipStream_t s) {
    if (proto == 0 && p.nbytes > kOneLineMaxBytes) {
        const size_t chunks = (p.nlines + 1) / 2;
        const size_t grid = (chunks + kBlockLL - 1) / kBlockLL;
        hipLaunchKernelGGL((ll_reduce_kernel<T, NR, 1, true>), dim3(uint32_t(grid)), dim3(kBlockLL), 0, s, p);
    } else if (proto == 0) {
        const size_t grid = (p.nlines + kBlockLL - 1) / kBlockLL;
        hipLaunchKernelGGL((ll_reduce1_kernel<T, NR, true>), dim3(uint32_t(grid)), dim3(kBlockLL), 0, s, p);
    } else {
        const size_t grid = (p.nlines + 7) / 8;
        hipLaunchKernelGGL((ll128_reduce_kernel<T, NR, 1, true>), dim3(uint32_t(grid)), dim3(kBlock128), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ll_pack(const void* const* src, void* const* wire, int count, size_t nbytes,
                          int proto, uint32_t step, hipStream_t s) {
    PackParams p{};
    for (int i = 0; i < count; ++i) {
        p.src[i] = static_cast<const uint8_t*>(src[i]);
        p.wire[i] = static_cast<uint8_t*>(wire[i]);
    }
    p.nbytes = nbytes;
    p.step = step;
    if (proto == 0) {
        // Four chunks per lane once the grid still spans every CU several
        // times over; one per lane for small messages, which want many
        // workgroups rather than deep ones.
        const size_t chunks = (nbytes + 7) / 8;
        if (chunks >= size_t(kBlock) * 4 * 2048) {
            const size_t grid = (chunks + kBlock * 4 - 1) / (kBlock * 4);
            hipLaunchKernelGGL(ll_pack_kernel<4>, dim3(uint32_t(grid), uint32_t(count)), dim3(kBlock), 0, s, p);
        } else {
            const size_t grid = (chunks + kBlock - 1) / kBlock;
            hipLaunchKernelGGL(ll_pack_kernel<1>, dim3(uint32_t(grid), uint32_t(count)), dim3(kBlock), 0, s, p);
        }
    } else {
        const size_t nlines = (nbytes + 119) / 120;
        const size_t grid = (nlines * 8 + kBlock - 1) / kBlock;
        hipLaunchKernelGGL(ll128_pack_kernel, dim3(uint32_t(grid), uint32_t(count)), dim3(kBlock), 0, s, p,
                           nlines);
    }
    return hipGetLastError();
}

hipError_t launch_ll_reduce(const void* const* wire, int n, void* out, size_t numel, int dtype,
                            int proto, uint32_t step, uint32_t* flags, uint64_t timeout_ticks,
                            hipStream_t s) {
    ReduceParams p{};
    for (int i = 0; i < n; ++i) p.wire[i] = static_cast<const uint8_t*>(wire[i]);
    p.out = static_cast<uint8_t*>(out);
    p.flags = flags;
    p.timeout_ticks = timeout_ticks;
    p.nbytes = numel * (dtype == 0 ? 4 : 2);
    p.nlines = proto == 0 ? (p.nbytes + 3) / 4 : (p.nbytes + 119) / 120;
    p.step = step;
    return dispatch_ranks(n, [&](auto nr) {
        constexpr int NR = decltype(nr)::value;
        return dtype == 0 ? launch_reduce_t<float, NR>(p, proto, s) : launch_reduce_t<bf16_t, NR>(p, proto, s);
    });
}

}  // namespace ar

namespace ar {

hipError_t launch_ll_allreduce(const void* src, const void* const* wire, int n, int me, void* out, size_t numel,
                               int dtype, int proto, uint32_t step, uint32_t* flags, uint64_t timeout_ticks,
                               hipStream_t s) {
    ReduceParams p{};
    for (int i = 0; i < n; ++i) p.wire[i] = static_cast<const uint8_t*>(wire[i]);
    p.out = static_cast<uint8_t*>(out);
    p.flags = flags;
    p.timeout_ticks = timeout_ticks;
    p.nbytes = numel * (dtype == 0 ? 4 : 2);
    p.nlines = proto == 0 ? (p.nbytes + 3) / 4 : (p.nbytes + 119) / 120;
    p.step = step;
    p.me = me;
    p.src = static_cast<const uint8_t*>(src);
    p.own_wire = const_cast<uint8_t*>(static_cast<const uint8_t*>(wire[me]));
    // rank me's wire is written, not read: its slot loads a peer's line,
    // which the fold does not use (the LL kernel skips the slot).  That line
    // is ready when the peers' are, so one readiness test covers every slot;
    // loading rank me's own, still stale, line there instead sent every unit
    // down the re-read path (1.5 to 5 times slower when measured).
    p.wire[me] = static_cast<const uint8_t*>(wire[(me + 1) % n]);
    return dispatch_ranks(n, [&](auto nr) {
        constexpr int NR = decltype(nr)::value;
        return dtype == 0 ? launch_fused_t<float, NR>(p, proto, s) : launch_fused_t<bf16_t, NR>(p, proto, s);
    });
}

}  // namespace ar
