// LL and LL128 flag-packed protocols for gfx950 ("集合通信：NCCL 的算法、协议与
// 推理框架的定制 all-reduce", 协议 table): the sender packs its message into
// lines that carry their own flag (the step id); the receiver polls the flags,
// takes the data out and reduces the n messages exactly as the one-shot path.
//
// LL line  : 8 bytes  = 4 data bytes, then a 32-bit flag.
// LL128 line: 128 bytes = 120 data bytes, then a 64-bit flag.
// Data bytes past the message in the last line are zero.
//
// LL receiver: a lane owns 32 wire bytes of every rank (4 lines, two 16-byte
// loads per rank) and produces 16 output bytes with one 16-byte store.
// LL128 receiver: a wavefront owns 1 KiB of wire per rank = 8 lines; lane l
// holds 16 bytes at part l % 8 of line l / 8, and the lane at part 7 holds 8
// data bytes plus the flag.  Readiness of the whole wavefront is one ballot.
// If a line is behind, the slow path re-reads with agent-coherent 64-bit
// atomic loads until every flag is >= step or the wall-clock budget runs out.
#include "ar_device.hpp"
#include "ar_launch.hpp"

namespace ar {
namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;

// ------------------------------------------------------------------ pack --
struct PackParams {
    const uint8_t* src[kMaxRanks];
    uint8_t* wire[kMaxRanks];
    size_t nbytes;
    uint32_t step;
};

// LL pack: lane c takes message bytes [16c, 16c+16) and writes 2 x 16 wire
// bytes = 4 lines.  blockIdx.y selects the message.  The lane whose 16 bytes
// run past the end reads byte by byte and zero-fills.
__global__ __launch_bounds__(kBlock) void ll_pack_kernel(PackParams p) {
    const uint8_t* src = p.src[blockIdx.y];
    u32x4* wire = reinterpret_cast<u32x4*>(p.wire[blockIdx.y]);
    const size_t c = size_t(blockIdx.x) * kBlock + threadIdx.x;
    const size_t full = p.nbytes / 16;
    const size_t words = (p.nbytes + 3) / 4;  // = lines
    if (c < full) {
        const u32x4 v = ld_stream(reinterpret_cast<const u32x4*>(src) + c);
        st_stream(wire + 2 * c, u32x4{v.x, p.step, v.y, p.step});
        st_stream(wire + 2 * c + 1, u32x4{v.z, p.step, v.w, p.step});
    } else if (c * 4 < words) {
        // last, partial chunk: lines 4c .. words-1, one 8-byte line at a time
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        for (size_t b = 16 * c; b < p.nbytes; ++b) w[(b >> 2) & 3] |= uint32_t(src[b]) << (8 * (b & 3));
        u32x2* lines = reinterpret_cast<u32x2*>(p.wire[blockIdx.y]);
        for (size_t l = 4 * c; l < words; ++l) lines[l] = u32x2{w[l - 4 * c], p.step};
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
    if (part == 7) { w[2] = p.step; w[3] = 0u; }  // 64-bit flag = step, little endian
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
};

// Wait (bounded) until every LL line of this lane's chunk is ready in every
// rank; reloads with agent-coherent atomic 64-bit loads.  Returns false on
// timeout (after reporting it).
template <int NR>
__device__ bool ll_slow_wait(const ReduceParams& p, size_t line0, uint32_t nl, uint64_t (&ln)[NR][4],
                             int lane) {
    const uint64_t t0 = now_ticks();
    while (true) {
        bool ok = true;
        int bad_r = 0;
        uint32_t bad_l = 0;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const uint64_t* w = reinterpret_cast<const uint64_t*>(p.wire[r]) + line0;
#pragma unroll
            for (uint32_t l = 0; l < 4; ++l) {
                if (l < nl && uint32_t(ln[r][l] >> 32) < p.step) {
                    ln[r][l] = line_load_relaxed(w + l);
                    if (uint32_t(ln[r][l] >> 32) < p.step && ok) { ok = false; bad_r = r; bad_l = l; }
                }
            }
        }
        const uint64_t missing = ~wave_ballot(ok) & wave_exec();
        if (missing == 0) return true;
        if (now_ticks() - t0 > p.timeout_ticks) {
            const int bl = __ffsll((unsigned long long)missing) - 1;
            const int rr = __shfl(bad_r, bl);
            const uint32_t ll = uint32_t(__shfl(uint32_t(line0 + bad_l), bl));
            if (lane == bl) report_timeout(p.flags, 2u, uint32_t(rr), ll);
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

template <typename T, int NR>
__global__ __launch_bounds__(kBlock) void ll_reduce_kernel(ReduceParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const size_t c = size_t(blockIdx.x) * kBlock + threadIdx.x;  // 16-byte output chunk
    const size_t line0 = 4 * c;
    const bool active = line0 < p.nlines;
    const uint32_t nl = active ? uint32_t(min(size_t(4), p.nlines - line0)) : 0u;
    uint64_t ln[NR][4];
    if (nl == 4) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const u32x4* w = reinterpret_cast<const u32x4*>(p.wire[r]) + 2 * c;
            const u32x4 a = ld_stream(w), b = ld_stream(w + 1);
            ln[r][0] = uint64_t(a.x) | (uint64_t(a.y) << 32);
            ln[r][1] = uint64_t(a.z) | (uint64_t(a.w) << 32);
            ln[r][2] = uint64_t(b.x) | (uint64_t(b.y) << 32);
            ln[r][3] = uint64_t(b.z) | (uint64_t(b.w) << 32);
        }
    } else {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const uint64_t* w = reinterpret_cast<const uint64_t*>(p.wire[r]) + line0;
#pragma unroll
            for (int l = 0; l < 4; ++l) ln[r][l] = uint64_t(l < int(nl) ? w[l] : ~0ull);
        }
    }
    bool ok = true;
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int l = 0; l < 4; ++l) ok = ok && (l >= int(nl) || uint32_t(ln[r][l] >> 32) >= p.step);
    if (wave_ballot(!ok) != 0) {
        if (!ll_slow_wait<NR>(p, line0, nl, ln, lane)) return;
    }
    if (!active) return;
    Acc<T> acc;
#pragma unroll
    for (int r = 0; r < NR; ++r)
        acc.add(u32x4{uint32_t(ln[r][0]), uint32_t(ln[r][1]), uint32_t(ln[r][2]), uint32_t(ln[r][3])});
    const u32x4 res = acc.result();
    const size_t off = 16 * c;
    if (off + 16 <= p.nbytes) {
        st_stream(reinterpret_cast<u32x4*>(p.out) + c, res);
    } else {
        // partial chunk at the end: write only the message's bytes
        const uint32_t rw[4] = {res.x, res.y, res.z, res.w};
        for (size_t b = off; b < p.nbytes; b += elem<T>::bytes) {
            const uint32_t word = rw[(b - off) >> 2];
            if (elem<T>::bytes == 4) *reinterpret_cast<uint32_t*>(p.out + b) = word;
            else *reinterpret_cast<uint16_t*>(p.out + b) = uint16_t(word >> (8 * (b & 2)));
        }
    }
}

template <typename T, int NR, int U>
__global__ __launch_bounds__(kBlock) void ll128_reduce_kernel(ReduceParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t part = uint32_t(lane) & 7u;
    const size_t wave = size_t(blockIdx.x) * kWavesPerBlock + threadIdx.x / kWave;
    u32x4 x[U][NR];
    size_t line[U];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        line[u] = (wave * U + u) * 8 + size_t(lane) / 8;
        valid[u] = line[u] < p.nlines;
        if (valid[u]) {
#pragma unroll
            for (int r = 0; r < NR; ++r)
                x[u][r] = ld_stream(reinterpret_cast<const u32x4*>(p.wire[r]) + line[u] * 8 + part);
        }
    }
    bool ok = true;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < NR; ++r)
            ok = ok && (!valid[u] || part != 7u || x[u][r].z >= p.step || x[u][r].w != 0u);
    if (wave_ballot(!ok) != 0) {
        // Slow path: poll the flags with coherent 64-bit loads, then re-read
        // the data of every line after an acquire fence.
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
                        if (f < uint64_t(p.step) && ready) { ready = false; bad_r = r; bad_line = line[u]; }
                    }
                }
            }
            const uint64_t missing = ~wave_ballot(ready) & wave_exec();
            if (missing == 0) break;
            if (now_ticks() - t0 > p.timeout_ticks) {
                const int bl = __ffsll((unsigned long long)missing) - 1;
                const int rr = __shfl(bad_r, bl);
                const uint32_t ll = uint32_t(__shfl(uint32_t(bad_line), bl));
                if (lane == bl) report_timeout(p.flags, 3u, uint32_t(rr), ll);
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
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (!valid[u]) continue;
        Acc<T> acc;
        if (part != 7u) {
#pragma unroll
            for (int r = 0; r < NR; ++r) acc.add(x[u][r]);
        } else {
#pragma unroll
            for (int r = 0; r < NR; ++r) acc.add_half(x[u][r]);
        }
        const u32x4 res = acc.result();
        const size_t off = line[u] * 120 + size_t(part) * 16;
        const uint32_t nb = part == 7u ? 8u : 16u;
        if (off + nb <= p.nbytes) {
            u32x2* d = reinterpret_cast<u32x2*>(p.out + off);  // 8-byte aligned
            d[0] = u32x2{res.x, res.y};
            if (nb == 16u) d[1] = u32x2{res.z, res.w};
        } else if (off < p.nbytes) {
            const uint32_t rw[4] = {res.x, res.y, res.z, res.w};
            for (size_t b = off; b < p.nbytes; b += elem<T>::bytes) {
                const uint32_t word = rw[(b - off) >> 2];
                if (elem<T>::bytes == 4) *reinterpret_cast<uint32_t*>(p.out + b) = word;
                else *reinterpret_cast<uint16_t*>(p.out + b) = uint16_t(word >> (8 * (b & 2)));
            }
        }
    }
}

template <typename T, int NR>
hipError_t launch_reduce_t(const ReduceParams& p, int proto, hipStream_t s) {
    if (proto == 0) {
        const size_t chunks = (p.nlines + 3) / 4;
        const size_t grid = (chunks + kBlock - 1) / kBlock;
        hipLaunchKernelGGL((ll_reduce_kernel<T, NR>), dim3(uint32_t(grid)), dim3(kBlock), 0, s, p);
    } else {
        constexpr int U = NR <= 8 ? 2 : 1;
        const size_t wave_units = (p.nlines + 7) / 8;
        const size_t waves = (wave_units + U - 1) / U;
        const size_t grid = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
        hipLaunchKernelGGL((ll128_reduce_kernel<T, NR, U>), dim3(uint32_t(grid)), dim3(kBlock), 0, s, p);
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
        const size_t chunks = (nbytes + 15) / 16;
        const size_t grid = (chunks + kBlock - 1) / kBlock;
        hipLaunchKernelGGL(ll_pack_kernel, dim3(uint32_t(grid), uint32_t(count)), dim3(kBlock), 0, s, p);
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
