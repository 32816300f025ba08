// All-reduce fused with a residual add and RMSNorm, for gfx950: a one-shot
// form (every rank's launch reduces and norms every row) and a two-shot
// form (each rank reduces and norms its own rows, then gathers its peers').
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
// One-shot form.  A workgroup owns a row (above 2^20 rows the workgroups stride over
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
// Rows whose n + 1 input streams hold at least this many bytes are split
// into parts (one compute unit pulling such a row is the bottleneck; below
// it the parts' exchange costs more than it saves); see the launch rules.
constexpr uint32_t kCoopMinRowBytes = 128u << 10;

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

// Where one row's results go: residual_out and out (nontemporal stores),
// and, in the two-shot's reduce-scatter, the row's copies in the rank's
// segment (device-coherent stores: the peers' all-gathers read them).  A
// null pointer is not written.  Each is the row's first vector.
struct RowDst {
    u32x4* res_out;
    u32x4* out;
    u32x4* seg_res;
    u32x4* seg_out;
};

__device__ __forceinline__ void row_store_coherent(u32x4* row, uint32_t row_bytes, uint32_t off, u32x4 v) {
    st_coherent(buffer_range(row, row_bytes), off, v);
}

// One row: base = the row's first vector in the ranks' inputs, residual =
// the row's first vector of the residual.
template <typename T, int NR, int VPT, int RBMAX = (VPT == 1 ? kMaxRanks : 8)>
__device__ __forceinline__ void rmsnorm_row(const RmsParams& p, size_t base, const u32x4* residual, RowDst d,
                                            float (&part)[kMaxWaves], float& factor) {
    constexpr int E = Vec<T>::E;
    constexpr int RB = NR <= RBMAX ? NR : RBMAX;  // loads in flight per vector
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & (kWave - 1);
    const uint32_t wave = tid / kWave;
    const uint32_t nwaves = blockDim.x / kWave;
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
        const u32x4 rv = row_load<kCachePolicyNt>(buffer_range(residual, row_bytes), off);
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
            const u32x4 hv = Vec<T>::narrow(h[j]);
            if (d.res_out) row_store(buffer_range(d.res_out, row_bytes), off, hv);
            if (d.seg_res) row_store_coherent(d.seg_res, row_bytes, off, hv);
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
            const u32x4 yv = Vec<T>::narrow(y);
            if (d.out) row_store(buffer_range(d.out, row_bytes), v * 16u, yv);
            if (d.seg_out) row_store_coherent(d.seg_out, row_bytes, v * 16u, yv);
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
            const size_t base = row * p.vecs;
            rmsnorm_row<T, NR, VPT>(p, base, p.residual + base,
                                    RowDst{p.residual_out + base, p.out + base, nullptr, nullptr}, part, factor);
            __syncthreads();  // part and factor are rewritten by the next row
        }
    } else {
        const size_t base = size_t(blockIdx.x) * p.vecs;
        rmsnorm_row<T, NR, VPT>(p, base, p.residual + base,
                                RowDst{p.residual_out + base, p.out + base, nullptr, nullptr}, part, factor);
    }
}

// ---------------------------------------------------------------------------
// The two-shot form.  The reduce-scatter owns whole rows: rank r's group is
// rows [r G, (r + 1) G), G = rows / n, so a rank finishes the norm of its
// rows alone (a workgroup per row, the same per-row code as above, so the
// same bits).  It writes its own outputs' rows and copies both results of
// its rows into its segment (out rows, then residual_out rows) with
// device-coherent stores; each tile of rows is published with an arrival
// slot in the flag region once every store of the tile is complete.  The
// all-gather of one rank's share polls a peer tile's slot and copies that
// tile's out and residual_out rows into its outputs.  One rank's share is
// one launch (no workgroup waits on another of the same launch); every
// rank's reduce-scatter alone is another (for the peers, or for all ranks
// before their shares).
struct TsRmsParams {
    RmsParams p;  // inputs, weight, row size, eps (residual and outputs unused)
    const u32x4* residual[kMaxRanks];
    u32x4* seg[kMaxRanks];
    u32x4* res_out[kMaxRanks];
    u32x4* out[kMaxRanks];
    uint32_t* flags;
    uint64_t timeout_ticks;
    uint32_t step;    // 0: auto, each wavefront's epoch (in a segment) + 1
    int r0, r1;
    uint32_t group;   // rows per rank
    uint32_t tile;    // rows per arrival slot
    uint32_t ntiles;  // slots per rank
    uint32_t parts;   // 64-vector parts per row
    int do_ag;
    size_t ep_off;    // byte offset of a segment's epoch words (auto ids)
    uint32_t wpb;     // wavefronts per workgroup
};

// Auto step ids.  A segment ends with one epoch word per wavefront of its
// rank's work in either role: first its reduce-scatter items, then the
// items of its all-gather (for the peers' n - 1 groups, in order), a word
// per wavefront of each.  A wavefront takes its word + 1 as the step id
// when it starts and stores that id back when it ends, so every launch
// advances every word it owns by one: the words of a rank's reduce-scatter
// advance once per step whether the rank's share or a reduce-scatter-only
// launch runs them, those of its all-gather with its share, and all agree
// with no wavefront waiting on another.  A call captured once into a graph
// takes a new id on every replay.  The words sit beside the done flags and
// partial sums they must stay above, so zeroing the segments restarts both.
struct AutoId {
    uint32_t* word = nullptr;  // this wavefront's epoch word, null for explicit ids
    uint32_t step = 0;
};
// The word's load goes out before the wavefront's first data load and its
// value is taken only where the step is first needed, so its round trip
// overlaps theirs.
__device__ __forceinline__ uint32_t ts_epoch_load(const TsRmsParams& q, uint32_t r, uint32_t index, AutoId& id) {
    if (q.step != 0) return 0u;
    id.word = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(q.seg[r]) + q.ep_off) + index;
    return flag_load_relaxed(id.word);
}
__device__ __forceinline__ uint32_t ts_take_step(const TsRmsParams& q, uint32_t epoch, AutoId& id) {
    id.step = q.step != 0 ? q.step : __builtin_amdgcn_readfirstlane(epoch) + 1u;
    return id.step;
}
__device__ __forceinline__ void ts_finish(const AutoId& id) {
    if (id.word && id.step != 0 && (threadIdx.x & (kWave - 1)) == 0) flag_store_relaxed(id.word, id.step);
}

// Parts of rows.  A rank's 64 rows of the prefill message would put each
// row's n + 1 streams through one compute unit (the workgroup-per-row form
// above), so here every row is cut into parts of 64 vectors, one wavefront
// each, as in the one-shot form's few-rows path: a part folds its vectors,
// stores residual_out (its own and its segment's copy), publishes its
// partial sum of h^2 with the step id as one 8-byte store in the segment,
// polls its siblings' (bounded), scales its h by the row's factor and stores
// out; once all its stores are complete it sets its done flag (the step id)
// in the segment.  An all-gather item is a part of a peer's row: it polls
// that part's done flag and copies its vectors of both results.  Segment of
// a rank, in bytes: G out rows and G residual_out rows (16 V each), then
// G P partial slots of 8 bytes, then G P done flags of 4 bytes.
__host__ __device__ constexpr size_t ts_partial_off(size_t G, size_t V) { return 32 * G * V; }
__host__ __device__ constexpr size_t ts_done_off(size_t G, size_t V, size_t P) { return 32 * G * V + 8 * G * P; }

template <typename T, int NR>
__device__ __forceinline__ void twoshot_rmsnorm_parts(const TsRmsParams& q, AutoId& id) {
    constexpr int E = Vec<T>::E;
    const RmsParams& p = q.p;
    const uint32_t lane = threadIdx.x;
    const uint32_t b = blockIdx.x;
    const uint32_t R = uint32_t(q.r1 - q.r0);
    const uint32_t G = q.group, P = q.parts, V = p.vecs;
    const uint32_t row_bytes = V * 16u;
    const uint32_t rs_items = R * G * P;
    if (b < rs_items) {
        const uint32_t rr = b / (G * P), rem = b - rr * (G * P);
        const uint32_t k = rem / P, pp = rem - k * P;
        const uint32_t r = uint32_t(q.r0) + rr;
        const uint32_t epoch = ts_epoch_load(q, r, rem, id);  // word k P + pp of rank r's
        const size_t base = (size_t(r) * G + k) * V;
        const uint32_t v = pp * kWave + lane;
        const bool valid = v < V;
        const uint32_t off = (valid ? v : 0u) * 16u;
        const u32x4 wv = row_load<0>(buffer_range(p.weight, row_bytes), off);
        const u32x4 rv = row_load<kCachePolicyNt>(buffer_range(q.residual[r] + base, row_bytes), off);
        u32x4 x[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) x[i] = row_load<kCachePolicyNt>(buffer_range(p.in[i] + base, row_bytes), off);
        Acc<T> acc;
#pragma unroll
        for (int i = 0; i < NR; ++i) acc.add(x[i]);
        const uint32_t step = ts_take_step(q, epoch, id);
        float res[E], h[E];
        Vec<T>::widen(rv, res);
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) h[e] = acc.a[e] + res[e];
        u32x4* seg = q.seg[r];
        if (valid) {
            const u32x4 hv = Vec<T>::narrow(h);
            if (q.do_ag) row_store(buffer_range(q.res_out[r] + base, row_bytes), off, hv);
            row_store_coherent(seg + (size_t(G) + k) * V, row_bytes, off, hv);
#pragma unroll
            for (int e = 0; e < E; ++e) ss += h[e] * h[e];
        }
        ss = wave_sum(ss);
        uint8_t* segb = reinterpret_cast<uint8_t*>(seg);
        const __amdgpu_buffer_rsrc_t slots = buffer_range(segb + ts_partial_off(G, V) + size_t(k) * P * 8u, P * 8u);
        if (lane == 0)
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(ss), step}, slots, int(pp * 8u), 0,
                                                  kCachePolicySc1);
        const bool mine = lane < P;
        const uint32_t soff = (mine ? lane : 0u) * 8u;
        u32x2 sl = __builtin_amdgcn_raw_buffer_load_b64(slots, int(soff), 0, kCachePolicySc1);
        const uint64_t t0 = now_ticks();
        while (true) {
            const uint64_t missing = ~wave_ballot(!mine || sl.y >= step) & wave_exec();
            if (missing == 0) break;
            if (now_ticks() - t0 > q.timeout_ticks) {
                if (lane == 0) report_timeout(q.flags, kPhaseRmsnorm, r, k);
                return;  // no output, no done flag
            }
            __builtin_amdgcn_s_sleep(1);
            if (mine && sl.y < step) sl = __builtin_amdgcn_raw_buffer_load_b64(slots, int(soff), 0, kCachePolicySc1);
        }
        // the same values in the same lanes in every part of the row
        const float total = wave_sum(mine ? __uint_as_float(sl.x) : 0.0f);
        const float f = 1.0f / sqrtf(total / p.hidden + p.eps);
        if (valid) {
            float w[E], y[E];
            Vec<T>::widen(wv, w);
#pragma unroll
            for (int e = 0; e < E; ++e) y[e] = (h[e] * f) * w[e];
            const u32x4 yv = Vec<T>::narrow(y);
            if (q.do_ag) row_store(buffer_range(q.out[r] + base, row_bytes), off, yv);
            row_store_coherent(seg + size_t(k) * V, row_bytes, off, yv);
        }
        // done: every store of this part complete, then its flag
        wait_stores();
        if (lane == 0)
            __builtin_amdgcn_raw_buffer_store_b32(step, buffer_range(segb + ts_done_off(G, V, P), G * P * 4u),
                                                  int((k * P + pp) * 4u), 0, kCachePolicySc1);
        return;
    }
    // all-gather item: (output rank, peer, row, part)
    const uint32_t c = b - rs_items;
    const uint32_t per_out = uint32_t(NR - 1) * G * P;
    const uint32_t oo = c / per_out;
    if (oo >= R) return;
    const uint32_t rem = c - oo * per_out;
    const uint32_t r = uint32_t(q.r0) + oo;
    const uint32_t epoch = ts_epoch_load(q, r, G * P + rem, id);  // after the G P words of its reduce-scatter
    const uint32_t jj = rem / (G * P), rem2 = rem - jj * (G * P);
    const uint32_t j = jj < r ? jj : jj + 1u;  // every rank but r
    const uint32_t k = rem2 / P, pp = rem2 - k * P;
    uint8_t* segb = reinterpret_cast<uint8_t*>(q.seg[j]);
    const __amdgpu_buffer_rsrc_t done = buffer_range(segb + ts_done_off(G, V, P), G * P * 4u);
    const uint32_t doff = (k * P + pp) * 4u;
    uint32_t seen = __builtin_amdgcn_raw_buffer_load_b32(done, int(doff), 0, kCachePolicySc1);
    const uint32_t step = ts_take_step(q, epoch, id);
    const uint64_t t0 = now_ticks();
    while (__builtin_amdgcn_readfirstlane(seen) < step) {
        if (now_ticks() - t0 > q.timeout_ticks) {
            if (lane == 0) report_timeout(q.flags, kPhaseTwoshotAg, j, k);
            return;
        }
        __builtin_amdgcn_s_sleep(1);
        seen = __builtin_amdgcn_raw_buffer_load_b32(done, int(doff), 0, kCachePolicySc1);
    }
    const uint32_t v = pp * kWave + lane;
    if (v < V) {
        const u32x4 yv = ld_coherent(buffer_range(q.seg[j] + size_t(k) * V, row_bytes), v * 16u);
        const u32x4 hv = ld_coherent(buffer_range(q.seg[j] + (size_t(G) + k) * V, row_bytes), v * 16u);
        const size_t dst = (size_t(j) * G + k) * V + v;
        st_stream(q.out[r] + dst, yv);
        st_stream(q.res_out[r] + dst, hv);
    }
}

template <typename T, int NR>
__global__ __launch_bounds__(kWave) void twoshot_rmsnorm_parts_kernel(TsRmsParams q) {
    AutoId id;
    twoshot_rmsnorm_parts<T, NR>(q, id);
    ts_finish(id);
}

template <typename T, int NR, int VPT>
__device__ __forceinline__ void twoshot_rmsnorm_rows(const TsRmsParams& q, float (&part)[kMaxWaves],
                                                     float& factor, AutoId& id) {
    const RmsParams& p = q.p;
    const uint32_t R = uint32_t(q.r1 - q.r0);
    const uint32_t rs_items = R * q.ntiles;
    uint32_t* slots = q.flags + kStatusWords;
    const uint32_t b = blockIdx.x;
    if (b < rs_items) {
        const uint32_t rr = b / q.ntiles, t = b - rr * q.ntiles;
        const uint32_t r = uint32_t(q.r0) + rr;
        const uint32_t epoch = ts_epoch_load(q, r, t * q.wpb + threadIdx.x / kWave, id);
        const uint32_t k1 = min((t + 1u) * q.tile, q.group);
        for (uint32_t k = t * q.tile; k < k1; ++k) {
            const size_t base = (size_t(r) * q.group + k) * p.vecs;
            RowDst d{q.do_ag ? q.res_out[r] + base : nullptr, q.do_ag ? q.out[r] + base : nullptr,
                     q.seg[r] + (size_t(q.group) + k) * p.vecs, q.seg[r] + size_t(k) * p.vecs};
            rmsnorm_row<T, NR, VPT, (NR > 15 ? 4 : 8)>(p, base, q.residual[r] + base, d, part, factor);
            __syncthreads();  // part and factor are rewritten by the next row
        }
        const uint32_t step = ts_take_step(q, epoch, id);
        // publish the tile once every wavefront's stores are complete
        wait_stores();
        __syncthreads();
        if (threadIdx.x == 0) flag_store_relaxed(slots + r * kSlotsPerRank + t, step);
        return;
    }
    // all-gather item: (output rank, peer, tile)
    const uint32_t c = b - rs_items;
    const uint32_t per_out = uint32_t(NR - 1) * q.ntiles;
    const uint32_t oo = c / per_out;
    if (oo >= R) return;
    const uint32_t rem = c - oo * per_out;
    const uint32_t r = uint32_t(q.r0) + oo;
    const uint32_t jj = rem / q.ntiles, t = rem - jj * q.ntiles;
    const uint32_t j = jj < r ? jj : jj + 1u;  // every rank but r
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t epoch = ts_epoch_load(q, r, (q.ntiles + rem) * q.wpb + threadIdx.x / kWave, id);
    // every wavefront polls the tile's slot itself (bounded)
    uint32_t seen = flag_load_relaxed(slots + j * kSlotsPerRank + t);
    const uint32_t step = ts_take_step(q, epoch, id);
    const uint64_t t0 = now_ticks();
    while (__builtin_amdgcn_readfirstlane(seen) < step) {
        if (now_ticks() - t0 > q.timeout_ticks) {
            if (lane == 0) report_timeout(q.flags, kPhaseTwoshotAg, j, t);
            return;
        }
        __builtin_amdgcn_s_sleep(1);
        seen = flag_load_relaxed(slots + j * kSlotsPerRank + t);
    }
    // the tile's rows of both results: out rows k, then residual_out rows
    const uint32_t k0 = t * q.tile, k1 = min(k0 + q.tile, q.group);
    const uint32_t tv = (k1 - k0) * p.vecs;  // vectors per result in this tile
    const __amdgpu_buffer_rsrc_t so = buffer_range(q.seg[j] + size_t(k0) * p.vecs, tv * 16u);
    const __amdgpu_buffer_rsrc_t sr = buffer_range(q.seg[j] + (size_t(q.group) + k0) * p.vecs, tv * 16u);
    u32x4* o = q.out[r] + (size_t(j) * q.group + k0) * p.vecs;
    u32x4* ro = q.res_out[r] + (size_t(j) * q.group + k0) * p.vecs;
    for (uint32_t v = threadIdx.x; v < tv; v += blockDim.x) {
        const u32x4 a = ld_coherent(so, v * 16u);
        const u32x4 e = ld_coherent(sr, v * 16u);
        st_stream(o + v, a);
        st_stream(ro + v, e);
    }
}

// With one vector per lane the kernel is held to 64 VGPRs (8 waves per
// SIMD), so two 1024-lane workgroups share a compute unit; the rows' rank
// loads go out in batches of 8 (4 at 16 ranks) so that this needs no spill.
// At 66 VGPRs one workgroup did: 57 against 52 us for one rank's share of
// 64 MiB (n = 8 bf16), 60 against 52 us at n = 16.
template <typename T, int NR, int VPT>
__global__ __launch_bounds__(kMaxBlock, VPT == 1 ? 8 : 1) void twoshot_rmsnorm_kernel(TsRmsParams q) {
    __shared__ float part[kMaxWaves];
    __shared__ float factor;
    AutoId id;
    twoshot_rmsnorm_rows<T, NR, VPT>(q, part, factor, id);
    ts_finish(id);
}

// Which two-shot form runs, by rank count and size (the same for every
// rank's launch of a step, so a share and its peers' reduce-scatters agree):
// parts where a row's n + 1 streams hold at least kCoopMinRowBytes and a
// rank owns fewer than kTsPartsMaxRows rows.  Measured, one rank's share,
// bf16, rows of 8192: n = 8 at 8 MiB per rank 9.3 against 12.1 us (parts
// against a workgroup per row), at 1 MiB 5.6 against 7.8, 1 row per rank
// 5.1 against 7.2; n = 16 at 8 MiB 9.5 against 14.0; but n = 8 at 64 MiB
// (512 rows per rank) 55.4 against 52.5, and n = 2 at 8 MiB 13.2 against
// 10.3 (light rows).
constexpr uint32_t kTsPartsMaxRows = 256;
inline bool ts_parts(int nr, uint32_t group, uint32_t vecs) {
    return group < kTsPartsMaxRows && uint32_t(nr + 1) * vecs * 16u >= kCoopMinRowBytes;
}
// A workgroup per row: vectors per lane, wavefronts per workgroup (every row
// fits one workgroup of at most 1024 lanes with 1, 2 or 4 vectors each).
inline int ts_vpt(uint32_t vecs) { return vecs <= 1024u ? 1 : (vecs <= 2048u ? 2 : 4); }
inline uint32_t ts_wpb(uint32_t vecs) {
    const uint32_t v = uint32_t(ts_vpt(vecs));
    return ((vecs + v - 1) / v + kWave - 1) / kWave;
}
inline uint32_t ts_tiles(uint32_t group) {
    const uint32_t tile = (group + uint32_t(kSlotsPerRank) - 1) / uint32_t(kSlotsPerRank);
    return (group + tile - 1) / tile;
}

template <typename T, int NR>
hipError_t launch_ts_t(const TsRmsParams& q, hipStream_t s) {
    const uint32_t V = q.p.vecs;
    if (ts_parts(NR, q.group, V)) {
        const uint32_t R = uint32_t(q.r1 - q.r0);
        const uint64_t per = uint64_t(q.group) * q.parts;
        const uint64_t items = uint64_t(R) * per + (q.do_ag ? uint64_t(R) * (NR - 1) * per : 0u);
        hipLaunchKernelGGL((twoshot_rmsnorm_parts_kernel<T, NR>), dim3(uint32_t(items)), dim3(kWave), 0, s, q);
        return hipGetLastError();
    }
    const int vpt = ts_vpt(V);
    const uint32_t block = q.wpb * kWave;
    const uint32_t R = uint32_t(q.r1 - q.r0);
    const uint64_t items = uint64_t(R) * q.ntiles + (q.do_ag ? uint64_t(R) * (NR - 1) * q.ntiles : 0u);
    const dim3 grid = dim3(uint32_t(items)), blk = dim3(block);
    const TsRmsParams& qa = q;
    if (vpt == 1)
        hipLaunchKernelGGL((twoshot_rmsnorm_kernel<T, NR, 1>), grid, blk, 0, s, qa);
    else if (vpt == 2)
        hipLaunchKernelGGL((twoshot_rmsnorm_kernel<T, NR, 2>), grid, blk, 0, s, qa);
    else
        hipLaunchKernelGGL((twoshot_rmsnorm_kernel<T, NR, 4>), grid, blk, 0, s, qa);
    return hipGetLastError();
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
                if (lane == 0) report_timeout(ws, kPhaseRmsnorm, 0u, row);
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

// Segment: the parts' layout above, then the epoch words: n G P for parts
// of rows, n (tiles) (wavefronts per workgroup) for a workgroup per row.
static size_t ts_ep_off(int n, size_t rows, size_t hidden, int dtype) {
    const size_t G = rows / size_t(n), V = hidden * (dtype == 0 ? 4u : 2u) / 16u, P = (V + kWave - 1) / kWave;
    return (ts_done_off(G, V, P) + 4 * G * P + 15) / 16 * 16;
}

size_t twoshot_rmsnorm_segment_bytes(int n, size_t rows, size_t hidden, int dtype) {
    const uint32_t G = uint32_t(rows / size_t(n)), V = uint32_t(hidden * (dtype == 0 ? 4u : 2u) / 16u);
    const size_t words = ts_parts(n, G, V) ? size_t(n) * G * ((V + kWave - 1) / kWave)
                                           : size_t(n) * ts_tiles(G) * ts_wpb(V);
    return (ts_ep_off(n, rows, hidden, dtype) + 4 * words + 15) / 16 * 16;
}

hipError_t launch_twoshot_rmsnorm(const void* const* in, int n, const void* const* residual, const void* weight,
                                  void* const* seg, void* const* residual_out, void* const* out, size_t rows,
                                  size_t hidden, float eps, int dtype, int r0, int r1, uint32_t* flags,
                                  uint32_t step, uint64_t timeout_ticks, hipStream_t s) {
    TsRmsParams q{};
    for (int r = 0; r < n; ++r) {
        q.p.in[r] = static_cast<const u32x4*>(in[r]);
        q.seg[r] = static_cast<u32x4*>(seg[r]);
        if (r >= r0 && r < r1) {
            q.residual[r] = static_cast<const u32x4*>(residual[r]);
            if (out) {
                q.res_out[r] = static_cast<u32x4*>(residual_out[r]);
                q.out[r] = static_cast<u32x4*>(out[r]);
            }
        }
    }
    q.p.weight = static_cast<const u32x4*>(weight);
    q.p.rows = rows;
    q.p.vecs = uint32_t(hidden * (dtype == 0 ? 4u : 2u) / 16u);
    q.p.hidden = float(hidden);
    q.p.eps = eps;
    q.flags = flags;
    q.timeout_ticks = timeout_ticks;
    q.step = step;
    q.r0 = r0;
    q.r1 = r1;
    q.group = uint32_t(rows / size_t(n));
    q.tile = (q.group + uint32_t(kSlotsPerRank) - 1) / uint32_t(kSlotsPerRank);
    q.ntiles = ts_tiles(q.group);
    q.parts = (q.p.vecs + kWave - 1) / kWave;
    q.do_ag = out != nullptr;
    q.ep_off = ts_ep_off(n, rows, hidden, dtype);
    q.wpb = ts_wpb(q.p.vecs);
    return dispatch_ranks(n, [&](auto nr) {
        constexpr int NR = decltype(nr)::value;
        return dtype == 0 ? launch_ts_t<float, NR>(q, s) : launch_ts_t<bf16_t, NR>(q, s);
    });
}

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
