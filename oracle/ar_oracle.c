/*
 * CPU oracle for the per-GPU reduction kernel of a custom all-reduce.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition that the HIP path is checked against.  Only the tests, the smoke
 * check and the CPU-baseline leg of the benchmark load it; the product
 * library never links, includes or calls anything here, and this file shares
 * no code, header or table with the HIP sources.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC (no FMA
 * contraction, IEEE single-precision adds on x86-64 SSE, subnormals kept).
 *
 * Sources (page titles as printed):
 *  [P1] "0-custom-all-reduce" (obnotes, sglang/jit_kernel): 实现 steps 1-6 --
 *       16-byte vectors, fp32 accumulation of every GPU's data in GPU-index
 *       order starting from a zero accumulator, one round-to-nearest cast.
 *  [P3] "集合通信：NCCL 的算法、协议与推理框架的定制 all-reduce": 算法 section
 *       (one-shot / two-shot), 协议 table (LL, LL128, Simple).
 *  [P4] "多 GPU 与 NCCL": 集合通信 table and identity all-reduce =
 *       reduce-scatter + all-gather; ring all-reduce section.
 *  [P3] also names, in its 推理框架 section, an all-reduce fused with
 *       RMSNorm (the FlashInfer kernel SGLang integrates) without defining
 *       it; O10 below is this repository's reading of that op.
 *
 * Readings where the pages are silent are marked [reading].
 *
 * dtype codes: 0 = float32, 1 = bfloat16 (stored as raw uint16 patterns).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <stdlib.h>

#define OR_F32 0
#define OR_BF16 1

/* ------------------------------------------------------------------ O1 --- */
/* bfloat16 -> float32: a bfloat16 is the upper half of a float32 pattern, so
 * widening is exact: put the 16 bits on top, zeros below.                     */
float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* float32 -> bfloat16, round to nearest, ties to even ([P1] step 4: the
 * result is cast back with round-to-nearest; "ties to even" is the IEEE 754
 * default [reading]).  Keep the top 16 bits; look at the 16 dropped bits:
 * above half -> round up, exactly half -> round up only if the kept part is
 * odd.  A carry out of the mantissa moves into the exponent, which also
 * turns values at or beyond max-finite + half an ulp into infinity.
 * NaN [reading]: stays NaN, sign kept, made quiet (mantissa MSB set) and its
 * payload truncated, as IEEE 754-2008 section 6.2.3 recommends for narrowing. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xFFFFu;
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u)
        return (uint16_t)(kept | 0x0040u);
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        kept += 1u;
    return (uint16_t)kept;
}

void oracle_f32_to_bf16_array(const float* src, uint16_t* dst, size_t count)
{
    for (size_t i = 0; i < count; ++i)
        dst[i] = oracle_f32_to_bf16(src[i]);
}

static float load_elem(const void* p, size_t k, int dtype)
{
    if (dtype == OR_F32)
        return ((const float*)p)[k];
    return oracle_bf16_to_f32(((const uint16_t*)p)[k]);
}

static void store_elem(void* p, size_t k, int dtype, float v)
{
    if (dtype == OR_F32)
        ((float*)p)[k] = v;
    else
        ((uint16_t*)p)[k] = oracle_f32_to_bf16(v);
}

static size_t elem_size(int dtype) { return dtype == OR_F32 ? 4u : 2u; }

/* ------------------------------------------------------------------ O2 --- */
/* One-shot all-reduce ([P1] steps 3-5, [P3] 算法 "one-shot"): every element k
 * of the output is the sum over ranks 0..n-1, taken in rank order, of the
 * ranks' element k widened to fp32, starting from a +0 accumulator, rounded
 * once to the output type.                                                    */
void oracle_oneshot(const void* const* in, int n, void* out, size_t numel, int dtype)
{
    for (size_t k = 0; k < numel; ++k) {
        float acc = 0.0f;
        for (int i = 0; i < n; ++i)
            acc = acc + load_elem(in[i], k, dtype);
        store_elem(out, k, dtype, acc);
    }
}

/* ------------------------------------------------------------------ O3 --- */
/* Two-shot all-reduce ([P3] 算法 "two-shot"; [P4] all-reduce = reduce-scatter
 * + all-gather).  m = numel / n (caller guarantees divisibility, as the two-
 * shot kernel on [P1] requires).
 *   reduce-scatter: rank r sums segment r of every rank -> seg[r] (m elements,
 *                   same per-element fold as O2, rounded once into seg[r]);
 *   all-gather    : every rank r copies seg[0..n-1] in order into out[r].
 * seg[] and out[] each hold n buffers; out may be NULL (reduce-scatter only). */
void oracle_twoshot(const void* const* in, int n, void* const* seg, void* const* out,
                    size_t numel, int dtype)
{
    size_t m = numel / (size_t)n;
    size_t es = elem_size(dtype);
    for (int r = 0; r < n; ++r) {
        for (size_t k = 0; k < m; ++k) {
            float acc = 0.0f;
            for (int i = 0; i < n; ++i)
                acc = acc + load_elem(in[i], (size_t)r * m + k, dtype);
            store_elem(seg[r], k, dtype, acc);
        }
    }
    if (!out)
        return;
    for (int r = 0; r < n; ++r)
        for (int j = 0; j < n; ++j)
            memcpy((char*)out[r] + (size_t)j * m * es, seg[j], m * es);
}

/* ------------------------------------------------------------------ O4 --- */
/* Ring all-reduce, simulated step by step ([P4] ring all-reduce section; [P3]
 * 算法 "ring": n-1 reduce-scatter steps and n-1 all-gather steps, each rank
 * sending 2(n-1)/n of the data).  Rank r starts with a copy of in[r] in
 * buf[r]; the data is cut into n chunks, chunk c = [c*N/n, (c+1)*N/n).
 * Schedule [reading; the pages give none]: in reduce-scatter step s
 * (s = 0..n-2) rank r sends chunk (r - s) mod n to rank (r + 1) mod n, which
 * adds it to its own copy of that chunk; after n-1 steps rank r holds the
 * complete chunk (r + 1) mod n.  In all-gather step s rank r sends chunk
 * (r + 1 - s) mod n to rank r + 1, which overwrites its copy.  Messages of a
 * step are all taken before any is applied (every rank sends at once).  The
 * wire carries the buffer type, so a bfloat16 ring rounds after every hop.
 * bytes_sent[r] counts what rank r put on the wire.                           */
void oracle_ring(const void* const* in, int n, void* const* buf, size_t numel, int dtype,
                 uint64_t* bytes_sent)
{
    size_t es = elem_size(dtype);
    for (int r = 0; r < n; ++r) {
        memcpy(buf[r], in[r], numel * es);
        bytes_sent[r] = 0;
    }
    size_t maxchunk = numel / (size_t)n + 1;
    char* msg = (char*)malloc((size_t)n * maxchunk * es + 1);
    /* reduce-scatter */
    for (int s = 0; s < n - 1; ++s) {
        for (int r = 0; r < n; ++r) {
            int c = ((r - s) % n + n) % n;
            size_t lo = (size_t)c * numel / (size_t)n, hi = (size_t)(c + 1) * numel / (size_t)n;
            memcpy(msg + (size_t)r * maxchunk * es, (char*)buf[r] + lo * es, (hi - lo) * es);
            bytes_sent[r] += (hi - lo) * es;
        }
        for (int r = 0; r < n; ++r) {
            int dst = (r + 1) % n;
            int c = ((r - s) % n + n) % n;
            size_t lo = (size_t)c * numel / (size_t)n, hi = (size_t)(c + 1) * numel / (size_t)n;
            const char* m = msg + (size_t)r * maxchunk * es;
            for (size_t k = lo; k < hi; ++k) {
                float recv = load_elem(m, k - lo, dtype);
                float own = load_elem(buf[dst], k, dtype);
                store_elem(buf[dst], k, dtype, recv + own);
            }
        }
    }
    /* all-gather */
    for (int s = 0; s < n - 1; ++s) {
        for (int r = 0; r < n; ++r) {
            int c = ((r + 1 - s) % n + n) % n;
            size_t lo = (size_t)c * numel / (size_t)n, hi = (size_t)(c + 1) * numel / (size_t)n;
            memcpy(msg + (size_t)r * maxchunk * es, (char*)buf[r] + lo * es, (hi - lo) * es);
            bytes_sent[r] += (hi - lo) * es;
        }
        for (int r = 0; r < n; ++r) {
            int dst = (r + 1) % n;
            int c = ((r + 1 - s) % n + n) % n;
            size_t lo = (size_t)c * numel / (size_t)n, hi = (size_t)(c + 1) * numel / (size_t)n;
            memcpy((char*)buf[dst] + lo * es, msg + (size_t)r * maxchunk * es, (hi - lo) * es);
        }
    }
    free(msg);
}

/* --------------------------------------------------------------- O5/O6 --- */
/* Line formats ([P3] 协议 table):
 *   LL    : 8-byte line = 4 bytes of data + 4 bytes of flag.
 *   LL128 : 128-byte line = 120 bytes of data + 8 bytes of flag.
 * [reading] Data first, flag last, little-endian; the flag is the step id
 * (u32 for LL, u64 for LL128); the message is taken as bytes, line k carries
 * message bytes [k*D, (k+1)*D) with D = 4 or 120, zero past the end.        */
#define OR_LL 0
#define OR_LL128 1

static size_t line_payload(int proto) { return proto == OR_LL ? 4u : 120u; }
static size_t line_bytes(int proto) { return proto == OR_LL ? 8u : 128u; }

size_t oracle_ll_lines(int proto, size_t nbytes)
{
    size_t d = line_payload(proto);
    return (nbytes + d - 1) / d;
}

size_t oracle_ll_wire_bytes(int proto, size_t nbytes)
{
    return oracle_ll_lines(proto, nbytes) * line_bytes(proto);
}

/* Sender: write every line of the message with the step id as flag. */
void oracle_ll_pack(int proto, const void* src, size_t nbytes, void* wire, uint32_t step)
{
    size_t d = line_payload(proto), lb = line_bytes(proto);
    size_t lines = oracle_ll_lines(proto, nbytes);
    for (size_t l = 0; l < lines; ++l) {
        unsigned char* line = (unsigned char*)wire + l * lb;
        memset(line, 0, d);
        size_t lo = l * d;
        size_t take = nbytes - lo < d ? nbytes - lo : d;
        memcpy(line, (const unsigned char*)src + lo, take);
        if (proto == OR_LL) {
            uint32_t f = step;
            memcpy(line + 4, &f, 4);
        } else {
            uint64_t f = step;
            memcpy(line + 120, &f, 8);
        }
    }
}

/* Receiver side of one line: its flag, widened to 64 bits. */
static uint64_t line_flag(int proto, const unsigned char* line)
{
    if (proto == OR_LL) {
        uint32_t f;
        memcpy(&f, line + 4, 4);
        return f;
    }
    uint64_t f;
    memcpy(&f, line + 120, 8);
    return f;
}

/* Unpack: copy each line's data into dst; a line is ready when its flag is at
 * least the expected step [reading: ">=" so a sender that has moved on to a
 * later step never strands a slower receiver].  Returns 1 when every line is
 * ready, else 0 with *bad_line = the first line that is not.                  */
int oracle_ll_unpack(int proto, const void* wire, size_t nbytes, void* dst, uint32_t step,
                     size_t* bad_line)
{
    size_t d = line_payload(proto), lb = line_bytes(proto);
    size_t lines = oracle_ll_lines(proto, nbytes);
    for (size_t l = 0; l < lines; ++l) {
        const unsigned char* line = (const unsigned char*)wire + l * lb;
        if (line_flag(proto, line) < (uint64_t)step) {
            if (bad_line)
                *bad_line = l;
            return 0;
        }
        size_t lo = l * d;
        size_t take = nbytes - lo < d ? nbytes - lo : d;
        memcpy((unsigned char*)dst + lo, line, take);
    }
    return 1;
}

/* ------------------------------------------------------------------ O7 --- */
/* Flag-packed reduce: the receiver waits for every line of every rank, takes
 * the data out, then reduces exactly as O2.  Returns 1 on success; 0 if some
 * line is not ready (the real receiver would time out), with the first such
 * (rank, line) in rank-major order.                                            */
int oracle_ll_reduce(int proto, const void* const* wire, int n, void* out, size_t numel,
                     int dtype, uint32_t step, int* bad_rank, size_t* bad_line)
{
    size_t nbytes = numel * elem_size(dtype);
    void** msgs = (void**)calloc((size_t)n, sizeof(void*));
    int ok = 1;
    for (int i = 0; i < n && ok; ++i) {
        msgs[i] = malloc(nbytes + 1);
        size_t bl = 0;
        if (!oracle_ll_unpack(proto, wire[i], nbytes, msgs[i], step, &bl)) {
            ok = 0;
            if (bad_rank)
                *bad_rank = i;
            if (bad_line)
                *bad_line = bl;
        }
    }
    if (ok)
        oracle_oneshot((const void* const*)msgs, n, out, numel, dtype);
    for (int i = 0; i < n; ++i)
        free(msgs[i]);
    free(msgs);
    return ok;
}

/* ----------------------------------------------------------------- O10 --- */
/* One-shot all-reduce fused with a residual add and RMSNorm.  [P3] names the
 * fused op only; the definition here is a [reading]: RMSNorm as usually
 * defined (each element divided by the root mean square of its row, plus
 * eps inside the root, times a per-column weight), applied to the residual
 * stream after the all-reduced sum has been added to it.
 * The data are rows x hidden, row-major.  For element (i, k):
 *   h      = (O2's fold of the ranks' element, fp32, rank order, from +0)
 *            + residual[i, k]                              (one more fp32 add)
 *   residual_out[i, k] = h rounded once to the data type
 *   ms_i   = (sum over k of h^2) / hidden                  (fp64, k ascending)
 *   y[i, k] = h / sqrt(ms_i + eps) * weight[k]             (fp64, not rounded)
 * h is an fp32 value and is carried into the fp64 steps exactly; y is left
 * unrounded so a test can state its own tolerance for the device's fp32
 * arithmetic.  weight holds hidden elements of the data type.                 */
void oracle_oneshot_rmsnorm(const void* const* in, int n, const void* residual, const void* weight,
                            void* residual_out, double* y, size_t rows, size_t hidden, double eps,
                            int dtype)
{
    double* hrow = (double*)malloc(hidden * sizeof(double));
    for (size_t i = 0; i < rows; ++i) {
        double sumsq = 0.0;
        for (size_t k = 0; k < hidden; ++k) {
            size_t e = i * hidden + k;
            float acc = 0.0f;
            for (int r = 0; r < n; ++r)
                acc = acc + load_elem(in[r], e, dtype);
            float h = acc + load_elem(residual, e, dtype);
            store_elem(residual_out, e, dtype, h);
            hrow[k] = (double)h;
            sumsq += (double)h * (double)h;
        }
        double ms = sumsq / (double)hidden;
        double inv = 1.0 / sqrt(ms + eps);
        for (size_t k = 0; k < hidden; ++k)
            y[i * hidden + k] = hrow[k] * inv * (double)load_elem(weight, k, dtype);
    }
    free(hrow);
}
