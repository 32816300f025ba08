/*
 * The C ABI from plain C: device buffers from the HIP runtime, calls through
 * include/ar.h only, results compared bit for bit with the C oracle.
 *
 * Test infrastructure: it links the oracle (liboracle.so) to check the
 * library (libar.so).  Exit status 0 when every case matches.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ar.h"

/* the oracle's entry points (oracle/ar_oracle.c) */
void oracle_oneshot(const void* const* in, int n, void* out, size_t numel, int dtype);
size_t oracle_ll_wire_bytes(int proto, size_t nbytes);
void oracle_oneshot_rmsnorm(const void* const* in, int n, const void* residual, const void* weight,
                            void* residual_out, double* y, size_t rows, size_t hidden, double eps, int dtype);

#define CHECK_HIP(x)                                                              \
    do {                                                                          \
        hipError_t e_ = (x);                                                      \
        if (e_ != hipSuccess) {                                                   \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
            exit(2);                                                              \
        }                                                                         \
    } while (0)

static uint64_t lcg = 0x9E3779B97F4A7C15ull;
static uint32_t next32(void) {
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(lcg >> 32);
}

/* float32 in [-4, 4) with a random 23-bit mantissa; bf16 = its top half */
static void fill(void* dst, size_t numel, int dtype) {
    for (size_t i = 0; i < numel; ++i) {
        uint32_t u = 0x3F800000u | (next32() >> 9);  /* [1, 2) */
        float f;
        memcpy(&f, &u, 4);
        f = (f - 1.5f) * 8.0f;
        if (dtype == AR_F32) ((float*)dst)[i] = f;
        else { memcpy(&u, &f, 4); ((uint16_t*)dst)[i] = (uint16_t)(u >> 16); }
    }
}

typedef struct {
    int n;
    size_t numel, bytes;
    int dtype;
    void* host[AR_MAX_RANKS];
    void* dev[AR_MAX_RANKS];
    void* want;
} Case;

static void setup(Case* c, int n, size_t numel, int dtype) {
    c->n = n;
    c->numel = numel;
    c->dtype = dtype;
    c->bytes = numel * (dtype == AR_F32 ? 4 : 2);
    for (int i = 0; i < n; ++i) {
        c->host[i] = malloc(c->bytes);
        fill(c->host[i], numel, dtype);
        CHECK_HIP(hipMalloc(&c->dev[i], c->bytes));
        CHECK_HIP(hipMemcpy(c->dev[i], c->host[i], c->bytes, hipMemcpyHostToDevice));
    }
    c->want = malloc(c->bytes);
    oracle_oneshot((const void* const*)c->host, n, c->want, numel, dtype);
}

static int same(const Case* c, const void* dev_out, const char* what) {
    void* got = malloc(c->bytes);
    CHECK_HIP(hipMemcpy(got, dev_out, c->bytes, hipMemcpyDeviceToHost));
    const int ok = memcmp(got, c->want, c->bytes) == 0;
    printf("%-40s n=%2d numel=%8zu %s: %s\n", what, c->n, c->numel, c->dtype == AR_F32 ? "f32 " : "bf16",
           ok ? "match" : "MISMATCH");
    free(got);
    return ok;
}

static void teardown(Case* c) {
    for (int i = 0; i < c->n; ++i) {
        free(c->host[i]);
        CHECK_HIP(hipFree(c->dev[i]));
    }
    free(c->want);
}

int main(void) {
    int ok = 1;
    void* out;
    uint32_t* flags;
    Case c;

    /* one-shot and reduce-broadcast, ragged size */
    setup(&c, 8, 8 * 8192 + 3, AR_BF16);
    CHECK_HIP(hipMalloc(&out, c.bytes));
    ok &= ar_oneshot((const void* const*)c.dev, c.n, out, c.numel, c.dtype, NULL) == AR_OK;
    CHECK_HIP(hipDeviceSynchronize());
    ok &= same(&c, out, "ar_oneshot");
    void* outs[AR_MAX_RANKS];
    for (int i = 0; i < c.n; ++i) CHECK_HIP(hipMalloc(&outs[i], c.bytes));
    ok &= ar_reduce_bcast((const void* const*)c.dev, c.n, outs, c.numel, c.dtype, 0, c.n, NULL) == AR_OK;
    CHECK_HIP(hipDeviceSynchronize());
    for (int i = 0; i < c.n; ++i) ok &= same(&c, outs[i], "ar_reduce_bcast");
    /* a written buffer overlapping an input is refused before anything runs */
    ok &= ar_oneshot((const void* const*)c.dev, c.n, c.dev[3], c.numel, c.dtype, NULL) == AR_ERR_ALIAS;
    for (int i = 0; i < c.n; ++i) CHECK_HIP(hipFree(outs[i]));
    CHECK_HIP(hipFree(out));
    teardown(&c);

    /* fused two-shot, every rank, explicit then device-kept step ids */
    setup(&c, 8, 8 * 8192, AR_BF16);
    void* segs[AR_MAX_RANKS];
    for (int i = 0; i < c.n; ++i) {
        CHECK_HIP(hipMalloc(&segs[i], c.bytes / c.n));
        CHECK_HIP(hipMalloc(&outs[i], c.bytes));
    }
    CHECK_HIP(hipMalloc((void**)&flags, ar_flag_bytes(c.n)));
    ok &= ar_flag_barrier_reset(flags, c.n, NULL) == AR_OK;
    ok &= ar_twoshot_rs((const void* const*)c.dev, c.n, segs, c.numel, c.dtype, 0, c.n, flags, 1, outs, NULL) == AR_OK;
    CHECK_HIP(hipDeviceSynchronize());
    for (int i = 0; i < c.n; ++i) ok &= same(&c, outs[i], "ar_twoshot_rs (fused, step 1)");
    ok &= ar_flag_barrier_reset(flags, c.n, NULL) == AR_OK;
    for (int rep = 0; rep < 3; ++rep)
        ok &= ar_twoshot_rs((const void* const*)c.dev, c.n, segs, c.numel, c.dtype, 0, c.n, flags, 0, outs, NULL) ==
              AR_OK;
    CHECK_HIP(hipDeviceSynchronize());
    uint32_t status = 1;
    CHECK_HIP(hipMemcpy(&status, flags, 4, hipMemcpyDeviceToHost));
    ok &= status == 0;
    for (int i = 0; i < c.n; ++i) ok &= same(&c, outs[i], "ar_twoshot_rs (fused, auto step x3)");
    for (int i = 0; i < c.n; ++i) {
        CHECK_HIP(hipFree(segs[i]));
        CHECK_HIP(hipFree(outs[i]));
    }
    teardown(&c);

    /* LL and LL128, fp32, ragged */
    setup(&c, 4, 16384 + 1, AR_F32);
    CHECK_HIP(hipMalloc(&out, c.bytes));
    for (int proto = AR_PROTO_LL; proto <= AR_PROTO_LL128; ++proto) {
        const size_t W = ar_ll_wire_bytes(proto, c.bytes);
        ok &= W == oracle_ll_wire_bytes(proto, c.bytes);
        void* wires[AR_MAX_RANKS];
        for (int i = 0; i < c.n; ++i) CHECK_HIP(hipMalloc(&wires[i], W));
        ok &= ar_ll_pack((const void* const*)c.dev, wires, c.n, c.numel, c.dtype, proto, 7, NULL) == AR_OK;
        const int st = proto == AR_PROTO_LL
                           ? ar_ll_reduce_unpack((const void* const*)wires, c.n, out, c.numel, c.dtype, 7, flags, NULL)
                           : ar_ll128_reduce_unpack((const void* const*)wires, c.n, out, c.numel, c.dtype, 7, flags,
                                                    NULL);
        ok &= st == AR_OK;
        CHECK_HIP(hipDeviceSynchronize());
        ok &= same(&c, out, proto == AR_PROTO_LL ? "ar_ll_pack + ar_ll_reduce_unpack"
                                                 : "ar_ll_pack + ar_ll128_reduce_unpack");
        /* rank 2's step in one launch: the others' wires as packed above, at step 7 */
        CHECK_HIP(hipMemset(out, 0, c.bytes));
        ok &= ar_ll_allreduce(c.dev[2], wires, c.n, 2, out, c.numel, c.dtype, proto, 7, flags, NULL) == AR_OK;
        CHECK_HIP(hipDeviceSynchronize());
        ok &= same(&c, out, proto == AR_PROTO_LL ? "ar_ll_allreduce (LL)" : "ar_ll_allreduce (LL128)");
        for (int i = 0; i < c.n; ++i) CHECK_HIP(hipFree(wires[i]));
    }
    CHECK_HIP(hipMemcpy(&status, flags, 4, hipMemcpyDeviceToHost));
    ok &= status == 0;
    CHECK_HIP(hipFree(out));
    CHECK_HIP(hipFree(flags));
    teardown(&c);

    /* the fused all-reduce + residual add + RMSNorm, fp32, with a workspace: residual_out bit
     * for bit, out within 4e-6 of the oracle's fp64 value (the bound derived for the device's
     * fp32 sum of squares) */
    {
        const size_t rows = 8, hidden = 4096;
        setup(&c, 8, rows * hidden, AR_F32);
        float* res = malloc(c.bytes);
        float* w = malloc(hidden * 4);
        float* ro_want = malloc(c.bytes);
        float* got = malloc(c.bytes);
        double* y = malloc(c.numel * sizeof(double));
        fill(res, c.numel, AR_F32);
        fill(w, hidden, AR_F32);
        oracle_oneshot_rmsnorm((const void* const*)c.host, c.n, res, w, ro_want, y, rows, hidden, 1e-6, AR_F32);
        void *d_res, *d_w, *d_ro, *d_out, *d_ws;
        CHECK_HIP(hipMalloc(&d_res, c.bytes));
        CHECK_HIP(hipMalloc(&d_w, hidden * 4));
        CHECK_HIP(hipMalloc(&d_ro, c.bytes));
        CHECK_HIP(hipMalloc(&d_out, c.bytes));
        CHECK_HIP(hipMalloc(&d_ws, ar_rmsnorm_workspace_bytes()));
        CHECK_HIP(hipMemset(d_ws, 0, ar_rmsnorm_workspace_bytes()));
        CHECK_HIP(hipMemcpy(d_res, res, c.bytes, hipMemcpyHostToDevice));
        CHECK_HIP(hipMemcpy(d_w, w, hidden * 4, hipMemcpyHostToDevice));
        ok &= ar_oneshot_rmsnorm((const void* const*)c.dev, c.n, d_res, d_w, d_ro, d_out, rows, hidden, 1e-6f,
                                 AR_F32, (uint32_t*)d_ws, NULL) == AR_OK;
        CHECK_HIP(hipDeviceSynchronize());
        CHECK_HIP(hipMemcpy(got, d_ro, c.bytes, hipMemcpyDeviceToHost));
        int good = memcmp(got, ro_want, c.bytes) == 0;
        CHECK_HIP(hipMemcpy(got, d_out, c.bytes, hipMemcpyDeviceToHost));
        for (size_t i = 0; i < c.numel; ++i) good &= fabs((double)got[i] - y[i]) <= 4e-6 * fabs(y[i]);
        CHECK_HIP(hipMemcpy(&status, d_ws, 4, hipMemcpyDeviceToHost));
        good &= status == 0;
        printf("%-40s n=%2d numel=%8zu f32 : %s\n", "ar_oneshot_rmsnorm", c.n, c.numel, good ? "ok" : "MISMATCH");
        ok &= good;

        /* its two-shot form with auto step ids (step 0): the peers' reduce-scatters, then rank
         * 0's share into the same outputs, cleared first; the same bounds */
        const size_t sb = ar_rmsnorm_segment_bytes(c.n, rows, hidden, AR_F32);
        void* segs[AR_MAX_RANKS];
        const void* resids[AR_MAX_RANKS];
        void* ros[AR_MAX_RANKS] = {0};
        void* outs[AR_MAX_RANKS] = {0};
        for (int r = 0; r < c.n; ++r) {
            CHECK_HIP(hipMalloc(&segs[r], sb));
            CHECK_HIP(hipMemset(segs[r], 0, sb));
            resids[r] = d_res;
        }
        void* fl;
        CHECK_HIP(hipMalloc(&fl, ar_flag_bytes(c.n)));
        CHECK_HIP(hipMemset(fl, 0, ar_flag_bytes(c.n)));
        CHECK_HIP(hipMemset(d_ro, 0xff, c.bytes));
        CHECK_HIP(hipMemset(d_out, 0xff, c.bytes));
        ros[0] = d_ro;
        outs[0] = d_out;
        ok &= ar_twoshot_rmsnorm((const void* const*)c.dev, c.n, resids, d_w, segs, NULL, NULL, rows, hidden, 1e-6f,
                                 AR_F32, 1, c.n, (uint32_t*)fl, 0, NULL) == AR_OK;
        ok &= ar_twoshot_rmsnorm((const void* const*)c.dev, c.n, resids, d_w, segs, ros, outs, rows, hidden, 1e-6f,
                                 AR_F32, 0, 1, (uint32_t*)fl, 0, NULL) == AR_OK;
        CHECK_HIP(hipDeviceSynchronize());
        CHECK_HIP(hipMemcpy(got, d_ro, c.bytes, hipMemcpyDeviceToHost));
        good = memcmp(got, ro_want, c.bytes) == 0;
        CHECK_HIP(hipMemcpy(got, d_out, c.bytes, hipMemcpyDeviceToHost));
        for (size_t i = 0; i < c.numel; ++i) good &= fabs((double)got[i] - y[i]) <= 4e-6 * fabs(y[i]);
        CHECK_HIP(hipMemcpy(&status, fl, 4, hipMemcpyDeviceToHost));
        good &= status == 0;
        printf("%-40s n=%2d numel=%8zu f32 : %s\n", "ar_twoshot_rmsnorm (auto step ids)", c.n, c.numel,
               good ? "ok" : "MISMATCH");
        ok &= good;
        for (int r = 0; r < c.n; ++r) CHECK_HIP(hipFree(segs[r]));
        CHECK_HIP(hipFree(fl));
        CHECK_HIP(hipFree(d_res));
        CHECK_HIP(hipFree(d_w));
        CHECK_HIP(hipFree(d_ro));
        CHECK_HIP(hipFree(d_out));
        CHECK_HIP(hipFree(d_ws));
        free(res);
        free(w);
        free(ro_want);
        free(got);
        free(y);
        teardown(&c);
    }

    printf(ok ? "c abi ok\n" : "c abi FAILED\n");
    return ok ? 0 : 1;
}
