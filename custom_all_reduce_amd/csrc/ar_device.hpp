// Device-side helpers shared by the gfx950 kernels: 128-bit vector access,
// fp32 accumulation of packed inputs, round-to-nearest-even to bfloat16, and
// the bounded flag polling used by the two-shot barrier and the LL receivers.
//
// Written for CDNA4 (gfx950) only: 64-lane wavefronts, global_load/store_dwordx4,
// wall clock from s_memrealtime (wall_clock64), agent-scope fences.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ar_launch.hpp"

namespace ar {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

struct bf16_t {};  // tag type: bfloat16 elements stored as raw 16-bit patterns

template <typename T> struct elem;
template <> struct elem<float> { static constexpr int per_vec = 4; static constexpr int bytes = 4; };
template <> struct elem<bf16_t> { static constexpr int per_vec = 8; static constexpr int bytes = 2; };

// ---- memory access -------------------------------------------------------
// Streaming loads/stores: each input byte is read once, so mark them
// non-temporal (global_load_dwordx4 ... nt).
__device__ __forceinline__ u32x4 ld_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_stream(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ u32x4 ld_plain(const u32x4* p) { return *p; }

// Device-coherent 16-byte access for data that one wavefront writes and a
// wavefront on another XCD reads inside the same launch: raw buffer
// load/store with the sc1 cache policy (device scope).  Such stores are
// written through to the device's point of coherence and such loads are
// served from it, so neither side needs the L2-wide writeback (release) or
// invalidate (acquire) that an agent-scope fence costs; the producer only
// waits for its stores to complete (wait_stores) before it publishes a flag,
// and the consumer issues its loads after it has seen the flag.  The buffer
// resource covers one wavefront-uniform range (base and size in scalar
// registers); accesses past its size are dropped / read as zero by the
// hardware, so a resource is also a bounds check.
constexpr int kCachePolicySc1 = 16;  // the sc1 bit of the cache-policy operand
constexpr int kBufferConfigWord = 0x00020000;  // gfx9-family raw-buffer resource word 3

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_range(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), kBufferConfigWord);
}
__device__ __forceinline__ void st_coherent(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, int(byte_off), 0, kCachePolicySc1);
}
__device__ __forceinline__ u32x4 ld_coherent(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, int(byte_off), 0, kCachePolicySc1);
}
// An 8-byte load of the same kind (an LL128 line's flag).
__device__ __forceinline__ u32x2 ld_coherent8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, int(byte_off), 0, kCachePolicySc1);
}
// Wait until every memory operation this wavefront issued has completed
// (s_waitcnt with all counters at zero).
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0); }

// ---- rounding ---------------------------------------------------------------
// float32 -> bfloat16 pattern, round to nearest, ties to even; NaN keeps its
// sign and top payload bits and is made quiet.  gfx950 has this conversion
// in hardware for a pair of values (v_cvt_pk_bf16_f32, reached through a
// vector conversion to __bf16): one instruction per two results in place of
// the seven of an integer rounding sequence.  Checked on the device against
// the integer definition (add 0x7FFF plus the lowest kept bit, keep the high
// half; NaN -> pattern >> 16 | 0x40) for all 2^32 fp32 patterns: identical,
// NaN included, under the default rounding and denormal modes that these
// kernels run with.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) { return pack_bf16x2(f, 0.0f) & 0xFFFFu; }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---- accumulation -----------------------------------------------------------
// Accumulator for one 16-byte vector position: 4 fp32 or 8 bf16 elements,
// widened to fp32.  Starts at +0.0 and adds ranks in the order add() is
// called (callers go rank 0 first).  No fast-math: the adds are not
// reassociated or contracted.
template <typename T> struct Acc;

template <> struct Acc<float> {
    float a[4];
    __device__ __forceinline__ Acc() { a[0] = a[1] = a[2] = a[3] = 0.0f; }
    __device__ __forceinline__ void add(u32x4 v) {
        a[0] = a[0] + __uint_as_float(v.x);
        a[1] = a[1] + __uint_as_float(v.y);
        a[2] = a[2] + __uint_as_float(v.z);
        a[3] = a[3] + __uint_as_float(v.w);
    }
    // add only the low 2 words (8 data bytes)
    __device__ __forceinline__ void add_half(u32x4 v) {
        a[0] = a[0] + __uint_as_float(v.x);
        a[1] = a[1] + __uint_as_float(v.y);
    }
    __device__ __forceinline__ u32x4 result() const {
        return u32x4{__float_as_uint(a[0]), __float_as_uint(a[1]), __float_as_uint(a[2]),
                     __float_as_uint(a[3])};
    }
};

template <> struct Acc<bf16_t> {
    float a[8];
    __device__ __forceinline__ Acc() {
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = 0.0f;
    }
    __device__ __forceinline__ void add(u32x4 v) {
        a[0] = a[0] + bf16_lo(v.x); a[1] = a[1] + bf16_hi(v.x);
        a[2] = a[2] + bf16_lo(v.y); a[3] = a[3] + bf16_hi(v.y);
        a[4] = a[4] + bf16_lo(v.z); a[5] = a[5] + bf16_hi(v.z);
        a[6] = a[6] + bf16_lo(v.w); a[7] = a[7] + bf16_hi(v.w);
    }
    __device__ __forceinline__ void add_half(u32x4 v) {
        a[0] = a[0] + bf16_lo(v.x); a[1] = a[1] + bf16_hi(v.x);
        a[2] = a[2] + bf16_lo(v.y); a[3] = a[3] + bf16_hi(v.y);
    }
    __device__ __forceinline__ u32x4 result() const {
        return u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(a[4], a[5]),
                     pack_bf16x2(a[6], a[7])};
    }
};

// Accumulator for one 8-byte position: 2 fp32 or 4 bf16 elements, given as
// two 32-bit words per rank; same order and rounding as Acc.
template <typename T> struct Acc8;
template <> struct Acc8<float> {
    float a[2] = {0.0f, 0.0f};
    __device__ __forceinline__ void add(uint32_t w0, uint32_t w1) {
        a[0] = a[0] + __uint_as_float(w0);
        a[1] = a[1] + __uint_as_float(w1);
    }
    __device__ __forceinline__ void add(u32x2 v) { add(v.x, v.y); }
    __device__ __forceinline__ u32x2 result() const { return u32x2{__float_as_uint(a[0]), __float_as_uint(a[1])}; }
};
template <> struct Acc8<bf16_t> {
    float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    __device__ __forceinline__ void add(uint32_t w0, uint32_t w1) {
        a[0] = a[0] + bf16_lo(w0); a[1] = a[1] + bf16_hi(w0);
        a[2] = a[2] + bf16_lo(w1); a[3] = a[3] + bf16_hi(w1);
    }
    __device__ __forceinline__ void add(u32x2 v) { add(v.x, v.y); }
    __device__ __forceinline__ u32x2 result() const {
        return u32x2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
    }
};

// Scalar element access for the partial last vector.
__device__ __forceinline__ float load_scalar(const void* base, size_t k, float*) {
    return static_cast<const float*>(base)[k];
}
__device__ __forceinline__ float load_scalar(const void* base, size_t k, bf16_t*) {
    return __uint_as_float(uint32_t(static_cast<const uint16_t*>(base)[k]) << 16);
}
__device__ __forceinline__ void store_scalar(void* base, size_t k, float v, float*) {
    static_cast<float*>(base)[k] = v;
}
__device__ __forceinline__ void store_scalar(void* base, size_t k, float v, bf16_t*) {
    static_cast<uint16_t*>(base)[k] = uint16_t(f32_to_bf16_rne(v));
}

// ---- wave utilities -----------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }
__device__ __forceinline__ uint64_t wave_ballot(bool p) { return __ballot(p); }
__device__ __forceinline__ uint64_t wave_exec() { return __ballot(true); }

// ---- flags ----------------------------------------------------------------------
__device__ __forceinline__ uint32_t flag_load_relaxed(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void flag_store_relaxed(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t line_load_relaxed(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fence_acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

// Record the first asynchronous error of a launch in the flag region's
// status line: word 0 = code | phase << 8 | rank << 16, word 1 = detail.
__device__ __forceinline__ void report_timeout(uint32_t* status, uint32_t phase, uint32_t rank,
                                               uint32_t detail) {
    uint32_t code = kTimeoutCode | (phase << 8) | (rank << 16);
    if (atomicCAS(status, 0u, code) == 0u) flag_store_relaxed(status + 1, detail);
}

__device__ __forceinline__ uint64_t now_ticks() { return wall_clock64(); }

}  // namespace ar
