// Division by a launch-invariant divisor d for numerators below 2^31, as a
// multiply-high, an add and a shift (Granlund and Montgomery, "Division by
// invariant integers using multiplication", PLDI 1994, the round-up
// multiplier): with s = ceil(log2 d) and m = ceil(2^(32+s) / d) = 2^32 + mlo,
//   n / d = (mulhi(n, mlo) + n) >> s.
// m exceeds 2^(32+s)/d by less than 1, so n*m / 2^(32+s) exceeds n/d by
// less than n / (d * 2^32) < 1/d, which cannot reach the next integer: the
// quotient is exact for every n < 2^32.  n < 2^31 keeps the sum in 32 bits.
// The two-shot's item and unit indices stay far below 2^31.
//
// Plain C++ (no device code), so that a host test can check it.
#pragma once

#include <stdint.h>

namespace ar {

struct FastDiv {
    uint32_t d, mlo, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
    if (d == 0) return FastDiv{0, 0, 0};  // no items: never divided by
    uint32_t s = 0;
    while ((uint64_t(1) << s) < d) ++s;
    const uint64_t two32s = uint64_t(1) << (32 + s);  // s <= 31 here
    const uint64_t m = (two32s + d - 1) / d;            // in [2^32, 2^33)
    return FastDiv{d, uint32_t(m - (uint64_t(1) << 32)), s};
}

// The device's quotient, step for step in 32-bit arithmetic.
inline uint32_t fastdiv_quotient(uint32_t n, const FastDiv& f) {
    const uint32_t hi = uint32_t((uint64_t(n) * f.mlo) >> 32);
    return (hi + n) >> f.s;
}

}  // namespace ar
