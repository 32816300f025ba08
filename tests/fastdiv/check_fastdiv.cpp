// Host check of the two-shot's invariant-divisor quotient (fastdiv.hpp)
// against plain integer division: every divisor up to 2^16 with the
// numerators around each multiple of it, a band of numerators near 2^31,
// every numerator below 2^24 for the divisor shapes the tiling uses, and
// random pairs over the whole range.  Prints one line; exit status 0 iff
// every quotient matches.
#include <cstdint>
#include <cstdio>
#include <random>

#include "fastdiv.hpp"

int main() {
    uint64_t checks = 0, bad = 0;
    auto chk = [&](uint32_t n, const ar::FastDiv& f) {
        ++checks;
        if (ar::fastdiv_quotient(n, f) != n / f.d && bad++ < 8) std::printf("mismatch n=%u d=%u\n", n, f.d);
    };
    for (uint32_t d = 1; d <= (1u << 16); ++d) {
        const ar::FastDiv f = ar::make_fastdiv(d);
        for (uint32_t n = 0; n < 256; ++n) chk(n, f);
        // numerators at and next to multiples of d, spread up to 2^31 - 1
        for (uint32_t k = 1; k <= 64; ++k) {
            const uint64_t q = (uint64_t(0x7FFFFFFFu) / d) * k / 64;
            for (int e = -1; e <= 1; ++e) {
                const int64_t n = int64_t(q * d) + e;
                if (n >= 0 && n <= 0x7FFFFFFF) chk(uint32_t(n), f);
            }
        }
        for (uint32_t n = 0x7FFFFFFFu - 64; n < 0x7FFFFFFFu; ++n) chk(n, f);
        chk(0x7FFFFFFFu, f);
    }
    for (uint32_t d : {1u, 2u, 3u, 7u, 15u, 16u, 64u, 1023u, 1024u, 7168u, 15360u}) {
        const ar::FastDiv f = ar::make_fastdiv(d);
        for (uint32_t n = 0; n < (1u << 24); ++n) chk(n, f);
    }
    std::mt19937_64 g(20261202);
    for (int i = 0; i < 4000000; ++i) {
        const uint32_t d = uint32_t(g() % 0x7FFFFFFFu) + 1u;
        chk(uint32_t(g() & 0x7FFFFFFFu), ar::make_fastdiv(d));
    }
    std::printf("checks %llu mismatches %llu\n", (unsigned long long)checks, (unsigned long long)bad);
    return bad == 0 ? 0 : 1;
}
