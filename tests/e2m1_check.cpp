// Compares the device E2M1 rounding (compiled for the host) with the oracle's
// encoder on every float bit pattern in [2^-4, 2^5) of both signs and on a
// sample below 2^-4 (all of which encode 0) and above 2^5 (all of which
// saturate).  Prints the number of mismatches and exits non-zero if there is
// any.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "mxfp8.h"

extern "C" uint8_t or_e2m1_from_double(double v);

int main() {
    uint64_t n = 0, bad = 0;
    auto check = [&](uint32_t u) {
        float x;
        std::memcpy(&x, &u, 4);
        const uint8_t a = moe::e2m1_rne(x), b = or_e2m1_from_double((double)x);
        ++n;
        if (a != b) {
            if (bad < 8) std::printf("mismatch: bits %08x (%g): device %x oracle %x\n", u, (double)x, a, b);
            ++bad;
        }
    };
    for (uint32_t s = 0; s < 2; ++s) {
        const uint32_t sg = s << 31;
        for (uint32_t u = 0; u < 0x3D800000u; u += 4093) check(sg | u);          // below 2^-4
        for (uint32_t u = 0x3D800000u; u < 0x42000000u; ++u) check(sg | u);     // [2^-4, 2^5)
        for (uint32_t u = 0x42000000u; u < 0x7F800000u; u += 4093) check(sg | u);  // 2^5 up to the largest float
    }
    std::printf("%llu values, %llu mismatches\n", (unsigned long long)n, (unsigned long long)bad);
    return bad != 0;
}
