// Compares the device E4M3 rounding (compiled for the host) with the oracle's
// encoder on every float bit pattern in [2^-10, 2^10) of both signs and on a
// sample below 2^-10 (all of which encode 0 or the smallest subnormals).
// Prints the number of mismatches and exits non-zero if there is any.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "mxfp8.h"

extern "C" uint8_t or_e4m3_from_double(double v);

int main() {
    uint64_t n = 0, bad = 0;
    auto check = [&](uint32_t u) {
        float x;
        std::memcpy(&x, &u, 4);
        const uint8_t a = moe::e4m3_rne(x), b = or_e4m3_from_double((double)x);
        ++n;
        if (a != b) {
            if (bad < 8) std::printf("mismatch: bits %08x (%g): device %02x oracle %02x\n", u, (double)x, a, b);
            ++bad;
        }
    };
    for (uint32_t s = 0; s < 2; ++s) {
        const uint32_t sg = s << 31;
        for (uint32_t u = 0; u < 0x3A800000u; u += 4093) check(sg | u);           // below 2^-10
        for (uint32_t u = 0x3A800000u; u < 0x44800000u; ++u) check(sg | u);      // [2^-10, 2^10)
    }
    std::printf("%llu values, %llu mismatches\n", (unsigned long long)n, (unsigned long long)bad);
    return bad != 0;
}
