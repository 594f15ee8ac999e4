// Device helpers for MXFP8 encoding (OCP MX v1.0: E4M3 elements, E8M0 scales).
#pragma once

#include "moe_internal.h"

namespace moe {

// Shared exponent of a block with the given max |v|: floor(log2(amax)) - 8,
// clamped to [-127, 127]; an all-zero block gets -127 (scale code 0).
__device__ __forceinline__ int mx_shared_exp(float amax) {
    if (!(amax > 0.f)) return -127;
    int se = ilogbf(amax) - 8;
    return se < -127 ? -127 : (se > 127 ? 127 : se);
}

// Round-to-nearest-even to OCP E4M3 (bias 7, 3 mantissa bits, largest 448,
// smallest subnormal 2^-9), saturating to +-448; finite input.  Branch-free
// on the bits of |x| (every lane takes the same path):
//   - from 2^-6 up: round the float's 23-bit mantissa to 3 bits (add half a
//     unit less one plus the kept lowest bit: ties go to even; a carry moves
//     into the exponent) and rebias the exponent from 127 to 7;
//   - below 2^-6: the multiple of the subnormal quantum 2^-9 (RNE; 8 of them
//     encode 2^-6);
//   - 464 (the midpoint of 448 and the next E4M3 step, ties to 448) and up:
//     the largest finite code.
__host__ __device__ inline uint8_t e4m3_rne(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const uint32_t sign = (u >> 24) & 0x80u, a = u & 0x7FFFFFFFu;
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    uint32_t code = (r >> 20) - (120u << 3);
    code = code > 0x7Eu ? 0x7Eu : code;
    const uint32_t m = (uint32_t)__builtin_rintf(__builtin_bit_cast(float, a) * 512.0f);
    code = a < 0x3C800000u ? m : code;   // below 2^-6
    code = a >= 0x43E80000u ? 0x7Eu : code;  // 464 and above
    return (uint8_t)(sign | code);
}

}  // namespace moe
