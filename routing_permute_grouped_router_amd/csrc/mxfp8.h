// Device helpers for MX encoding (OCP MX v1.0: E4M3 or E2M1 elements, E8M0
// scales).
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

// MXFP4: shared exponent floor(log2(amax)) - 2 (E2M1's largest normal is
// 1.5 * 2^2), clamped to [-127, 127]; an all-zero block gets -127.
__device__ __forceinline__ int mx4_shared_exp(float amax) {
    if (!(amax > 0.f)) return -127;
    int se = ilogbf(amax) - 2;
    return se < -127 ? -127 : (se > 127 ? 127 : se);
}

// Round-to-nearest-even to OCP E2M1 (bias 1, 1 mantissa bit, largest 6,
// subnormal 0.5), saturating to +-6; finite input; a 4-bit code with the sign
// in bit 3 (a value that rounds to zero keeps its sign).  Branch-free on the
// bits of |x|:
//   - from 1 up: round the float's 23-bit mantissa to 1 bit (add half a unit
//     less one plus the kept bit: ties go to even; a carry moves into the
//     exponent); the code is then (unbiased exponent + 1) * 2 + mantissa bit,
//     which is (bits >> 22) - 252;
//   - below 1: the multiple of the subnormal quantum 0.5 (RNE), 0, 1 or 2, and
//     2 is the code of 1.0;
//   - 6 and up: the largest code (the next E2M1 step above 6 would be 8).
__host__ __device__ inline uint8_t e2m1_rne(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const uint32_t sign = (u >> 28) & 0x8u, a = u & 0x7FFFFFFFu;
    const uint32_t r = a + 0x1FFFFFu + ((a >> 22) & 1u);
    uint32_t code = (r >> 22) - 252u;
    const uint32_t m = (uint32_t)__builtin_rintf(__builtin_bit_cast(float, a) * 2.0f);
    code = a < 0x3F800000u ? m : code;    // below 1
    code = a >= 0x40C00000u ? 7u : code;  // 6 and above
    return (uint8_t)(sign | code);
}

}  // namespace moe
