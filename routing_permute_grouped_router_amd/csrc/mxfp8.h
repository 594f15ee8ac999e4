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
// smallest subnormal 2^-9), saturating to +-448.  Finite input.
__device__ __forceinline__ uint8_t e4m3_rne(float x) {
    const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
    const float a = fabsf(x);
    if (a >= 464.0f) return (uint8_t)(sign | 0x7Eu);  // 464 ties to 448; above rounds past 448
    if (a < 0.015625f) {                                // below 2^-6: subnormal, quantum 2^-9
        const int m = (int)__builtin_rintf(a * 512.0f);  // exact scaling; RNE; m in [0, 8]
        return (uint8_t)(sign | (uint32_t)m);           // m == 8 encodes 2^-6 exactly
    }
    int ex = ilogbf(a);                                           // a in [2^ex, 2^(ex+1)), ex >= -6
    int q = (int)__builtin_rintf(ldexpf(a, 3 - ex));              // in [8, 16]
    if (q == 16) {
        q = 8;
        ++ex;
    }
    uint32_t code = ((uint32_t)(ex + 7) << 3) | (uint32_t)(q - 8);
    if (code > 0x7Eu) code = 0x7Eu;
    return (uint8_t)(sign | code);
}

}  // namespace moe
