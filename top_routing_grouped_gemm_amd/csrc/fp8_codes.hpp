// OCP fp8 E4M3 encoding and the MX shared exponent, shared by the quantisers
// and the GEMM epilogue that re-quantises its output.
#pragma once

#include "moe_common.hpp"

namespace moe {

// float32 -> e4m3 code, round to nearest even, saturating at 448 (0x7E).
// Below 2^-6 the e4m3 grid is uniform with step 2^-9, so the code is the
// rounded multiple itself (a * 512 is exact); from 2^-6 up, rounding the
// float32 significand to 3 bits (carry into the exponent included) and
// rebiasing the exponent from 127 to 7 gives the code.
__device__ __forceinline__ uint32_t e4m3_rne(float r) {
    const uint32_t sign = (__float_as_uint(r) >> 24) & 0x80u;
    const float a = fabsf(r);
    uint32_t code;
    if (a < 0x1p-6f) {
        code = (uint32_t)__builtin_rintf(a * 512.0f);  // 0..8; 8 is the smallest normal, code 0x08
    } else {
        const uint32_t u = __float_as_uint(a);
        const uint32_t rounded = u + 0x7FFFFu + ((u >> 20) & 1u);
        code = min((rounded >> 20) - (120u << 3), 0x7Eu);
    }
    return code | sign;
}

// MX (OCP microscaling) shared exponent of a block with largest magnitude
// amax: floor(log2(amax)) - 8 (8 = exponent of the largest e4m3 power of
// two), 0 for an all-zero block, clamped to the E8M0 range [-127, 127].
__device__ __forceinline__ int mx_exponent(float amax) {
    if (amax == 0.0f) return 0;
    const int eb = (int)((__float_as_uint(amax) >> 23) & 0xffu);
    if (eb == 0) return -127;  // subnormal block maximum: below the E8M0 range
    return max(eb - 127 - 8, -127);
}

// Codes of four values of one MX block (exponent x), packed little-endian.
__device__ __forceinline__ uint32_t mx_codes4(float a, float b, float c, float d, int x) {
    return e4m3_rne(ldexpf(a, -x)) | (e4m3_rne(ldexpf(b, -x)) << 8) | (e4m3_rne(ldexpf(c, -x)) << 16) |
           (e4m3_rne(ldexpf(d, -x)) << 24);
}

}  // namespace moe
