// MXFP4 (OCP Microscaling) element and scale helpers shared by the quantising kernels.
#pragma once

#include "common.hpp"

namespace dit {

// E2M1 code (sign in bit 3) of the FP32 value y = v 2^(127 - E): the magnitude index counts the
// midpoints between neighbouring E2M1 values that |y| passes; at a midpoint it moves up only
// onto an even significand (midpoints after indices 1, 3, 5 count with >=, after 0, 2, 4, 6
// with >).  |y| >= 6 gives 7, the saturated maximum.
__device__ __forceinline__ uint32_t e2m1_code(float y) {
    const float a = fabsf(y);
    const uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
    return m | ((__float_as_uint(y) >> 28) & 8u);
}

// floor(log2(a)) of a positive finite float (normal or subnormal)
__device__ __forceinline__ int ilog2f(float a) {
    const uint32_t b = __float_as_uint(a);
    const int ex = (int)(b >> 23);
    return ex != 0 ? ex - 127 : (31 - __builtin_clz(b & 0x7FFFFFu)) - 149;
}

// E8M0 scale byte of a block with maximum magnitude amax: floor(log2(amax)) - 2 + 127, clamped
// to [0, 254]; 0 for an all-zero block
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
    if (!(amax > 0.f)) return 0u;
    const int e = ilog2f(amax) - 2 + 127;
    return (uint32_t)(e < 0 ? 0 : (e > 254 ? 254 : e));
}

// 2^(127 - E) as a normal float (E <= 252 for any finite bf16 amax)
__device__ __forceinline__ float mx_inv_scale(uint32_t E) { return __uint_as_float((254u - E) << 23); }

// four E2M1 codes of two packed bf16 pairs, element 2j in the low nibble of byte j
__device__ __forceinline__ uint32_t e2m1_pack4(uint32_t w0, uint32_t w1, float inv) {
    const uint32_t c0 = e2m1_code(bf_lo(w0) * inv), c1 = e2m1_code(bf_hi(w0) * inv);
    const uint32_t c2 = e2m1_code(bf_lo(w1) * inv), c3 = e2m1_code(bf_hi(w1) * inv);
    return (c0 | (c1 << 4)) | ((c2 | (c3 << 4)) << 8);
}

// byte offset of the scale of row r, block b (values 32 b ..) of a [*, K] matrix in the MX scale
// layout: group r / 128, stage b / 8, lane r % 16 + 16 (b % 4), byte 2 ((r % 128) / 16) + (b % 8) / 4
__device__ __forceinline__ int64_t mx_scale_offset(int64_t r, int64_t b, int64_t K) {
    const int64_t lane = r % 16 + 16 * (b % 4);
    return ((r / 128) * (K / 256) + b / 8) * 1024 + lane * 16 + 2 * ((r % 128) / 16) + (b % 8) / 4;
}

}  // namespace dit
