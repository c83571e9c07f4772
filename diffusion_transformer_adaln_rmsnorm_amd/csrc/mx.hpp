// MXFP4 (OCP Microscaling) element and scale helpers shared by the quantising kernels.
#pragma once

#include "common.hpp"

namespace dit {

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

// four E2M1 codes of two packed bf16 pairs, element 2j in the low nibble of byte j.  The
// magnitudes |v| 2^(127 - E) (exact in FP32 wherever they can round to a nonzero code) go
// through v_cvt_scalef32_pk_fp4_f32 with a unit scale: round to nearest, ties to the even
// significand, saturating at 6.  The sign bits are taken from the bf16 values themselves, so
// -0 and negative values that round to 0 keep their sign.
__device__ __forceinline__ uint32_t e2m1_pack4(uint32_t w0, uint32_t w1, float inv) {
    uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, fabsf(bf_lo(w0) * inv), fabsf(bf_hi(w0) * inv), 1.0f, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, fabsf(bf_lo(w1) * inv), fabsf(bf_hi(w1) * inv), 1.0f, 1);
    // bf16 sign bits 15 and 31 of each word -> bit 3 of nibbles 0, 1 (w0) and 2, 3 (w1)
    const uint32_t sgn = ((w0 >> 12) & 0x8u) | ((w0 >> 24) & 0x80u) | ((w1 >> 4) & 0x800u) | ((w1 >> 16) & 0x8000u);
    return (r & 0xFFFFu) | sgn;
}

// byte offset of the scale of row r, block b (values 32 b ..) of a [*, K] matrix in the MX scale
// layout: group r / 128, stage b / 8, lane r % 32 + 32 (b % 2), byte 4 ((r % 128) / 32) + (b % 8) / 2
__device__ __forceinline__ int64_t mx_scale_offset(int64_t r, int64_t b, int64_t K) {
    const int64_t lane = r % 32 + 32 * (b % 2);
    return ((r / 128) * (K / 256) + b / 8) * 1024 + lane * 16 + 4 * ((r % 128) / 32) + (b % 8) / 2;
}

}  // namespace dit
