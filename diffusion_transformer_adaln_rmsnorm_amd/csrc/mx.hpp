// MXFP4 (OCP Microscaling) element and scale helpers shared by the quantising kernels.
#pragma once

#include "common.hpp"

namespace dit {

// E8M0 scale byte of a block whose largest magnitude has bf16 bits amax: floor(log2(amax)) - 2 +
// 127 clamped to [0, 254], 0 for an all-zero block.  For a finite bf16 that is its exponent
// field minus 2, clamped at 0 (zero and subnormal maxima give 0; at most 252).
__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t amax) {
    const uint32_t ex = amax >> 7;
    return ex > 2u ? ex - 2u : 0u;
}

// Two E2M1 codes (one byte, the low half's code in the low nibble) of the bf16 pair w for scale
// 2^(E - 127) given as the float s, written into byte kByte of old: v_cvt_scalef32_pk_fp4_bf16
// divides by s (exactly: a power of two) and rounds to the nearest E2M1 value, ties to the even
// significand, saturating at 6 and keeping the sign (so -0 and small negative values give code 8).
// The pair arrives as a scalar: handed an element of a vector directly, the compiler has been seen
// to pass the vector's first element for every byte.
template <int kByte>
__device__ __forceinline__ uint32_t e2m1_pair(uint32_t old, uint32_t w, float s) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(old, __builtin_bit_cast(bf16x2, w), s, kByte);
}

// The 8 E2M1 codes of the 8 bf16 values of v in a block with scale byte E, element 2j in the low
// nibble of byte j (the nearest E2M1 value to v 2^(127 - E), as e2m1_pair rounds).  The scale
// 2^(E - 127) is a float: subnormal for E = 0.
__device__ __forceinline__ uint32_t e2m1_pack8(const u32x4& v, uint32_t E) {
    const float s = __uint_as_float(E != 0u ? E << 23 : 0x00400000u);
    const uint32_t w0 = v[0], w1 = v[1], w2 = v[2], w3 = v[3];
    uint32_t q = e2m1_pair<0>(0u, w0, s);
    q = e2m1_pair<1>(q, w1, s);
    q = e2m1_pair<2>(q, w2, s);
    return e2m1_pair<3>(q, w3, s);
}

// byte offset of the scale of row r, block b (values 32 b ..) of a [*, K] matrix in the MX scale
// layout: group r / 128, stage b / 8, lane r % 32 + 32 (b % 2), byte 4 ((r % 128) / 32) + (b % 8) / 2
__device__ __forceinline__ int64_t mx_scale_offset(int64_t r, int64_t b, int64_t K) {
    const int64_t lane = r % 32 + 32 * (b % 2);
    return ((r / 128) * (K / 256) + b / 8) * 1024 + lane * 16 + 4 * ((r % 128) / 32) + (b % 8) / 2;
}

}  // namespace dit
