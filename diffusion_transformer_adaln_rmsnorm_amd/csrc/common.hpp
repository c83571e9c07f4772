// Device helpers shared by the gfx950 kernels: vector types, bf16/e4m3 conversions,
// wavefront reductions.  CDNA4 only (64-lane wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

constexpr int kHidden = 5376;
constexpr int kHeads = 56;
constexpr int kHeadDim = 128;
constexpr int kQkvRows = 3 * kHeads * kHeadDim;   // 21504
constexpr int kAttnWidth = kHeads * kHeadDim;     // 7168
constexpr int kRopeCols = 96;
constexpr int kNFreq = 48;
constexpr int kInter = 14336;
constexpr int kFc1Rows = 2 * kInter;              // 28672

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 bit pattern -> float (exact)
__device__ __forceinline__ float bf2f(uint32_t b16) { return __uint_as_float(b16 << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest even (gfx950 v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t f2bf(float f) {
    __bf16 b = (__bf16)f;
    return (uint32_t)__builtin_bit_cast(uint16_t, b);
}
// two floats -> two bf16 (lo in bits 0-15), both rounded to nearest even by one
// v_cvt_pk_bf16_f32
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    const bf16x2 b = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}
// round a float to the nearest bf16 value, returned as float
__device__ __forceinline__ float rbf(float f) { return bf2f(f2bf(f)); }

// a.lo b.lo + a.hi b.hi + c for two packed bf16 pairs (v_dot2_f32_bf16, FP32 result).  The bf16
// products are exact, but the sum is not always the correctly rounded one: measured against
// exact sums of random terms it is one FP32 ulp off in about 1 case in 2000 with c = 0 (terms of
// very different size) and in about 1 in 20 with a general c, and products below 2^-126 are
// flushed to zero.  Where the exact sum is an FP32 value (1 + s for a bf16 s of magnitude at
// least 2^-16, say) it is exact.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c = 0.0f) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// r_i = a_i.lo b_i.lo + a_i.hi b_i.hi for four independent bf16 pairs, by the three-operand
// v_dot2_f32_bf16 with an inline zero addend.  For dot2_bf16 the compiler emits the accumulating
// two-operand form, which takes a freshly zeroed register per use; this form takes none.  A
// VALU instruction may read a three-operand v_dot2's result only 3 wait states after it is
// written: the compiler pads its own uses (s_nop 2) but sees nothing inside an asm block, so
// the block ends with those wait states.
__device__ __forceinline__ void dot2x4_zero(uint32_t a0, uint32_t b0, uint32_t a1, uint32_t b1, uint32_t a2,
                                            uint32_t b2, uint32_t a3, uint32_t b3, float (&r)[4]) {
    asm("v_dot2_f32_bf16 %0, %4, %5, 0\n\t"
        "v_dot2_f32_bf16 %1, %6, %7, 0\n\t"
        "v_dot2_f32_bf16 %2, %8, %9, 0\n\t"
        "v_dot2_f32_bf16 %3, %10, %11, 0\n\t"
        "s_nop 2"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(a0), "v"(b0), "v"(a1), "v"(b1), "v"(a2), "v"(b2), "v"(a3), "v"(b3));
}

// RoPE of four pairs by eight three-operand v_dot2 with an inline zero addend: with
// ua_e = (u_e, w_e), ub_e = (w_e, u_e) and cs_e = (c_e, s_e) (bf16 pairs),
//   o_e = u_e c_e - w_e s_e (neg_hi negates the high half of cs_e),  o_(4+e) = w_e c_e + u_e s_e,
// each product exact and the sum rounded once; the block ends with the wait states of dot2x4_zero.
__device__ __forceinline__ void rope_dot2x8(const uint32_t (&ua)[4], const uint32_t (&ub)[4], const uint32_t (&cs)[4],
                                            float (&o)[8]) {
    asm("v_dot2_f32_bf16 %0, %8, %16, 0 neg_hi:[0,1,0]\n\t"
        "v_dot2_f32_bf16 %1, %9, %17, 0 neg_hi:[0,1,0]\n\t"
        "v_dot2_f32_bf16 %2, %10, %18, 0 neg_hi:[0,1,0]\n\t"
        "v_dot2_f32_bf16 %3, %11, %19, 0 neg_hi:[0,1,0]\n\t"
        "v_dot2_f32_bf16 %4, %12, %16, 0\n\t"
        "v_dot2_f32_bf16 %5, %13, %17, 0\n\t"
        "v_dot2_f32_bf16 %6, %14, %18, 0\n\t"
        "v_dot2_f32_bf16 %7, %15, %19, 0\n\t"
        "s_nop 2"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
        : "v"(ua[0]), "v"(ua[1]), "v"(ua[2]), "v"(ua[3]), "v"(ub[0]), "v"(ub[1]), "v"(ub[2]), "v"(ub[3]),
          "v"(cs[0]), "v"(cs[1]), "v"(cs[2]), "v"(cs[3]));
}

// 1 + s for the eight bf16 values of four packed words s0 .. s3: per value one three-operand
// v_dot2 of its word with a unit weight on its half, plus the inline addend 1.0 (r[2i] from the
// low half of s_i, r[2i + 1] from the high half).  The weights sit in SGPRs; the block ends with
// the wait states of dot2x4_zero.  Exact wherever 1 + s is an FP32 value.
__device__ __forceinline__ void one_plus_x8(uint32_t s0, uint32_t s1, uint32_t s2, uint32_t s3, float (&r)[8]) {
    asm("v_dot2_f32_bf16 %0, %8, %12, 1.0\n\t"
        "v_dot2_f32_bf16 %1, %8, %13, 1.0\n\t"
        "v_dot2_f32_bf16 %2, %9, %12, 1.0\n\t"
        "v_dot2_f32_bf16 %3, %9, %13, 1.0\n\t"
        "v_dot2_f32_bf16 %4, %10, %12, 1.0\n\t"
        "v_dot2_f32_bf16 %5, %10, %13, 1.0\n\t"
        "v_dot2_f32_bf16 %6, %11, %12, 1.0\n\t"
        "v_dot2_f32_bf16 %7, %11, %13, 1.0\n\t"
        "s_nop 2"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(s0), "v"(s1), "v"(s2), "v"(s3), "s"(0x00003F80u), "s"(0x3F800000u));
}

// a / s rounded to nearest, given y = RN(1 / s) (one division per row instead of one per
// element): q0 = RN(a y), the remainder a - q0 s by fma, and one fma correction (Markstein's
// final step for a correctly rounded reciprocal).  For s > 0 the quotient has a's sign, which
// is put back on the result: the correction alone would turn the quotient of a = -0 into +0
// (everywhere else the sign is already a's, as the correction is below an ulp of q0).
__device__ __forceinline__ float div_by(float a, float s, float y) {
    const float q0 = a * y;
    const float r = fmaf(-q0, s, a);
    return __builtin_copysignf(fmaf(r, y, q0), a);
}

// fl32(a / s) for a positive per-row scale s: div_by with y = RN(1 / s) when s is a normal
// float, an IEEE division when s is subnormal.  Below 2^-126 the reciprocal can overflow (s <
// 2^-128), which would turn div_by's product into inf or NaN, and the fma remainder is no
// longer exact.  The choice is uniform over a row, so a wavefront that owns a row never splits.
__device__ __forceinline__ float div_row(float a, float s, float y, bool s_normal) {
    return s_normal ? div_by(a, s, y) : a / s;
}

// silu(t) = t / (1 + e^-t) from the hardware exp2 and reciprocal (each ~1 ulp); e^-t -> inf
// gives 0 and e^-t -> 0 gives t, the limits
__device__ __forceinline__ float silu_fast(float t) {
    const float ex = __builtin_amdgcn_exp2f(-t * 1.4426950408889634f);
    return t * __builtin_amdgcn_rcpf(1.0f + ex);
}

// unpack 8 bf16 (one 16-byte vector) to floats
__device__ __forceinline__ void unpack8(const u32x4& v, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf_lo(v[i]);
        f[2 * i + 1] = bf_hi(v[i]);
    }
}
__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = pack_bf2(f[2 * i], f[2 * i + 1]);
    return v;
}

// Two floats -> two float8_e4m3fn codes in the low 16 bits (OCP format on gfx950),
// round to nearest even; inputs are clamped to +-448 first so that magnitudes beyond the
// largest code saturate.
__device__ __forceinline__ uint32_t f2e4m3x2(float a, float b) {
    a = fminf(fmaxf(a, -448.0f), 448.0f);
    b = fminf(fmaxf(b, -448.0f), 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Largest magnitude among the 8 bf16 values of v, as bf16 bits with the sign cleared: for
// finite values the order of |v| is the unsigned order of those bits (two 16-bit maxima per
// instruction).  As float bits (<< 16) it is that magnitude in FP32.
__device__ __forceinline__ uint32_t amax_bits8(const u32x4& v) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    u16x2 m = __builtin_bit_cast(u16x2, v[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int e = 1; e < 4; ++e) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, v[e] & 0x7FFF7FFFu));
    return m.x > m.y ? m.x : m.y;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// Streaming (non-temporal) 16-byte load for data touched once.
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
// Streaming (non-temporal) 16-byte store for outputs the writer never reads back.
__device__ __forceinline__ void st16_nt(void* p, const u32x4& v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

}  // namespace dit
