// Per-head Q/K RMSNorm and split-half NeoX RoPE on packed bf16 values, shared by the QKV
// epilogues (the 256 x 256 tile of the QKV GEMM and the small-M kernel).
//
// FlashInfer "minimax_h3_bf16_pre_attention": description (per-head Q/K RMSNorm, then partial
// split-half NeoX RoPE on dims [0, 96)) and Parameters (q/k_norm_weight [128], qk_eps,
// rope_cos_sin [S, 96] with cos in columns [0, 48) and sin in [48, 96)).
//
// Layout: the 16 lanes of one DPP row own one (row, head), 8 dims each.  The chunks are placed
// so that the RoPE partner (pairs (j, j+48), i.e. chunk c and c + 6 for c < 6) is always 8
// lanes away: lanes 0-5 hold chunks 0-5, lanes 8-13 chunks 6-11, and lanes 6, 7, 14, 15 the
// pass-through chunks 12-15.  One row rotation by 8 then fetches every partner, with no
// lane-dependent choice (a DPP move must run with its source lanes active, which a select
// lowered to a branch would break).
#pragma once

#include "common.hpp"

namespace dit {

// Cross-lane moves inside a 16-lane DPP row (VALU, no LDS round trip).
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}
// (for moves whose source lane always exists, e.g. row rotations)
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kCtrl, 0xF, 0xF, true);
}
constexpr int kDppXor1 = 0xB1;         // quad_perm(1,0,3,2): lane i <- i ^ 1
constexpr int kDppXor2 = 0x4E;         // quad_perm(2,3,0,1): lane i <- i ^ 2
constexpr int kDppHalfMirror = 0x141;  // lane i <- 7 - i within each 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <- 15 - i within each 16 lanes
constexpr int kDppRor8 = 0x128;        // row_ror:8: lane i <- (i + 8) mod 16

// v_perm_b32 selectors on (src0, src1): low halves (src1.lo | src0.lo << 16) and high halves
// (src1.hi | src0.hi << 16), and the same with the sources' places swapped (src0.lo | src1.lo << 16,
// src0.hi | src1.hi << 16).
constexpr uint32_t kPermLo = 0x05040100u;
constexpr uint32_t kPermHi = 0x07060302u;
constexpr uint32_t kPermLoSwap = 0x01000504u;
constexpr uint32_t kPermHiSwap = 0x03020706u;

// Sum over the 16 lanes of a DPP row, left in every lane of it.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f<kDppXor1>(x);
    x += dpp_f<kDppXor2>(x);
    x += dpp_f<kDppHalfMirror>(x);    // pairs the two quads of each 8
    x += dpp_f<kDppMirror>(x);        // pairs the two 8s of the row
    return x;
}

// Q/K output of one (row, head) for the 16 lanes of a DPP row: vp holds this lane's 8 dims
// (chunk q) of the head as bf16; nwlo / nwhi its 8 norm weights as bf16 pairs with the high /
// low half zeroed; cs this lane's 16 bytes of the row's cos/sin: the cos of frequencies
// 8 q .. 8 q + 7 (q < 6) or the sin of frequencies 8 (q - 6) .. (6 <= q < 12).  The partner
// lane (chunk q +/- 6, 8 lanes away) holds the other one, so each lane loads half of what its
// rotation takes and one row rotation completes it.  All 16 lanes of the row must be active.
__device__ __forceinline__ u32x4 qk_norm_rope(const u32x4& vp, const u32x4& nwlo, const u32x4& nwhi, float qk_eps,
                                              int q, const u32x4& cs) {
    // per-head RMSNorm in fp32 on the packed bf16 values: the squares and v w are exact
    // bf16 products (v_dot2; a zero half picks one product), the sum of squares carries fp32
    // rounding (v_dot2's) only, and u = bf16((v w) r2); two partial sums halve the dependent chain
    float sq[4];
    dot2x4_zero(vp[0], vp[0], vp[1], vp[1], vp[2], vp[2], vp[3], vp[3], sq);
    const float ss = row16_sum((sq[0] + sq[1]) + (sq[2] + sq[3]));   // a (row, head)'s 16 lanes are one DPP row
    // v_rsq_f32 directly: its argument is at least qk_eps, a normal float, where the library
    // rsqrtf adds only a denormal-range rescaling around the same instruction
    const float r2 = __builtin_amdgcn_rsqf(ss * (1.0f / kHeadDim) + qk_eps);
    float u[8], vw[8];
    dot2x4_zero(vp[0], nwlo[0], vp[0], nwhi[0], vp[1], nwlo[1], vp[1], nwhi[1], *reinterpret_cast<float(*)[4]>(vw));
    dot2x4_zero(vp[2], nwlo[2], vp[2], nwhi[2], vp[3], nwlo[3], vp[3], nwhi[3], *reinterpret_cast<float(*)[4]>(vw + 4));
#pragma unroll
    for (int e = 0; e < 8; ++e) u[e] = vw[e] * r2;
    const u32x4 up = pack8(u);          // the bf16 u, packed
    // RoPE partner chunk q + 6 (q < 6) or q - 6 (6 <= q < 12), 8 lanes away; its sign flipped
    // for the first half, so both halves take o = u c + w s:
    // o_j = u_j c - u_{j+48} s, o_{j+48} = u_{j+48} c + u_j s
    const uint32_t sgn = q < 6 ? 0x80008000u : 0u;   // negates both bf16 halves of a word
    u32x4 pv, pc;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        pv[e] = dpp_u<kDppRor8>(up[e]) ^ sgn;
        pc[e] = dpp_u<kDppRor8>(cs[e]);     // the partner's cos/sin half: sin (q < 6) or cos
    }
    if (q >= 12) return up;
    // o = u c + w s per element as one v_dot2 of the bf16 pairs (u, w) and (c, s): the two
    // products are exact in fp32 and their sum is rounded to fp32 (within one ulp of the
    // correctly rounded sum that the fma form u c + (w s) gives, equal to it nearly always).
    // (c, s) pairs: cos from this lane (q < 6) or from the partner, through the selector.
    const uint32_t sel_lo = q < 6 ? kPermLo : kPermLoSwap, sel_hi = q < 6 ? kPermHi : kPermHiSwap;
    uint32_t uw[8], cw[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        uw[2 * e] = __builtin_amdgcn_perm(pv[e], up[e], kPermLo);       // (u_2e, w_2e)
        uw[2 * e + 1] = __builtin_amdgcn_perm(pv[e], up[e], kPermHi);   // (u_2e+1, w_2e+1)
        cw[2 * e] = __builtin_amdgcn_perm(pc[e], cs[e], sel_lo);        // (c_2e, s_2e)
        cw[2 * e + 1] = __builtin_amdgcn_perm(pc[e], cs[e], sel_hi);    // (c_2e+1, s_2e+1)
    }
    float o[8];
    dot2x4_zero(uw[0], cw[0], uw[1], cw[1], uw[2], cw[2], uw[3], cw[3], *reinterpret_cast<float(*)[4]>(o));
    dot2x4_zero(uw[4], cw[4], uw[5], cw[5], uw[6], cw[6], uw[7], cw[7], *reinterpret_cast<float(*)[4]>(o + 4));
    return pack8(o);
}

// 8-dim chunk of a head held by lane li of its DPP row (the partner chunk q +/- 6 sits at
// lane li ^ 8): lanes 0-5 hold chunks 0-5, lanes 8-13 chunks 6-11, lanes 6, 7, 14, 15 the
// pass-through chunks 12-15.
__device__ __forceinline__ int chunk_of_lane(int li) {
    return li < 6 ? li : (li < 8 ? 12 + (li - 6) : (li < 14 ? li - 2 : li));
}

}  // namespace dit
