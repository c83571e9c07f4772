// QKV projection with the fused Q/K RMSNorm, RoPE and pack epilogue (launch 2 of the bf16
// pre-attention stage).
//
// FlashInfer "minimax_h3_bf16_pre_attention": description (GEMM streams the workspace, the
// epilogue applies the per-head Q/K RMSNorm, partial split-half NeoX RoPE and the
// destination-major pack) and Parameters (qkv_weight row order [q_all | k_all | v_all] x 56
// heads x 128, q/k_norm_weight [128], rope_cos_sin [S, 96] with cos in columns [0,48) and sin
// in [48,96), rope_positions clamped to [0, S) or the identity, out [P, M, 56 / P, 3, 128] for
// P = ulysses_degree destinations, destination p holding heads [p 56/P, (p+1) 56/P)).
//
// A 256-wide n tile is exactly two heads of one kind (7168 = 28 x 256), so each tile owns
// whole heads and needs nothing from its neighbours.  After the main loop the tile is
// rounded to bf16 into LDS; then the 16 lanes of one DPP row own one (row, head), 8 dims
// each, and a 4-step DPP reduction gives the head's sum of squares.  The chunks are placed
// so that the RoPE partner (pairs (j, j+48), i.e. chunk c and c + 6 for c < 6) is always 8
// lanes away: lanes 0-5 hold chunks 0-5, lanes 8-13 chunks 6-11, and lanes 6, 7, 14, 15 the
// pass-through chunks 12-15.  One row rotation by 8 then fetches every partner, with no
// lane-dependent choice (a DPP move must run with its source lanes active, which a select
// lowered to a branch would break).  Each lane writes 16 contiguous bytes of out, so the 16
// lanes of a head store its 256 bytes in one piece.
#include "common.hpp"
#include "gemm.hpp"
#include "kernels.hpp"

namespace dit {

using namespace gemm;

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
// (src1.hi | src0.hi << 16).
constexpr uint32_t kPermLo = 0x05040100u;
constexpr uint32_t kPermHi = 0x07060302u;
// a.lo b.lo + a.hi b.hi (+ c) for two packed bf16 pairs (v_dot2_f32_bf16, fp32 result; the
// bf16 products are exact)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c = 0.0f) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

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
// low half zeroed; cv / sv the cos and sin of frequencies 8 (q mod 6) .. + 7 for the row's
// position (q < 12).  All 16 lanes of the row must be active.
__device__ __forceinline__ u32x4 qk_norm_rope(const u32x4& vp, const u32x4& nwlo, const u32x4& nwhi, float qk_eps,
                                              int q, const u32x4& cv, const u32x4& sv) {
    // per-head RMSNorm in fp32 on the packed bf16 values: the squares and v w are exact
    // bf16 products (v_dot2; a zero half picks one product), the sum of squares carries fp32
    // rounding only, and u = bf16((v w) r2); two partial sums halve the dependent chain
    const float s0 = dot2_bf16(vp[1], vp[1], dot2_bf16(vp[0], vp[0]));
    const float s1 = dot2_bf16(vp[3], vp[3], dot2_bf16(vp[2], vp[2]));
    const float ss = row16_sum(s0 + s1);   // the 16 lanes of a (row, head) are one DPP row
    // v_rsq_f32 directly: its argument is at least qk_eps, a normal float, where the library
    // rsqrtf adds only a denormal-range rescaling around the same instruction
    const float r2 = __builtin_amdgcn_rsqf(ss * (1.0f / kHeadDim) + qk_eps);
    float u[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        u[2 * e] = dot2_bf16(vp[e], nwlo[e]) * r2;
        u[2 * e + 1] = dot2_bf16(vp[e], nwhi[e]) * r2;
    }
    const u32x4 up = pack8(u);          // the bf16 u, packed
    // RoPE partner chunk q + 6 (q < 6) or q - 6 (6 <= q < 12), 8 lanes away; its sign flipped
    // for the first half, so both halves take o = u c + w s:
    // o_j = u_j c - u_{j+48} s, o_{j+48} = u_{j+48} c + u_j s
    const uint32_t sgn = q < 6 ? 0x80008000u : 0u;   // negates both bf16 halves of a word
    u32x4 pv;
#pragma unroll
    for (int e = 0; e < 4; ++e) pv[e] = dpp_u<kDppRor8>(up[e]) ^ sgn;
    if (q >= 12) return up;
    // o = u c + w s per element as one v_dot2 of the bf16 pairs (u, w) and (c, s): the two
    // products are exact in fp32 and their sum is rounded once, as the fma form u c + (w s) is
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t uw0 = __builtin_amdgcn_perm(pv[e], up[e], kPermLo);   // (u_2e, w_2e)
        const uint32_t uw1 = __builtin_amdgcn_perm(pv[e], up[e], kPermHi);   // (u_2e+1, w_2e+1)
        const uint32_t cs0 = __builtin_amdgcn_perm(sv[e], cv[e], kPermLo);
        const uint32_t cs1 = __builtin_amdgcn_perm(sv[e], cv[e], kPermHi);
        r[e] = pack_bf2(dot2_bf16(uw0, cs0), dot2_bf16(uw1, cs1));
    }
    return r;
}

// 8-dim chunk of a head held by lane li of its DPP row (the partner chunk q +/- 6 sits at
// lane li ^ 8): lanes 0-5 hold chunks 0-5, lanes 8-13 chunks 6-11, lanes 6, 7, 14, 15 the
// pass-through chunks 12-15.
__device__ __forceinline__ int chunk_of_lane(int li) {
    return li < 6 ? li : (li < 8 ? 12 + (li - 6) : (li < 14 ? li - 2 : li));
}

// a / s rounded to nearest (div_by), except that quotients far beyond the largest e4m3 value
// (which saturate either way) skip the correction, which an infinite first guess would turn
// into NaN
__device__ __forceinline__ float div_sat(float a, float s, float y) {
    const float q0 = a * y;
    return fabsf(q0) > 1024.0f ? q0 : div_by(a, s, y);
}

// e4m3 output mode ("minimax_h3_nvfp4_pre_attention", Parameters: out_mode "e4m3" with
// per-tensor q/k/v dequantization scales): the 8 bf16 values of o become e4m3(fl32(v / ds)),
// saturating at 448, packed little-endian into 8 bytes.  y = RN(1 / ds).
__device__ __forceinline__ u32x2 e4m3_codes8(const u32x4& o, float ds, float y) {
    float v[8];
    unpack8(o, v);
    u32x2 q;
    q.x = f2e4m3x2(div_sat(v[0], ds, y), div_sat(v[1], ds, y)) | (f2e4m3x2(div_sat(v[2], ds, y), div_sat(v[3], ds, y)) << 16);
    q.y = f2e4m3x2(div_sat(v[4], ds, y), div_sat(v[5], ds, y)) | (f2e4m3x2(div_sat(v[6], ds, y), div_sat(v[7], ds, y)) << 16);
    return q;
}

// The QKV epilogue of one 256 x 256 tile after the main loop (acc of this wave): Q/K RMSNorm,
// RoPE and the pack, or V as is.  kE4m3: out holds e4m3 codes (one byte per element) of the
// bf16 results divided by the descale of their kind (dq, dk, dv); else bf16 values.
template <bool kE4m3>
__device__ __forceinline__ void qkv_epilogue(Acc& acc, uint8_t* smem, int64_t m0, int64_t M, int n0,
                                             const uint16_t* __restrict__ qw, const uint16_t* __restrict__ kw,
                                             const uint16_t* __restrict__ cs, int64_t S,
                                             const int64_t* __restrict__ pos, float qk_eps, int hpd, float dq,
                                             float dk, float dv, void* __restrict__ out) {
    const int t = threadIdx.x;
    const int li = t & 15;              // lane within the (row, head) group
    // 8-dim chunk of the head held by this lane (partner chunk q +/- 6 sits at lane li ^ 8)
    const int q = chunk_of_lane(li);
    const int hh = (t >> 4) & 1;        // which of the tile's two heads
    const int rsub = t >> 5;            // 0..kThreads/32-1
    const int kind = n0 / kAttnWidth;   // 0 q, 1 k, 2 v
    const int head = (n0 % kAttnWidth) / kHeadDim + hh;
    // destination-major pack: destination dst takes heads [dst * hpd, (dst + 1) * hpd) of every
    // token (hpd = 56 / P), out[dst, m, hl, kind, :]
    const int dst = head / hpd, hl = head - dst * hpd;
    const int d0 = q * 8;
    const int j0 = (q % 6) * 8;         // frequency index of this chunk (q < 12)

    // Every global operand of the epilogue is requested before it is needed, so the loop
    // below pays one memory latency per tile rather than one per row: the positions of this
    // thread's kIters rows now (they land while the accumulators are staged), the cos/sin
    // rows right after the staging.  All epilogue loads and stores go through buffer descriptors and are
    // issued unconditionally (out-of-range lanes read zeros, stores past M are dropped).
    constexpr int kRowsPerPass = kThreads / 32;
    constexpr int kIters = kBM / kRowsPerPass;
    const bool need_cs = kind < 2 && q < 12;
    const __amdgpu_buffer_rsrc_t rcs = make_rsrc(cs, kind < 2 ? (uint32_t)(S * kRopeCols * 2) : 0u);
    const __amdgpu_buffer_rsrc_t rpos = make_rsrc(pos, pos ? (uint32_t)(M * 8) : 0u);
    const int64_t tile_rows = M - m0 < kBM ? M - m0 : kBM;
    constexpr int64_t kOutRow = (int64_t)kHeads * 3 * kHeadDim;        // elements per token
    constexpr int64_t kElemB = kE4m3 ? 1 : 2;                         // bytes per output element
    uint8_t* const out8 = static_cast<uint8_t*>(out);
    const __amdgpu_buffer_rsrc_t rout = make_rsrc(out8 + m0 * kOutRow * kElemB,
                                                  (uint32_t)(tile_rows * kOutRow * kElemB));
    // P = 1: byte offset (within the tile's rows) of this lane's 8 elements in the first pass;
    // each pass moves kRowsPerPass rows on
    const uint32_t o1 = (uint32_t)((((rsub * kHeads + head) * 3 + kind) * kHeadDim + d0) * kElemB);
    constexpr uint32_t kPassB = (uint32_t)(kRowsPerPass * kOutRow * kElemB);
    const float ds = kind == 0 ? dq : (kind == 1 ? dk : dv);          // this tile's descale
    const float ds_inv = kE4m3 ? 1.0f / ds : 0.0f;                     // RN(1 / ds)
    u32x4 nwv = {0u, 0u, 0u, 0u};       // this lane's 8 q/k norm weights
    if (kind < 2) nwv = ld16((kind == 0 ? qw : kw) + d0);
    int64_t praw[kIters];               // raw positions (read only when pos is given)
    if (pos != nullptr && kind < 2) {
#pragma unroll
        for (int it = 0; it < kIters; ++it)
            praw[it] = buf_ld_i64(rpos, (uint32_t)((m0 + it * kRowsPerPass + rsub) * 8));
    }

    stage_tile_bf16(acc, smem, nullptr, m0, M, nullptr, nullptr);
    // the cos/sin rows are requested once the accumulators are free and before the barrier, so
    // they are in flight while the other waves finish staging
    u32x4 cv[kIters], sv[kIters];
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
        const int64_t m = m0 + it * kRowsPerPass + rsub;
        const int64_t p = pos != nullptr ? praw[it] : m;      // identity positions: the row
        const int64_t pc = p < 0 ? 0 : (p > S - 1 ? S - 1 : p);
        const uint32_t off = need_cs ? (uint32_t)((pc * kRopeCols + j0) * 2) : kOffNone;
        cv[it] = buf_ld16(rcs, off);
        sv[it] = buf_ld16(rcs, off + (need_cs ? kNFreq * 2 : 0u));
    }
    __syncthreads();

    u32x4 nwlo, nwhi;                   // the norm weights, one bf16 of each pair kept
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        nwlo[e] = nwv[e] & 0xFFFFu;
        nwhi[e] = nwv[e] & 0xFFFF0000u;
    }

#pragma unroll
    for (int it = 0; it < kIters; ++it) {
        const int row = it * kRowsPerPass + rsub;
        const u32x4 vp = epi_ld(smem, row, hh * 128 + d0);
        u32x4 o = vp;
        if (kind < 2) o = qk_norm_rope(vp, nwlo, nwhi, qk_eps, q, cv[it], sv[it]);
        // one destination: rows past M fall outside rout and are dropped; else out[dst, m, hl, ...]
        const uint32_t e1 = o1 + (uint32_t)it * kPassB;
        const int64_t m = m0 + row;
        const int64_t eP = (((dst * M + m) * hpd + hl) * 3 + kind) * kHeadDim + d0;
        if constexpr (kE4m3) {
            const u32x2 q = e4m3_codes8(o, ds, ds_inv);
            if (hpd == kHeads) {
                __builtin_amdgcn_raw_buffer_store_b64(q, rout, (int)e1, 0, 0);
            } else if (m < M) {
                *reinterpret_cast<u32x2*>(out8 + eP) = q;
            }
        } else {
            if (hpd == kHeads) {
                buf_st16(rout, e1, o);
            } else if (m < M) {
                st16(out8 + eP * 2, o);
            }
        }
    }
}

// kE4m3: out holds e4m3 codes (one byte per element) of the bf16 results divided by the
// descale of their kind (dq, dk, dv); else bf16 values (the descales are unused).
template <bool kE4m3>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void k_qkv_gemm(const uint16_t* __restrict__ ws, int64_t M, const uint16_t* __restrict__ W,
                const uint16_t* __restrict__ qw, const uint16_t* __restrict__ kw,
                const uint16_t* __restrict__ cs, int64_t S, const int64_t* __restrict__ pos, float qk_eps,
                int hpd, float dq, float dk, float dv, void* __restrict__ out, int mt, int nt) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
    int tm, tn;
    tile_coords(blockIdx.x, mt, nt, tm, tn);
    const int64_t m0 = (int64_t)tm * kBM;
    const int n0 = tn * kBN;
    Acc acc;
    mainloop<Mma::kBf16>(reinterpret_cast<const uint8_t*>(ws), kHidden * 2, m0, M, reinterpret_cast<const uint8_t*>(W),
                    kHidden * 2, n0, n0 + 128, kHidden * 2 / kRowB, smem, acc);
    qkv_epilogue<kE4m3>(acc, smem, m0, M, n0, qw, kw, cs, S, pos, qk_eps, hpd, dq, dk, dv, out);
}

// The same tile on MXFP4 operands: the workspace's and the weight's E2M1 codes ([M, 2688],
// [21504, 2688]) with their scales in the MX scale layout; bf16 output.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void k_qkv_gemm_mxfp4(const uint8_t* __restrict__ ws_codes, const uint8_t* __restrict__ ws_scales, uint32_t ws_sbytes,
                      int64_t M, const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales,
                      uint32_t w_sbytes, const uint16_t* __restrict__ qw, const uint16_t* __restrict__ kw,
                      const uint16_t* __restrict__ cs, int64_t S, const int64_t* __restrict__ pos, float qk_eps,
                      int hpd, void* __restrict__ out, int mt, int nt) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
    int tm, tn;
    tile_coords(blockIdx.x, mt, nt, tm, tn);
    const int64_t m0 = (int64_t)tm * kBM;
    const int n0 = tn * kBN;
    Acc acc;
    MxScales mxs;
    mxs.a = ws_scales;
    mxs.a_bytes = ws_sbytes;
    mxs.b = w_scales;
    mxs.b_bytes = w_sbytes;
    constexpr int kRowBytes = kHidden / 2;
    mainloop<Mma::kMxFp4>(ws_codes, kRowBytes, m0, M, w_codes, kRowBytes, n0, n0 + 128, kRowBytes / kRowB, smem, acc,
                          mxs);
    qkv_epilogue<false>(acc, smem, m0, M, n0, qw, kw, cs, S, pos, qk_eps, hpd, 1.0f, 1.0f, 1.0f, out);
}

hipError_t launch_qkv_gemm(const uint16_t* ws, int64_t M, const uint16_t* W, const uint16_t* qw,
                           const uint16_t* kw, const uint16_t* cs, int64_t S, const int64_t* pos, float qk_eps,
                           int P, uint16_t* out, hipStream_t stream) {
    const int mt = (int)((M + kBM - 1) / kBM);
    const int nt = kQkvRows / kBN;
    hipLaunchKernelGGL(k_qkv_gemm<false>, dim3((unsigned)(mt * nt)), dim3(kThreads), 0, stream, ws, M, W, qw, kw, cs,
                       S, pos, qk_eps, kHeads / P, 1.0f, 1.0f, 1.0f, out, mt, nt);
    return hipGetLastError();
}

hipError_t launch_qkv_gemm_mxfp4(const uint8_t* ws_codes, const uint8_t* ws_scales, int64_t M, const uint8_t* w_codes,
                                 const uint8_t* w_scales, const uint16_t* qw, const uint16_t* kw, const uint16_t* cs,
                                 int64_t S, const int64_t* pos, float qk_eps, int P, uint16_t* out,
                                 hipStream_t stream) {
    const int mt = (int)((M + kBM - 1) / kBM);
    const int nt = kQkvRows / kBN;
    const uint32_t a_sb = (uint32_t)mx_scale_bytes(M, kHidden);
    const uint32_t w_sb = (uint32_t)mx_scale_bytes(kQkvRows, kHidden);
    hipLaunchKernelGGL(k_qkv_gemm_mxfp4, dim3((unsigned)(mt * nt)), dim3(kThreads), 0, stream, ws_codes, ws_scales, a_sb,
                       M, w_codes, w_scales, w_sb, qw, kw, cs, S, pos, qk_eps, kHeads / P, out, mt, nt);
    return hipGetLastError();
}

hipError_t launch_qkv_gemm_e4m3(const uint16_t* ws, int64_t M, const uint16_t* W, const uint16_t* qw,
                                const uint16_t* kw, const uint16_t* cs, int64_t S, const int64_t* pos,
                                float qk_eps, int P, float dq, float dk, float dv, uint8_t* out, hipStream_t stream) {
    const int mt = (int)((M + kBM - 1) / kBM);
    const int nt = kQkvRows / kBN;
    hipLaunchKernelGGL(k_qkv_gemm<true>, dim3((unsigned)(mt * nt)), dim3(kThreads), 0, stream, ws, M, W, qw, kw, cs,
                       S, pos, qk_eps, kHeads / P, dq, dk, dv, out, mt, nt);
    return hipGetLastError();
}

}  // namespace dit
