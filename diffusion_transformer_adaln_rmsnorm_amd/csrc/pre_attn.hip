// QKV projection with the fused Q/K RMSNorm, RoPE and pack epilogue (launch 2 of the bf16
// pre-attention stage).
//
// FlashInfer "minimax_h3_bf16_pre_attention": description (GEMM streams the workspace, the
// epilogue applies the per-head Q/K RMSNorm, partial split-half NeoX RoPE and the
// destination-major pack) and Parameters (qkv_weight row order [q_all | k_all | v_all] x 56
// heads x 128, q/k_norm_weight [128], rope_cos_sin [S, 96] with cos in columns [0,48) and sin
// in [48,96), rope_positions clamped to [0, S) or the identity, out [1, M, 56, 3, 128]).
//
// A 256-wide n tile is exactly two heads of one kind (7168 = 28 x 256), so each tile owns
// whole heads and needs nothing from its neighbours.  After the main loop the tile is
// rounded to bf16 into LDS; then 16 consecutive lanes own one (row, head): 8 dims each, a
// 4-step xor reduction gives the head's sum of squares, and the RoPE partner of dims
// [8q, 8q+8) (q < 12) sits 6 lanes away (pairs (j, j+48)).  Each lane writes 16 contiguous
// bytes of out, so the 16 lanes of a head store its 256 bytes in one piece.
#include "common.hpp"
#include "gemm.hpp"
#include "kernels.hpp"

namespace dit {

using namespace gemm;

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void k_qkv_gemm(const uint16_t* __restrict__ ws, int64_t M, const uint16_t* __restrict__ W,
                const uint16_t* __restrict__ qw, const uint16_t* __restrict__ kw,
                const uint16_t* __restrict__ cs, int64_t S, const int64_t* __restrict__ pos, float qk_eps,
                uint16_t* __restrict__ out, int mt, int nt) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
    int tm, tn;
    tile_coords(blockIdx.x, mt, nt, tm, tn);
    const int64_t m0 = (int64_t)tm * kBM;
    const int n0 = tn * kBN;
    f32x16 acc[4][kNB];
    mainloop<false>(reinterpret_cast<const uint8_t*>(ws), kHidden * 2, m0, M, reinterpret_cast<const uint8_t*>(W),
                    kHidden * 2, n0, n0 + 128, kHidden * 2 / kRowB, smem, acc);
    stage_tile_bf16(acc, smem, nullptr, m0, M, nullptr, nullptr);
    __syncthreads();

    const int t = threadIdx.x;
    const int q = t & 15;               // 8-dim chunk of the head
    const int hh = (t >> 4) & 1;        // which of the tile's two heads
    const int rsub = t >> 5;            // 0..kThreads/32-1
    const int kind = n0 / kAttnWidth;   // 0 q, 1 k, 2 v
    const int head = (n0 % kAttnWidth) / kHeadDim + hh;
    const int d0 = q * 8;
    const int lane = t & 63;
    const int partner = (lane & ~15) | (q < 6 ? q + 6 : (q < 12 ? q - 6 : q));
    const int j0 = (q % 6) * 8;         // frequency index of this chunk (q < 12)

    float nw[8];
    if (kind < 2) {
        const u32x4 w = ld16((kind == 0 ? qw : kw) + d0);
        unpack8(w, nw);
    }

    // The cos/sin rows of iteration it + 1 (and the position of it + 2) are loaded while
    // iteration it computes, so the global-load latency is not paid once per row.
    constexpr int kRowsPerPass = kThreads / 32;
    constexpr int kIters = kBM / kRowsPerPass;
    const bool need_cs = kind < 2 && q < 12;
    auto row_pos = [&](int it) -> int64_t {
        const int64_t m = m0 + it * kRowsPerPass + rsub;
        if (it >= kIters || m >= M) return 0;
        const int64_t p = pos ? pos[m] : m;
        return p < 0 ? 0 : (p > S - 1 ? S - 1 : p);
    };
    u32x4 c_cur = {0u, 0u, 0u, 0u}, s_cur = {0u, 0u, 0u, 0u};
    int64_t p_nx = 0;
    if (need_cs) {
        const int64_t p0 = row_pos(0);
        c_cur = ld16(cs + p0 * kRopeCols + j0);
        s_cur = ld16(cs + p0 * kRopeCols + kNFreq + j0);
        p_nx = row_pos(1);
    }

    for (int it = 0; it < kIters; ++it) {
        const int row = it * kRowsPerPass + rsub;
        const int64_t m = m0 + row;
        u32x4 c_nx = {0u, 0u, 0u, 0u}, s_nx = {0u, 0u, 0u, 0u};
        int64_t p_nx2 = 0;
        if (need_cs && it + 1 < kIters) {
            c_nx = ld16(cs + p_nx * kRopeCols + j0);
            s_nx = ld16(cs + p_nx * kRopeCols + kNFreq + j0);
            p_nx2 = row_pos(it + 2);
        }
        float v[8];
        unpack8(epi_ld(smem, row, hh * 128 + d0), v);
        u32x4 o;
        if (kind < 2) {
            // per-head RMSNorm in fp32: bf16 squares are exact, the sum carries fp32 rounding
            // only, and u = bf16((v * r2) * w)
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
            ss += __shfl_xor(ss, 1);
            ss += __shfl_xor(ss, 2);
            ss += __shfl_xor(ss, 4);
            ss += __shfl_xor(ss, 8);
            const float r2 = rsqrtf(ss * (1.0f / kHeadDim) + qk_eps);
            float u[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) u[e] = rbf(v[e] * r2 * nw[e]);
            const u32x4 up = pack8(u);
            u32x4 pv;
#pragma unroll
            for (int e = 0; e < 4; ++e) pv[e] = (uint32_t)__shfl((int)up[e], partner);
            if (q < 12 && m < M) {
                float c[8], s[8], w2[8];
                unpack8(c_cur, c);
                unpack8(s_cur, s);
                unpack8(pv, w2);
                // bf16 x bf16 products are exact in fp32, so each fma is one rounding of
                // u c -/+ w s, then one rounding to bf16
                float r[8];
                if (q < 6) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) r[e] = rbf(fmaf(u[e], c[e], -(w2[e] * s[e])));
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) r[e] = rbf(fmaf(u[e], c[e], w2[e] * s[e]));
                }
                o = pack8(r);
            } else {
                o = up;
            }
        } else {
            o = pack8(v);
        }
        if (m < M) st16(out + ((m * kHeads + head) * 3 + kind) * kHeadDim + d0, o);
        c_cur = c_nx;
        s_cur = s_nx;
        p_nx = p_nx2;
    }
}

hipError_t launch_qkv_gemm(const uint16_t* ws, int64_t M, const uint16_t* W, const uint16_t* qw,
                           const uint16_t* kw, const uint16_t* cs, int64_t S, const int64_t* pos, float qk_eps,
                           uint16_t* out, hipStream_t stream) {
    const int mt = (int)((M + kBM - 1) / kBM);
    const int nt = kQkvRows / kBN;
    hipLaunchKernelGGL(k_qkv_gemm, dim3((unsigned)(mt * nt)), dim3(kThreads), 0, stream, ws, M, W, qw, kw, cs, S,
                       pos, qk_eps, out, mt, nt);
    return hipGetLastError();
}

}  // namespace dit
