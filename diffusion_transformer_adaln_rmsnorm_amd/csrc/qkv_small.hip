// QKV projection with the fused Q/K RMSNorm, RoPE and pack epilogue for M <= 16 rows (launch 2
// of the bf16 pre-attention stage at small token counts).
//
// FlashInfer "minimax_h3_bf16_pre_attention": description and Parameters, as the 256 x 256 tile
// kernel (pre_attn.hip) computes them; this kernel serves the same entry points when M <= 16.
//
// At M <= 16 the GEMM is bound by streaming the 231 MB weight (16 flop per weight byte), and
// a 256-row tile would put the whole weight on 84 workgroups.  Here one workgroup owns one head
// of one kind (168 workgroups): its 128 weight rows are split along K over 12 waves (448 values
// each, 14 k-steps of 32), which stream them from global memory straight into MFMA operand
// registers, three k-steps ahead (each weight element feeds exactly one MFMA lane, so nothing is
// staged in LDS).  The 16 x 128 fp32 partial sums of the 12 waves are added in LDS in a fixed
// order, rounded to bf16, and the head goes through the same per-head Q/K RMSNorm, RoPE and pack
// as the tile kernel's epilogue.
#include "common.hpp"
#include "gemm.hpp"
#include "kernels.hpp"
#include "qk_epi.hpp"

namespace dit {

using gemm::buf_ld16;
using gemm::buf_ld_i64;
using gemm::lds_barrier;
using gemm::make_rsrc;

constexpr int kSmallM = 16;
constexpr int kSmWaves = 12;
constexpr int kSmThreads = 64 * kSmWaves;
constexpr int kSmKPerWave = kHidden / kSmWaves;   // 448
constexpr int kSmSteps = kSmKPerWave / 32;        // 14 k-steps of 32 bf16
constexpr int kSmDepth = 3;                       // k-steps of operands in flight per wave
constexpr int kSmPitch = kHeadDim + 4;            // fp32 row pitch of the partial sums in LDS
static_assert(kSmKPerWave * kSmWaves == kHidden && kSmKPerWave % 32 == 0, "K split");

__global__ __launch_bounds__(kSmThreads) void k_qkv_small(const uint16_t* __restrict__ ws, int64_t M,
                                                          const uint16_t* __restrict__ W,
                                                          const uint16_t* __restrict__ qw,
                                                          const uint16_t* __restrict__ kw,
                                                          const uint16_t* __restrict__ cs, int64_t S,
                                                          const int64_t* __restrict__ pos, float qk_eps, int hpd,
                                                          uint16_t* __restrict__ out) {
    // partial sums of each wave: rows 16 x head dims 128 (row pitch padded: the 4 lane groups of a
    // write land 16 banks apart)
    __shared__ __attribute__((aligned(16))) float red[kSmWaves * kSmallM * kSmPitch];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int kind = blockIdx.x / kHeads, head = blockIdx.x % kHeads;
    const int n0 = kind * kAttnWidth + head * kHeadDim;
    // A: the workspace (rows past M read as zeros); B: the head's 128 weight rows
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(ws, (uint32_t)(M * kHidden * 2));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(W + (int64_t)n0 * kHidden, (uint32_t)(kHeadDim * kHidden * 2));
    // lane l supplies row (A) or column (B) l % 16 of a 16-block and k values 8 (l / 16) .. + 7 of
    // a k-step, the same (lane group, k) assignment for both operands
    const uint32_t koff = (uint32_t)((wave * kSmKPerWave + 8 * (lane >> 4)) * 2);
    const uint32_t a_off = (uint32_t)((lane & 15) * kHidden * 2) + koff;
    const uint32_t b_off = a_off;
    constexpr uint32_t kBlkB = 16 * kHidden * 2;      // bytes between 16-row weight blocks
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 aq[kSmDepth], bq[kSmDepth][8];
#pragma unroll
    for (int s = 0; s < kSmDepth; ++s) {
        aq[s] = buf_ld16(ra, a_off + s * 64);
#pragma unroll
        for (int j = 0; j < 8; ++j) bq[s][j] = buf_ld16(rb, b_off + j * kBlkB + s * 64);
    }
#pragma unroll
    for (int s = 0; s < kSmSteps; ++s) {
        const int slot = s % kSmDepth;
        const bf16x8 a = __builtin_bit_cast(bf16x8, aq[slot]);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, bq[slot][j]), acc[j], 0, 0,
                                                             0);
        if (s + kSmDepth < kSmSteps) {
            aq[slot] = buf_ld16(ra, a_off + (s + kSmDepth) * 64);
#pragma unroll
            for (int j = 0; j < 8; ++j) bq[slot][j] = buf_ld16(rb, b_off + j * kBlkB + (s + kSmDepth) * 64);
        }
    }
    // lane l, register r of block j: row 4 (l / 16) + r, head dim 16 j + l % 16
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            red[(wave * kSmallM + 4 * (lane >> 4) + r) * kSmPitch + 16 * j + (lane & 15)] = acc[j][r];

    // epilogue: threads 0..255, the 16 lanes of a DPP row on one token row, 8 dims each
    const int row = t >> 4, li = t & 15;
    const int q = chunk_of_lane(li);
    const int d0 = q * 8;
    const int j0 = (q % 6) * 8;                     // frequency index of this chunk (q < 12)
    const bool epi = t < kSmallM * 16;
    const bool need_cs = epi && kind < 2 && q < 12;
    u32x4 cv = {0u, 0u, 0u, 0u}, sv = cv, nwv = cv;
    if (need_cs) {
        // position: clamp(pos[row], 0, S - 1), or the row (identity); rows past M read position 0
        const __amdgpu_buffer_rsrc_t rpos = make_rsrc(pos, pos ? (uint32_t)(M * 8) : 0u);
        const int64_t p = pos != nullptr ? buf_ld_i64(rpos, (uint32_t)(row * 8)) : (int64_t)row;
        const int64_t pc = p < 0 ? 0 : (p > S - 1 ? S - 1 : p);
        const __amdgpu_buffer_rsrc_t rcs = make_rsrc(cs, (uint32_t)(S * kRopeCols * 2));
        const uint32_t off = (uint32_t)((pc * kRopeCols + j0) * 2);
        cv = buf_ld16(rcs, off);
        sv = buf_ld16(rcs, off + kNFreq * 2);
    }
    if (epi && kind < 2) nwv = ld16((kind == 0 ? qw : kw) + d0);
    lds_barrier();
    if (!epi) return;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
    // the 12 partial sums in wave order (a fixed order: the result is deterministic)
#pragma unroll
    for (int w = 0; w < kSmWaves; ++w) {
        const float* p = red + (w * kSmallM + row) * kSmPitch + d0;
        const f32x4 lo = *reinterpret_cast<const f32x4*>(p);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] += lo[e];
            v[4 + e] += hi[e];
        }
    }
    const u32x4 vp = pack8(v);                      // qkv = bf16(acc)
    u32x4 o = vp;
    if (kind < 2) {
        u32x4 nwlo, nwhi;                           // the norm weights, one bf16 of each pair kept
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            nwlo[e] = nwv[e] & 0xFFFFu;
            nwhi[e] = nwv[e] & 0xFFFF0000u;
        }
        o = qk_norm_rope(vp, nwlo, nwhi, qk_eps, q, cv, sv);
    }
    // destination-major pack: out[dst, m, hl, kind, d], destination dst holding heads
    // [dst hpd, (dst + 1) hpd)
    if (row < M) {
        const int dst = head / hpd, hl = head - dst * hpd;
        const int64_t e = ((((int64_t)dst * M + row) * hpd + hl) * 3 + kind) * kHeadDim + d0;
        st16(out + e, o);
    }
}

hipError_t launch_qkv_small(const uint16_t* ws, int64_t M, const uint16_t* W, const uint16_t* qw, const uint16_t* kw,
                            const uint16_t* cs, int64_t S, const int64_t* pos, float qk_eps, int P, uint16_t* out,
                            hipStream_t stream) {
    hipLaunchKernelGGL(k_qkv_small, dim3(3 * kHeads), dim3(kSmThreads), 0, stream, ws, M, W, qw, kw, cs, S, pos,
                       qk_eps, kHeads / P, out);
    return hipGetLastError();
}

}  // namespace dit
