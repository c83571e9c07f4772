// QKV projection with the fused Q/K RMSNorm, RoPE and pack epilogue for M <= 16 rows (launch 2
// of the bf16 pre-attention stage at small token counts).
//
// FlashInfer "minimax_h3_bf16_pre_attention": description and Parameters, as the 256 x 256 tile
// kernel (pre_attn.hip) computes them; this kernel serves the same entry points when M <= 16.
//
// At M <= 16 the GEMM is bound by streaming the 231 MB weight (16 flop per weight byte), and
// a 256-row tile would put the whole weight on 84 workgroups.  Here one workgroup owns one head
// of one kind (168 workgroups, 8 waves), and each wave owns 16 of the head's 128 weight rows
// (one 16-column block of the output) over the whole K:
//   - the wave copies its rows into its own ring of LDS slots with buffer_load ... lds, 128 K
//     values (256 contiguous bytes of each row) per stage and four stages ahead;
//   - the 16-byte chunks of a row are XOR-swizzled by the row (on the global side, since the 64
//     lanes of a fill write 1 KiB of LDS in lane order), so the MFMA operand reads of 16 rows
//     hit 16 distinct bank groups;
//   - the weight is read once, so its fills carry the non-temporal cache policy: with it, the
//     231 MB stream ran at 4.1 TB/s instead of 3.2 (a plain read of the same bytes with 16-row
//     blocks in this operand layout: 4.4 against 3.4 TB/s);
//   - the activation's operand (16 rows of the workspace, 172 KB, read by every wave) is loaded
//     from L2 straight into registers, cached.
// No wave reads another's rows, so the main loop has no barrier.  The 16 x 128 fp32 result goes
// through LDS to the same per-head Q/K RMSNorm, RoPE and pack code as the tile kernel's epilogue.
#include "common.hpp"
#include "gemm.hpp"
#include "kernels.hpp"
#include "qk_epi.hpp"

namespace dit {

using gemm::buf_ld16;
using gemm::buf_ld_i64;
using gemm::lds_barrier;
using gemm::lds_u8;
using gemm::make_rsrc;

constexpr int kSmWaves = 8;                       // 8 x 16 = the head's 128 weight rows
constexpr int kSmThreads = 64 * kSmWaves;
constexpr int kSmStageK = 128;                    // K values per stage (256 contiguous bytes of a row)
constexpr int kSmStages = kHidden / kSmStageK;
constexpr int kSmChunks = kSmStageK / 8;          // 16-byte chunks of a row per stage
constexpr int kSmSlot = 16 * kSmStageK * 2;       // one stage of a wave's 16 rows
constexpr int kSmAhead = 4;                       // stages in flight per wave
constexpr int kSmRing = kSmAhead + 1;             // slots per wave (one being read)
constexpr int kSmPieces = kSmSlot / 1024;         // 1 KiB fill loads per stage
constexpr int kSmSteps = kSmStageK / 32;          // MFMA k-steps per stage
constexpr int kSmLoads = kSmPieces + kSmSteps;    // loads per stage: fills, then A operands
static_assert(kHidden % kSmStageK == 0 && kSmStages > kSmAhead && kSmChunks % 16 == 0, "K stages");
static_assert(kSmLoads * kSmAhead < 64, "vmcnt range");
static_assert(kSmWaves * kSmRing * kSmSlot <= 160 * 1024, "LDS");

template <int N>
__device__ __forceinline__ void wait_vm() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__global__ __launch_bounds__(kSmThreads) void k_qkv_small(const uint16_t* __restrict__ ws, int64_t M,
                                                          const uint16_t* __restrict__ W,
                                                          const uint16_t* __restrict__ qw,
                                                          const uint16_t* __restrict__ kw,
                                                          const uint16_t* __restrict__ cs, int64_t S,
                                                          const int64_t* __restrict__ pos, float qk_eps, int hpd,
                                                          uint16_t* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kSmWaves * kSmRing * kSmSlot];
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int kind = blockIdx.x / kHeads, head = blockIdx.x % kHeads;
    const int n0 = kind * kAttnWidth + head * kHeadDim + 16 * wave;   // this wave's first weight row
    uint8_t* ring = lds + wave * kSmRing * kSmSlot;
    // A: the workspace (rows past M read as zeros); B: this wave's 16 weight rows
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(ws, (uint32_t)(M * kHidden * 2));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(W + (int64_t)n0 * kHidden, (uint32_t)(16 * kHidden * 2));
    // fill: the slot holds the stage's 16 rows one after the other, kSmChunks 16-byte chunks
    // each; lane i of piece q lands at slot chunk p = 64 q + i, i.e. row p / kSmChunks, position
    // p % kSmChunks, and loads the row's chunk (position) ^ (row % 16)
    uint32_t fill_off[kSmPieces];
#pragma unroll
    for (int q = 0; q < kSmPieces; ++q) {
        const int p = 64 * q + lane;
        const int r = p / kSmChunks, c = p % kSmChunks;
        fill_off[q] = (uint32_t)(r * kHidden * 2 + ((c ^ (r % 16)) << 4));
    }
    // MFMA operands, k-step s (32 values) of a stage: lane l supplies row (A) or column (B) l % 16
    // and k values 8 (l / 16) .. + 7, i.e. 16-byte chunk 4 s + l / 16 of the stage
    const int r = lane % 16, g = lane / 16;
    const uint32_t a_off = (uint32_t)(r * kHidden * 2 + g * 16);
    auto ra_at = [&](int st, int s) { return a_off + (uint32_t)(st * kSmStageK * 2 + s * 64); };
    auto rd_at = [&](int s) { return (uint32_t)(r * kSmStageK * 2 + (((4 * s + g) ^ r) << 4)); };
    static_assert(kSmAhead <= 4, "waits below");
    auto fill = [&](int st) {
        lds_u8* S = (lds_u8*)ring + (st % kSmRing) * kSmSlot;
#pragma unroll
        for (int q = 0; q < kSmPieces; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, S + q * 1024, 16, (int)fill_off[q], st * kSmStageK * 2, 0,
                                                     gemm::kCpolNt);
    };
    u32x4 aq[kSmRing][kSmSteps];     // A operands of the stages in flight, by stage % kSmRing
#pragma unroll
    for (int st = 0; st < kSmAhead; ++st) {
        fill(st);
#pragma unroll
        for (int s = 0; s < kSmSteps; ++s) aq[st][s] = buf_ld16(ra, ra_at(st, s));
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < kSmStages; ++st) {
        // the ring slot refilled next held stage st - 1, whose operand reads fed the MFMAs above
        asm volatile("" ::: "memory");
        if (st + kSmAhead < kSmStages) {
            fill(st + kSmAhead);
#pragma unroll
            for (int s = 0; s < kSmSteps; ++s)
                aq[(st + kSmAhead) % kSmRing][s] = buf_ld16(ra, ra_at(st + kSmAhead, s));
        }
        // stage st's fill and A operands have landed once at most the later stages' loads are
        // outstanding (kSmLoads per stage)
        const int later = kSmStages - 1 - st < kSmAhead ? kSmStages - 1 - st : kSmAhead;
        if (later >= 4) wait_vm<4 * kSmLoads>();
        else if (later == 3) wait_vm<3 * kSmLoads>();
        else if (later == 2) wait_vm<2 * kSmLoads>();
        else if (later == 1) wait_vm<kSmLoads>();
        else wait_vm<0>();
        asm volatile("" ::: "memory");   // the operand reads below stay after the wait
        const uint8_t* S = ring + (st % kSmRing) * kSmSlot;
#pragma unroll
        for (int s = 0; s < kSmSteps; ++s) {
            const u32x4 b = *reinterpret_cast<const u32x4*>(S + rd_at(s));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, aq[st % kSmRing][s]),
                                                          __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
        }
    }
    // every wave's result (16 x 16, lane l register v: row 4 (l / 16) + v, column l % 16) into
    // the first 8 KiB of LDS as a [16][128] fp32 tile, once every wave has finished its reads
    __syncthreads();
    float* res = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int v = 0; v < 4; ++v) res[(4 * g + v) * kHeadDim + 16 * wave + r] = acc[v];

    // epilogue: threads 0..255, the 16 lanes of a DPP row on one token row, 8 dims each
    const int row = t >> 4, li = t & 15;
    const int q = chunk_of_lane(li);
    const int d0 = q * 8;
    const int j0 = (q % 6) * 8;                     // frequency index of this chunk (q < 12)
    const bool epi = t < 16 * 16;
    const bool need_cs = epi && kind < 2 && q < 12;
    u32x4 csv = {0u, 0u, 0u, 0u}, nwv = csv;
    if (need_cs) {
        // position: clamp(pos[row], 0, S - 1), or the row (identity); rows past M read position 0
        const __amdgpu_buffer_rsrc_t rpos = make_rsrc(pos, pos ? (uint32_t)(M * 8) : 0u);
        const int64_t p = pos != nullptr ? buf_ld_i64(rpos, (uint32_t)(row * 8)) : (int64_t)row;
        const int64_t pc = p < 0 ? 0 : (p > S - 1 ? S - 1 : p);
        const __amdgpu_buffer_rsrc_t rcs = make_rsrc(cs, (uint32_t)(S * kRopeCols * 2));
        // this lane's half: the cos chunk (q < 6) or the sin chunk (6 <= q < 12)
        csv = buf_ld16(rcs, (uint32_t)((pc * kRopeCols + (q < 6 ? j0 : kNFreq + j0)) * 2));
    }
    if (epi && kind < 2) nwv = ld16((kind == 0 ? qw : kw) + d0);
    lds_barrier();
    if (!epi) return;
    float v[8];
    {
        const float* p = res + row * kHeadDim + d0;
        const f32x4 lo = *reinterpret_cast<const f32x4*>(p);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = lo[e];
            v[4 + e] = hi[e];
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
        o = qk_norm_rope(vp, nwlo, nwhi, qk_eps, q, csv);
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
