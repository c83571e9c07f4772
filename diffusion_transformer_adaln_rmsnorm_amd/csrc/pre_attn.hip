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
#include <type_traits>

#include "common.hpp"
#include "gemm.hpp"
#include "kernels.hpp"
#include "qk_epi.hpp"

namespace dit {

using namespace gemm;

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
template <bool kE4m3, class AccT>
__device__ __forceinline__ void qkv_epilogue(AccT& acc, uint8_t* smem, int64_t m0, int64_t M, int n0,
                                             const uint16_t* __restrict__ qw, const uint16_t* __restrict__ kw,
                                             const uint16_t* __restrict__ cs, int64_t S,
                                             const int64_t* __restrict__ pos, float qk_eps, int hpd, float dq,
                                             float dk, float dv, void* __restrict__ out) {
    const int t = opaque_tid();
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

    if constexpr (std::is_same_v<AccT, AccMx>) {
        stage_tile_bf16(acc, smem);
    } else {
        stage_tile_bf16(acc, smem, nullptr, m0, M, nullptr, nullptr);
    }
    // the cos/sin rows are requested once the accumulators are free and before the barrier, so
    // they are in flight while the other waves finish staging
    // this lane's half of the row's cos/sin: the cos chunk (q < 6) or the sin chunk (6 <= q < 12)
    const int cs_col = q < 6 ? j0 : kNFreq + j0;
    u32x4 csv[kIters];
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
        const int64_t m = m0 + it * kRowsPerPass + rsub;
        const int64_t p = pos != nullptr ? praw[it] : m;      // identity positions: the row
        const int64_t pc = p < 0 ? 0 : (p > S - 1 ? S - 1 : p);
        csv[it] = buf_ld16(rcs, need_cs ? (uint32_t)((pc * kRopeCols + cs_col) * 2) : kOffNone);
    }
    lds_barrier();

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
        if (kind < 2) o = qk_norm_rope(vp, nwlo, nwhi, qk_eps, q, csv[it]);
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
// Persistent: tiles are claimed from the queue tq (see TileQueue).
template <bool kE4m3>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void k_qkv_gemm(const uint16_t* __restrict__ ws, int64_t M, const uint16_t* __restrict__ W,
                const uint16_t* __restrict__ qw, const uint16_t* __restrict__ kw,
                const uint16_t* __restrict__ cs, int64_t S, const int64_t* __restrict__ pos, float qk_eps,
                int hpd, float dq, float dk, float dv, void* __restrict__ out, int mt, int nt, uint32_t* tq_ctr) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
    const TileQueue tq(tq_ctr, mt, nt);
    tq.claim(smem);
    __syncthreads();
    for (int k = tq.claimed(smem); k < tq.cnt; k = tq.claimed(smem)) {
        int tm, tn;
        logical_coords(tq.lo + k, mt, nt, tm, tn);
        const int64_t m0 = (int64_t)tm * kBM;
        const int n0 = tn * kBN;
        Acc acc;
        mainloop<Mma::kBf16>(reinterpret_cast<const uint8_t*>(ws), kHidden * 2, m0, M,
                             reinterpret_cast<const uint8_t*>(W), kHidden * 2, n0, n0 + 128, kHidden * 2 / kRowB,
                             smem, acc);
        tq.claim(smem);
        qkv_epilogue<kE4m3>(acc, smem, m0, M, n0, qw, kw, cs, S, pos, qk_eps, hpd, dq, dk, dv, out);
        __syncthreads();
    }
    tq.finish();
}

// The same tile on MXFP4 operands: the workspace's and the weight's E2M1 codes ([M, 2688],
// [21504, 2688]) with their scales in the MX scale layout; bf16 output.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void k_qkv_gemm_mxfp4(const uint8_t* __restrict__ ws_codes, const uint8_t* __restrict__ ws_scales, uint32_t ws_sbytes,
                      int64_t M, const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales,
                      uint32_t w_sbytes, const uint16_t* __restrict__ qw, const uint16_t* __restrict__ kw,
                      const uint16_t* __restrict__ cs, int64_t S, const int64_t* __restrict__ pos, float qk_eps,
                      int hpd, void* __restrict__ out, int mt, int nt, uint32_t* tq_ctr) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
    MxScales mxs;
    mxs.a = ws_scales;
    mxs.a_bytes = ws_sbytes;
    mxs.b = w_scales;
    mxs.b_bytes = w_sbytes;
    constexpr int kRowBytes = kHidden / 2;
    const TileQueue tq(tq_ctr, mt, nt);
    tq.claim(smem);
    __syncthreads();
    for (int k = tq.claimed(smem); k < tq.cnt; k = tq.claimed(smem)) {
        int tm, tn;
        logical_coords(tq.lo + k, mt, nt, tm, tn);
        const int64_t m0 = (int64_t)tm * kBM;
        const int n0 = tn * kBN;
        AccMx acc;
        mainloop<Mma::kMxFp4>(ws_codes, kRowBytes, m0, M, w_codes, kRowBytes, n0, n0 + 128, kRowBytes / kRowB, smem,
                              acc, mxs);
        tq.claim(smem);
        qkv_epilogue<false>(acc, smem, m0, M, n0, qw, kw, cs, S, pos, qk_eps, hpd, 1.0f, 1.0f, 1.0f, out);
        __syncthreads();
    }
    tq.finish();
}

hipError_t launch_qkv_gemm(const uint16_t* ws, int64_t M, const uint16_t* W, const uint16_t* qw,
                           const uint16_t* kw, const uint16_t* cs, int64_t S, const int64_t* pos, float qk_eps,
                           int P, uint16_t* out, hipStream_t stream) {
    // up to 16 rows the weight stream bounds the launch: spread it over one workgroup per head
    if (M <= 16) return launch_qkv_small(ws, M, W, qw, kw, cs, S, pos, qk_eps, P, out, stream);
    const int mt = (int)((M + kBM - 1) / kBM);
    const int nt = kQkvRows / kBN;
    uint32_t* q = nullptr;
    int grid = 0;
    const hipError_t e = tile_queue(stream, &q, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_qkv_gemm<false>, dim3((unsigned)grid), dim3(kThreads), 0, stream, ws, M, W, qw, kw, cs, S,
                       pos, qk_eps, kHeads / P, 1.0f, 1.0f, 1.0f, out, mt, nt, q);
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
    uint32_t* q = nullptr;
    int grid = 0;
    const hipError_t e = tile_queue(stream, &q, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_qkv_gemm_mxfp4, dim3((unsigned)grid), dim3(kThreads), 0, stream, ws_codes, ws_scales, a_sb, M,
                       w_codes, w_scales, w_sb, qw, kw, cs, S, pos, qk_eps, kHeads / P, out, mt, nt, q);
    return hipGetLastError();
}

hipError_t launch_qkv_gemm_e4m3(const uint16_t* ws, int64_t M, const uint16_t* W, const uint16_t* qw,
                                const uint16_t* kw, const uint16_t* cs, int64_t S, const int64_t* pos,
                                float qk_eps, int P, float dq, float dk, float dv, uint8_t* out, hipStream_t stream) {
    const int mt = (int)((M + kBM - 1) / kBM);
    const int nt = kQkvRows / kBN;
    uint32_t* q = nullptr;
    int grid = 0;
    const hipError_t e = tile_queue(stream, &q, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_qkv_gemm<true>, dim3((unsigned)grid), dim3(kThreads), 0, stream, ws, M, W, qw, kw, cs, S, pos,
                       qk_eps, kHeads / P, dq, dk, dv, out, mt, nt, q);
    return hipGetLastError();
}

}  // namespace dit
