// Gated-residual epilogue shared by the out-projection and FC2 kernels.
//
// FlashInfer "minimax_h3_nvfp4_out_proj", description, and "minimax_h3_mlp_fp8_sm120", the
// formula block's last line: out = BF16(residual + BF16(gate[index[m]] * o)), where o is the
// tile's bf16 GEMM output and rows whose index lies outside [0, gate rows) take gate 0
// (out = residual).
//
// Thread t owns 8 consecutive columns (c8 = (t % 32) * 8) of the tile rows it * 16 + t / 32,
// it = 0..15.  Residual and out are addressed through buffer descriptors over the tile's rows,
// so rows past M read zeros and their stores are dropped with no branch, and each row costs
// one 32-bit add of address arithmetic.  The row indices (load_index) and, where registers
// allow, the residual chunks (load_residual) are requested before the accumulators are staged,
// the gate chunks of all 16 rows right after, so a tile pays about one memory latency rather
// than one per row.  Each thread reads its residual chunk before it writes the same chunk of
// out, so out may be the residual buffer.
#pragma once

#include "gemm.hpp"

namespace dit {
namespace gemm {

template <typename Idx>
struct GatedResidual {
    static constexpr int kRowsPerPass = kThreads / 32;
    static constexpr int kIters = kBM / kRowsPerPass;
    static constexpr uint32_t kPassB = (uint32_t)(kRowsPerPass * kHidden * 2);
    int32_t gi[kIters];     // the gate row of each of this thread's rows, -1 for gate 0
    u32x4 rr[kIters];       // the residual chunks of this thread's rows

    // index[m] of this thread's rows, checked against [0, gate_rows) at full width and kept
    // as a 32-bit row or -1 (rows past M read index 0: their stores are dropped)
    __device__ __forceinline__ void load_index(const Idx* index, int64_t m0, int64_t M, int64_t gate_rows) {
        const int rsub = opaque_tid() >> 5;
        const int64_t tile_rows = M - m0 < kBM ? M - m0 : kBM;
        const __amdgpu_buffer_rsrc_t ri = make_rsrc(index + m0, (uint32_t)(tile_rows * sizeof(Idx)));
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const uint32_t off = (uint32_t)((it * kRowsPerPass + rsub) * sizeof(Idx));
            int64_t i;
            if constexpr (sizeof(Idx) == 8) {
                i = buf_ld_i64(ri, off);
            } else {
                i = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(ri, (int)off, 0, 0);
            }
            gi[it] = (i >= 0 && i < gate_rows) ? (int32_t)i : -1;
        }
    }

    // the residual chunks of all rows (the out-projections request them before the accumulators
    // are staged, so their latency hides behind the staging; FC2's row and column scales leave
    // no registers for that, and it requests them after)
    __device__ __forceinline__ void load_residual(int64_t m0, int64_t M, int n0, const uint16_t* residual) {
        const int t = opaque_tid();
        const int64_t tile_rows = M - m0 < kBM ? M - m0 : kBM;
        const __amdgpu_buffer_rsrc_t rres = make_rsrc(residual + m0 * kHidden, (uint32_t)(tile_rows * kHidden * 2));
        const uint32_t o1 = (uint32_t)(((t >> 5) * kHidden + n0 + (t & 31) * 8) * 2);
#pragma unroll
        for (int it = 0; it < kIters; ++it) rr[it] = buf_ld16(rres, o1 + it * kPassB);
    }

    // After the bf16 tile is staged in LDS (and a barrier): the residual chunks, then finish().
    __device__ __forceinline__ void run(const uint8_t* smem, int64_t m0, int64_t M, int n0, const uint16_t* gate,
                                        int64_t gate_rows, int64_t gate_ld, const uint16_t* residual, uint16_t* out) {
        load_residual(m0, M, n0, residual);
        finish(smem, m0, M, n0, gate, gate_rows, gate_ld, out);
    }

    // With the residual chunks requested: out = bf16(r + bf16(g * o)).
    __device__ __forceinline__ void finish(const uint8_t* smem, int64_t m0, int64_t M, int n0, const uint16_t* gate,
                                           int64_t gate_rows, int64_t gate_ld, uint16_t* out) const {
        const int t = opaque_tid();
        const int c8 = (t & 31) * 8;
        const int rsub = t >> 5;
        const int64_t tile_rows = M - m0 < kBM ? M - m0 : kBM;
        const uint32_t bytes = (uint32_t)(tile_rows * kHidden * 2);
        const __amdgpu_buffer_rsrc_t rout = make_rsrc(out + m0 * kHidden, bytes);
        const uint32_t o1 = (uint32_t)((rsub * kHidden + n0 + c8) * 2);
        const u32x4 zero = {0u, 0u, 0u, 0u};
        u32x4 gg[kIters];
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            gg[it] = zero;
            if (gi[it] >= 0) gg[it] = ld16(gate + (int64_t)gi[it] * gate_ld + n0 + c8);
        }
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const u32x4 ov = epi_ld(smem, it * kRowsPerPass + rsub, c8);
            u32x4 res;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                // g o rounded to bf16 (two at a time), then r + that in FP32: two bf16 values add
                // exactly in FP32 (or the smaller is below half a bf16 ulp of the larger), so
                // the RNE to bf16 is one rounding of the exact sum
                const uint32_t go = pack_bf2(bf_lo(gg[it][k]) * bf_lo(ov[k]), bf_hi(gg[it][k]) * bf_hi(ov[k]));
                res[k] = pack_bf2(bf_lo(rr[it][k]) + bf_lo(go), bf_hi(rr[it][k]) + bf_hi(go));
            }
            buf_st16(rout, o1 + it * kPassB, res);
        }
    }
};

// The same gated residual straight from the accumulators: 64 x 128 wave tiles (AccW) with the
// B rows in Cols8BRows order, so wave (wm, h) holds rows 64 wm + 16 i + 4 (l / 16) + r
// (i, r < 4) of the tile and, for each, the 8 columns n0 + 128 h + 8 (l % 16) .. + 7 (block j:
// column + j).  kScaled: o = bf16((acc s_row) s_col) with the row scales rowscale[m] and the
// column scales colscale[n] (FC2), else o = bf16(acc).  Then out = bf16(r + bf16(g o)) with
// the staged epilogue's arithmetic, 16 bytes per row and lane for r, g and out.  The 16 lanes of
// a DPP row share their 16 rows: lane l % 16 = c loads the index of row (c / 4, c % 4) and hands
// the checked gate row to the others (ds_bpermute).  No LDS and no barrier, so G0 can run it
// while G1 finishes its last compute phase.  Each lane reads its residual chunk before it
// writes the same chunk of out, so out may be the residual buffer.
template <typename Idx, bool kScaled>
__device__ __forceinline__ void gated_epilogue_regs(const AccW& acc, int64_t m0, int64_t M, int n0,
                                                    const float* __restrict__ rowscale,
                                                    const float* __restrict__ colscale, const Idx* __restrict__ index,
                                                    const uint16_t* __restrict__ gate, int64_t gate_rows,
                                                    int64_t gate_ld, const uint16_t* residual, uint16_t* out) {
    const int t = opaque_tid();
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave / AccW::kWavesN, h = wave % AccW::kWavesN;
    const int c = lane & 15, rq = lane >> 4;
    const int rbase = wm * AccW::kRows + 4 * rq;          // + 16 i + r: this lane's rows
    const int col0 = n0 + 128 * h + 8 * c;                // this lane's 8 columns
    const int64_t tile_rows = M - m0 < kBM ? M - m0 : kBM;
    // residual, out and the row indices through descriptors over the tile's rows: rows past M
    // read zeros (index 0) and their stores are dropped
    const uint32_t bytes = (uint32_t)(tile_rows * kHidden * 2);
    const __amdgpu_buffer_rsrc_t rres = make_rsrc(residual + m0 * kHidden, bytes);
    const __amdgpu_buffer_rsrc_t rout = make_rsrc(out + m0 * kHidden, bytes);
    const uint32_t vo = (uint32_t)((rbase * kHidden + col0) * 2);   // row (i, r) adds (16 i + r) kHidden 2
    int32_t gi_own;
    {
        const __amdgpu_buffer_rsrc_t ri = make_rsrc(index + m0, (uint32_t)(tile_rows * sizeof(Idx)));
        const uint32_t off = (uint32_t)((rbase + 16 * (c >> 2) + (c & 3)) * sizeof(Idx));
        int64_t iv;
        if constexpr (sizeof(Idx) == 8) {
            iv = buf_ld_i64(ri, off);
        } else {
            iv = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(ri, (int)off, 0, 0);
        }
        gi_own = (iv >= 0 && iv < gate_rows) ? (int32_t)iv : -1;
    }
    // one 4-row block's residual and gate chunks (requested a block ahead)
    auto load_block = [&](int i, u32x4 (&rr)[4], u32x4 (&gg)[4]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            rr[r] = buf_ld16(rres, vo + (uint32_t)((16 * i + r) * kHidden * 2));
            const int gi = __builtin_amdgcn_ds_bpermute(4 * (16 * rq + 4 * i + r), gi_own);
            gg[r] = u32x4{0u, 0u, 0u, 0u};
            if (gi >= 0) gg[r] = ld16(gate + (int64_t)gi * gate_ld + col0);
        }
    };
    u32x4 rr_nx[4], gg_nx[4];
    load_block(0, rr_nx, gg_nx);
    // o as bf16, packed: op[i][r][k] = columns 2 k, 2 k + 1 of row (i, r)
    u32x4 op[AccW::MB][4];
    if constexpr (kScaled) {
        float cs[8];    // (the column scales need only 4-byte alignment: one load each)
#pragma unroll
        for (int e = 0; e < 8; ++e) cs[e] = colscale[col0 + e];
        const __amdgpu_buffer_rsrc_t rrs = make_rsrc(rowscale + m0, (uint32_t)(tile_rows * 4));
#pragma unroll
        for (int i = 0; i < AccW::MB; ++i) {
            const u32x4 rsv = buf_ld16(rrs, (uint32_t)((rbase + 16 * i) * 4));
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float rs = __uint_as_float(rsv[r]);
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    op[i][r][k] = pack_bf2((acc.v[i][2 * k][r] * rs) * cs[2 * k],
                                           (acc.v[i][2 * k + 1][r] * rs) * cs[2 * k + 1]);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < AccW::MB; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int k = 0; k < 4; ++k) op[i][r][k] = pack_bf2(acc.v[i][2 * k][r], acc.v[i][2 * k + 1][r]);
    }
#pragma unroll
    for (int i = 0; i < AccW::MB; ++i) {
        u32x4 rr[4], gg[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            rr[r] = rr_nx[r];
            gg[r] = gg_nx[r];
        }
        if (i + 1 < AccW::MB) load_block(i + 1, rr_nx, gg_nx);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            u32x4 res;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                // as in finish(): g o rounded to bf16, then r + that, one rounding of the exact sum
                const uint32_t ov = op[i][r][k];
                const uint32_t go = pack_bf2(bf_lo(gg[r][k]) * bf_lo(ov), bf_hi(gg[r][k]) * bf_hi(ov));
                res[k] = pack_bf2(bf_lo(rr[r][k]) + bf_lo(go), bf_hi(rr[r][k]) + bf_hi(go));
            }
            buf_st16(rout, vo + (uint32_t)((16 * i + r) * kHidden * 2), res);
        }
    }
}

}  // namespace gemm
}  // namespace dit
