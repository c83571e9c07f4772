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

}  // namespace gemm
}  // namespace dit
