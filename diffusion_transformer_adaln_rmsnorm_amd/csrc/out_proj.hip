// BF16 attention output projection with the fused gated residual.
//
// FlashInfer "minimax_h3_nvfp4_out_proj", description: the GEMM epilogue computes
// out = BF16(residual + BF16(gate[gate_index[m]] * o)) and rows whose gate_index lies outside
// [0, rows) get gate 0 (out = residual).  Here the operands are bf16 and o = bf16(acc), the
// rounding the fp8 MLP page prints for its own o.
//
// After the main loop the tile holds bf16(o) in LDS; each thread then owns 8 consecutive
// columns of a row: it reads the residual and the gate row with 16-byte loads, and writes
// out with one 16-byte store.  The residual is read before out is written by the same
// thread, so out may be the residual buffer.
#include "common.hpp"
#include "gemm.hpp"
#include "kernels.hpp"

namespace dit {

using namespace gemm;

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void k_out_proj_gemm(const uint16_t* __restrict__ attn, int64_t M, const uint16_t* __restrict__ Wo,
                     const uint16_t* __restrict__ gate, int64_t gate_rows, int64_t gate_ld,
                     const int32_t* __restrict__ gate_index, const uint16_t* residual, uint16_t* out, int mt,
                     int nt) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
    int tm, tn;
    tile_coords(blockIdx.x, mt, nt, tm, tn);
    const int64_t m0 = (int64_t)tm * kBM;
    const int n0 = tn * kBN;
    Acc acc;
    mainloop<false>(reinterpret_cast<const uint8_t*>(attn), kAttnWidth * 2, m0, M,
                    reinterpret_cast<const uint8_t*>(Wo), kAttnWidth * 2, n0, n0 + 128, kAttnWidth * 2 / kRowB, smem,
                    acc);
    stage_tile_bf16(acc, smem, nullptr, m0, M, nullptr, nullptr);
    __syncthreads();

    const int t = threadIdx.x;
    const int c8 = (t & 31) * 8;
    const int rsub = t >> 5;
    constexpr int kRowsPerPass = kThreads / 32;
    constexpr int kIters = kBM / kRowsPerPass;
    // The residual and gate chunks of row it + 1 (and the gate index of row it + 2) are loaded
    // while row it computes.  Rows grow with it, so the first row past M ends the loop.
    auto gate_of = [&](int it) -> int64_t {
        const int64_t m = m0 + it * kRowsPerPass + rsub;
        return it < kIters && m < M ? (int64_t)gate_index[m] : -1;
    };
    auto load_row = [&](int it, int64_t gi, u32x4& rr, u32x4& gg) {
        const int64_t m = m0 + it * kRowsPerPass + rsub;
        if (it < kIters && m < M) {
            rr = ld16(residual + m * kHidden + n0 + c8);
            if (gi >= 0 && gi < gate_rows) gg = ld16(gate + gi * gate_ld + n0 + c8);
        }
    };
    const u32x4 zero = {0u, 0u, 0u, 0u};
    u32x4 r_cur = zero, g_cur = zero;
    load_row(0, gate_of(0), r_cur, g_cur);
    int64_t gi_nx = gate_of(1);
#ifndef DIT_EPI_UNROLL
#define DIT_EPI_UNROLL 1
#endif
#pragma unroll DIT_EPI_UNROLL
    for (int it = 0; it < kIters; ++it) {
        const int row = it * kRowsPerPass + rsub;
        const int64_t m = m0 + row;
        if (m >= M) break;
        u32x4 r_nx = zero, g_nx = zero;
        load_row(it + 1, gi_nx, r_nx, g_nx);
        const int64_t gi_nx2 = gate_of(it + 2);
        float o[8], g[8], r[8];
        unpack8(epi_ld(smem, row, c8), o);
        unpack8(g_cur, g);
        unpack8(r_cur, r);
        // two bf16 values add exactly in fp32 (or the smaller is below half a bf16 ulp of the
        // larger), so this is one rounding of the exact sum
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = rbf(r[e] + rbf(g[e] * o[e]));
        st16(out + m * kHidden + n0 + c8, pack8(r));
        r_cur = r_nx;
        g_cur = g_nx;
        gi_nx = gi_nx2;
    }
}

hipError_t launch_out_proj_gemm(const uint16_t* attn, int64_t M, const uint16_t* Wo, const uint16_t* gate,
                                int64_t gate_rows, int64_t gate_ld, const int32_t* gate_index,
                                const uint16_t* residual, uint16_t* out, hipStream_t stream) {
    const int mt = (int)((M + kBM - 1) / kBM);
    const int nt = kHidden / kBN;
    hipLaunchKernelGGL(k_out_proj_gemm, dim3((unsigned)(mt * nt)), dim3(kThreads), 0, stream, attn, M, Wo, gate,
                       gate_rows, gate_ld, gate_index, residual, out, mt, nt);
    return hipGetLastError();
}

}  // namespace dit
