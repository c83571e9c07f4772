// BF16 attention output projection with the fused gated residual.
//
// FlashInfer "minimax_h3_nvfp4_out_proj", description: the GEMM epilogue computes
// out = BF16(residual + BF16(gate[gate_index[m]] * o)) and rows whose gate_index lies outside
// [0, rows) get gate 0 (out = residual).  Here the operands are bf16 and o = bf16(acc), the
// rounding the fp8 MLP page prints for its own o.
//
// After the main loop the tile holds bf16(o) in LDS, and the gated-residual epilogue
// (gated.hpp) writes out; out may be the residual buffer.
#include "common.hpp"
#include "gated.hpp"
#include "gemm.hpp"
#include "kernels.hpp"

namespace dit {

using namespace gemm;

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void k_out_proj_gemm(const uint16_t* __restrict__ attn, int64_t M, const uint16_t* __restrict__ Wo,
                     const uint16_t* __restrict__ gate, int64_t gate_rows, int64_t gate_ld,
                     const int32_t* __restrict__ gate_index, const uint16_t* residual, uint16_t* out, int mt,
                     int nt, uint32_t* tq_ctr) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
    const TileQueue tq(tq_ctr, mt, nt);
    auto tile = [&](int k, TileOps& t, Cols8BRows&) {
        int tm, tn;
        logical_coords(tq.lo + k, mt, nt, tm, tn);
        const int n0 = tn * kBN;
        t = TileOps{reinterpret_cast<const uint8_t*>(attn), kAttnWidth * 2, (int64_t)tm * kBM, M,
                    reinterpret_cast<const uint8_t*>(Wo), kAttnWidth * 2, n0, n0 + 128, kAttnWidth * 2 / kRowB};
    };
    auto epi = [&](const AccW& acc, const TileOps& t) {
        gated_epilogue_regs<int32_t, false>(acc, t.m0, M, (int)t.nb0, nullptr, nullptr, gate_index, gate, gate_rows,
                                            gate_ld, residual, out);
    };
    persistent_tiles<Mma::kBf16, false, false, AccW, Cols8BRows>(tq, smem, tile, epi);
}

hipError_t launch_out_proj_gemm(const uint16_t* attn, int64_t M, const uint16_t* Wo, const uint16_t* gate,
                                int64_t gate_rows, int64_t gate_ld, const int32_t* gate_index,
                                const uint16_t* residual, uint16_t* out, hipStream_t stream) {
    const int mt = (int)((M + kBM - 1) / kBM);
    const int nt = kHidden / kBN;
    uint32_t* q = nullptr;
    int grid = 0;
    const hipError_t e = tile_queue(stream, &q, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_out_proj_gemm, dim3((unsigned)grid), dim3(kThreads), 0, stream, attn, M, Wo, gate, gate_rows,
                       gate_ld, gate_index, residual, out, mt, nt, q);
    return hipGetLastError();
}

}  // namespace dit
