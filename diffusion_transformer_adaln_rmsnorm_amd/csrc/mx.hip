// MXFP4 (OCP Microscaling) W4A4 out-projection: the gfx950-native counterpart of the NVFP4
// W4A4 out-projection.
//
// FlashInfer "minimax_h3_nvfp4_out_proj", description: the activation attn_out is quantised to
// 4-bit E2M1 with block scales, multiplied with the pre-quantised E2M1 weight by a block-scaled
// MMA, and the epilogue computes out = BF16(residual + BF16(gate[gate_index[m]] * o)).  That
// page's format is NVFP4 (block 16, UE4M3 scales and a global scale); gfx950's scaled MFMA takes
// OCP MXFP4: block 32 along K with one E8M0 (power-of-two) scale, so no global scale.
//  - k_mx_quant_fp4: one thread per 32-value block.  E = floor(log2(amax)) - 2 + 127 clamped to
//    [0, 254] (0 for an all-zero block), code = E2M1 nearest to v 2^(127 - E), ties to the even
//    significand, saturating at 6, the sign kept (mx.hpp: the hardware's scaled bf16 -> fp4
//    conversion).  Scales go to the MX scale layout (gemm.hpp); the scales of padding rows up to
//    the next multiple of 128 are written as 0.
//  - k_out_proj_mxfp4: the GEMM core on E2M1 codes (128 bytes = 256 values per stage), scales
//    through LDS, then bf16(o) staged and the shared gated-residual epilogue.
#include "common.hpp"
#include "gated.hpp"
#include "gemm.hpp"
#include "kernels.hpp"
#include "mx.hpp"

namespace dit {

using namespace gemm;

// x [R, K] bf16 rows (K % 256 == 0) -> codes [R, K / 2], scales in the MX scale layout for
// ceil(R / 128) * 128 rows.  Thread = (row, block of 32); rows R .. padded end write scale 0.
__global__ __launch_bounds__(256) void k_mx_quant_fp4(const uint16_t* __restrict__ x, int64_t R, int64_t K,
                                                      int64_t R_pad, uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales) {
    const int64_t nb = K / 32;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= R_pad * nb) return;
    const int64_t r = t / nb, b = t - r * nb;
    uint32_t E = 0;
    if (r < R) {
        const uint16_t* v = x + r * K + b * 32;
        u32x4 w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = ld16(v + 8 * q);
        uint32_t amax = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) amax = max(amax, amax_bits8(w[q]));
        E = mx_scale_byte(amax);
        u32x4 out;
#pragma unroll
        for (int q = 0; q < 4; ++q) out[q] = e2m1_pack8(w[q], E);
        st16(codes + r * (K / 2) + b * 16, out);
    }
    scales[mx_scale_offset(r, b, K)] = (uint8_t)E;
}

// out = bf16(residual + bf16(gate[gate_index[m]] * bf16(A . W))) with A, W MXFP4 (codes
// [M, 3584], [5376, 3584]; scales in the MX scale layout).  Tiles as the bf16 out-projection.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void k_out_proj_mxfp4(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, uint32_t a_sbytes,
                      int64_t M, const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales,
                      uint32_t w_sbytes, const uint16_t* __restrict__ gate, int64_t gate_rows, int64_t gate_ld,
                      const int32_t* __restrict__ gate_index, const uint16_t* residual, uint16_t* out, int mt,
                      int nt, uint32_t* tq_ctr) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
    MxScales mxs;
    mxs.a = a_scales;
    mxs.a_bytes = a_sbytes;
    mxs.b = w_scales;
    mxs.b_bytes = w_sbytes;
    constexpr int kRowBytes = kAttnWidth / 2;
    const TileQueue tq(tq_ctr, mt, nt);
    tq.claim(smem);
    __syncthreads();
    for (int k = tq.claimed(smem); k < tq.cnt; k = tq.claimed(smem)) {
        int tm, tn;
        logical_coords(tq.lo + k, mt, nt, tm, tn);
        const int64_t m0 = (int64_t)tm * kBM;
        const int n0 = tn * kBN;
        AccMx acc;
        mainloop<Mma::kMxFp4>(a_codes, kRowBytes, m0, M, w_codes, kRowBytes, n0, n0 + 128, kRowBytes / kRowB, smem,
                              acc, mxs);
        tq.claim(smem);
        GatedResidual<int32_t> gr;
        gr.load_index(gate_index, m0, M, gate_rows);
        gr.load_residual(m0, M, n0, residual);
        stage_tile_bf16(acc, smem);
        lds_barrier();
        gr.finish(smem, m0, M, n0, gate, gate_rows, gate_ld, out);
        __syncthreads();
    }
    tq.finish();
}

int64_t mx_scale_bytes(int64_t rows, int64_t K) { return (rows + 127) / 128 * 128 * (K / 32); }

hipError_t launch_mx_quant_fp4(const uint16_t* x, int64_t R, int64_t K, uint8_t* codes, uint8_t* scales,
                               hipStream_t stream) {
    const int64_t R_pad = (R + 127) / 128 * 128;
    const int64_t threads = R_pad * (K / 32);
    hipLaunchKernelGGL(k_mx_quant_fp4, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, x, R, K, R_pad,
                       codes, scales);
    return hipGetLastError();
}

hipError_t launch_out_proj_mxfp4(const uint8_t* a_codes, const uint8_t* a_scales, int64_t M, const uint8_t* w_codes,
                                 const uint8_t* w_scales, const uint16_t* gate, int64_t gate_rows, int64_t gate_ld,
                                 const int32_t* gate_index, const uint16_t* residual, uint16_t* out,
                                 hipStream_t stream) {
    const int mt = (int)((M + kBM - 1) / kBM);
    const int nt = kHidden / kBN;
    const uint32_t a_sb = (uint32_t)mx_scale_bytes(M, kAttnWidth);
    const uint32_t w_sb = (uint32_t)mx_scale_bytes(kHidden, kAttnWidth);
    uint32_t* q = nullptr;
    int grid = 0;
    const hipError_t e = tile_queue(stream, &q, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_out_proj_mxfp4, dim3((unsigned)grid), dim3(kThreads), 0, stream, a_codes, a_scales, a_sb, M,
                       w_codes, w_scales, w_sb, gate, gate_rows, gate_ld, gate_index, residual, out, mt, nt, q);
    return hipGetLastError();
}

}  // namespace dit
