// FP8 (W8A8) MLP block: FC1 + SwiGLU, per-token y quantisation, FC2 + gated residual.
//
// FlashInfer "minimax_h3_mlp_fp8_sm120", per-row formula block:
//   h = bf16(a_q @ fc1^T * s_a * fc1_scale)            FP32 accumulation, [M, 28672]
//   y = bf16(bf16(silu(h_gate)) * h_up)                 [M, 14336]
//   y_q = e4m3(y / s_y), s_y = RN(amax_row|y| / 448)
//   o = bf16(y_q @ fc2^T * s_y * fc2_scale)
//   out = bf16(residual + bf16(gate[i] * o)), gate 0 where i is outside [0, rows).
//
// FC1 tile: 256 rows x (128 gate columns j0.. and the 128 up columns 14336+j0..), so the
// SwiGLU pair of every column is in the same tile.  Its epilogue writes y and folds |y| into
// a per-row maximum with an atomic max on the float bits (|y| >= 0, so the unsigned order is
// the float order and the result does not depend on tile order).  The quantisation kernel then
// turns each row's maximum into s_y and writes y_q; FC2 consumes y_q.  Stream order separates
// the three launches, so no tile-ready flags are needed.
#include "common.hpp"
#include "gated.hpp"
#include "gemm.hpp"
#include "kernels.hpp"
#include "qk_epi.hpp"

namespace dit {

using namespace gemm;

// FC1 epilogue of one tile (rows m0.., gate columns j0.. and up columns kInter + j0..):
// h = bf16((acc * a_scale[row]) * w1s[col]) staged in LDS, then y = bf16(bf16(silu(h_gate)) *
// h_up) stored and the row maxima of |y| folded into y_amax.
__device__ __forceinline__ void fc1_epilogue(const Acc& acc, uint8_t* smem, int64_t m0, int64_t M, int j0,
                                             const float* __restrict__ a_scale, const float* __restrict__ w1s,
                                             uint16_t* __restrict__ y, float* __restrict__ y_amax) {
    stage_tile_bf16(acc, smem, a_scale, m0, M, w1s + j0, w1s + kInter + j0);
    lds_barrier();

    const int t = opaque_tid();
    const int c8 = (t & 15) * 8;
    const int rsub = t >> 4;            // 0..kThreads/16-1
    constexpr int kRowsPerPass = kThreads / 16;
    // y rows of this tile through a descriptor: stores of rows past M are dropped by its bound
    const int64_t tile_rows = M - m0 < kBM ? M - m0 : kBM;
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(y + m0 * kInter, (uint32_t)(tile_rows * kInter * 2));
    const uint32_t o1 = (uint32_t)((rsub * kInter + j0 + c8) * 2);
    constexpr uint32_t kPassB = (uint32_t)(kRowsPerPass * kInter * 2);
#pragma unroll
    for (int it = 0; it < kBM / kRowsPerPass; ++it) {
        const int row = it * kRowsPerPass + rsub;
        const u32x4 hg = epi_ld(smem, row, c8), hu = epi_ld(smem, row, 128 + c8);
        u32x4 yv;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            // two columns at a time: bf16(silu(h_gate)), then y = bf16(that * h_up)
            const uint32_t sl = pack_bf2(silu_fast(bf_lo(hg[k])), silu_fast(bf_hi(hg[k])));
            yv[k] = pack_bf2(bf_lo(sl) * bf_lo(hu[k]), bf_hi(sl) * bf_hi(hu[k]));
        }
        // max |y| of the row's 128 columns on the bf16 bits (the row's 16 lanes are one DPP
        // row); as float bits it is the FP32 value, whose unsigned order the atomic max keeps
        const uint32_t amax = row16_max_u32(amax_bits8(yv)) << 16;
        buf_st16(ry, o1 + it * kPassB, yv);
        if ((t & 15) == 0 && row < (int)tile_rows)
            atomicMax(reinterpret_cast<unsigned int*>(y_amax + m0 + row), amax);
    }
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void k_fc1_swiglu(const uint8_t* __restrict__ a_q, const float* __restrict__ a_scale, int64_t M,
                  const uint8_t* __restrict__ W1, const float* __restrict__ w1s, uint16_t* __restrict__ y,
                  float* __restrict__ y_amax, int mt, int nt, uint32_t* tq_ctr) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
    const TileQueue tq(tq_ctr, mt, nt);
    tq.claim(smem);
    __syncthreads();
    for (int k = tq.claimed(smem); k < tq.cnt; k = tq.claimed(smem)) {
        int tm, tn;
        logical_coords(tq.lo + k, mt, nt, tm, tn);
        const int64_t m0 = (int64_t)tm * kBM;
        const int j0 = tn * 128;
        Acc acc;
        mainloop<Mma::kE4m3>(a_q, kHidden, m0, M, W1, kHidden, j0, kInter + j0, kHidden / kRowB, smem, acc);
        tq.claim(smem);
        fc1_epilogue(acc, smem, m0, M, j0, a_scale, w1s, y, y_amax);
        __syncthreads();
    }
    tq.finish();
}

// y quantisation: one wavefront per row; 14336 = 1792 chunks of 8, 28 per lane.
__global__ __launch_bounds__(256) void k_quant_rows(const uint16_t* __restrict__ y, int64_t M,
                                                    float* __restrict__ y_scale, uint8_t* __restrict__ y_q) {
    const int lane = threadIdx.x & 63;
    const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M) return;
    const float amax = y_scale[m];
    const float s = amax / 448.0f;            // RN(amax / 448)
    const float inv = 1.0f / s;               // RN(1 / s); unused when s == 0
    const bool s_normal = s >= 1.17549435e-38f;   // FLT_MIN
    const uint16_t* yr = y + m * kInter;
    uint8_t* qr = y_q + m * kInter;
    constexpr int kPerLane = kInter / 8 / 64;    // 28
#pragma unroll 4
    for (int j = 0; j < kPerLane; ++j) {
        const int c = (j * 64 + lane) * 8;
        float a[8];
        unpack8(ld16(yr + c), a);
        uint2 q;
        if (s == 0.f) {
            q = make_uint2(0u, 0u);
        } else {
            q.x = f2e4m3x2(div_row(a[0], s, inv, s_normal), div_row(a[1], s, inv, s_normal)) |
                  (f2e4m3x2(div_row(a[2], s, inv, s_normal), div_row(a[3], s, inv, s_normal)) << 16);
            q.y = f2e4m3x2(div_row(a[4], s, inv, s_normal), div_row(a[5], s, inv, s_normal)) |
                  (f2e4m3x2(div_row(a[6], s, inv, s_normal), div_row(a[7], s, inv, s_normal)) << 16);
        }
        *reinterpret_cast<uint2*>(qr + c) = q;
    }
    // every lane has read y_scale[m] above; the store below follows a wave-wide barrier
    __builtin_amdgcn_wave_barrier();
    if (lane == 0) y_scale[m] = s;
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void k_fc2_gated(const uint8_t* __restrict__ y_q, const float* __restrict__ y_scale, int64_t M,
                 const uint8_t* __restrict__ W2, const float* __restrict__ w2s, const uint16_t* __restrict__ gate,
                 int64_t gate_rows, int64_t gate_ld, const int64_t* __restrict__ idx, const uint16_t* residual,
                 uint16_t* out, int mt, int nt, uint32_t* tq_ctr) {
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
        mainloop<Mma::kE4m3>(y_q, kInter, m0, M, W2, kInter, n0, n0 + 128, kInter / kRowB, smem, acc);
        tq.claim(smem);
        GatedResidual<int64_t> gr;
        gr.load_index(idx, m0, M, gate_rows);
        stage_tile_bf16(acc, smem, y_scale, m0, M, w2s + n0, w2s + n0 + 128);
        lds_barrier();
        gr.run(smem, m0, M, n0, gate, gate_rows, gate_ld, residual, out);
        __syncthreads();
    }
    tq.finish();
}

hipError_t launch_fc1_swiglu(const uint8_t* a_q, const float* a_scale, int64_t M, const uint8_t* W1,
                             const float* w1s, uint16_t* y, float* y_amax, hipStream_t stream) {
    const int mt = (int)((M + kBM - 1) / kBM);
    const int nt = kInter / 128;
    uint32_t* q = nullptr;
    int grid = 0;
    const hipError_t e = tile_queue(stream, &q, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_fc1_swiglu, dim3((unsigned)grid), dim3(kThreads), 0, stream, a_q, a_scale, M, W1, w1s, y,
                       y_amax, mt, nt, q);
    return hipGetLastError();
}

hipError_t launch_quant_rows(const uint16_t* y, int64_t M, float* y_scale_inout, uint8_t* y_q,
                             hipStream_t stream) {
    hipLaunchKernelGGL(k_quant_rows, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, stream, y, M, y_scale_inout, y_q);
    return hipGetLastError();
}

hipError_t launch_fc2_gated(const uint8_t* y_q, const float* y_scale, int64_t M, const uint8_t* W2,
                            const float* w2s, const uint16_t* gate, int64_t gate_rows, int64_t gate_ld,
                            const int64_t* idx, const uint16_t* residual, uint16_t* out, hipStream_t stream) {
    const int mt = (int)((M + kBM - 1) / kBM);
    const int nt = kHidden / kBN;
    uint32_t* q = nullptr;
    int grid = 0;
    const hipError_t e = tile_queue(stream, &q, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_fc2_gated, dim3((unsigned)grid), dim3(kThreads), 0, stream, y_q, y_scale, M, W2, w2s, gate,
                       gate_rows, gate_ld, idx, residual, out, mt, nt, q);
    return hipGetLastError();
}

}  // namespace dit
