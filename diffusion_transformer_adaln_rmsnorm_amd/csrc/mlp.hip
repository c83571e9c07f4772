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
// SwiGLU pair of every column is in the same tile; its epilogue writes y straight from the
// accumulators.  The quantisation kernel then reads each row of y once, takes its maximum |y|
// for s_y and writes y_q; FC2 consumes y_q.  Stream order separates the three launches, so no
// tile-ready flags are needed.
#include "common.hpp"
#include "gated.hpp"
#include "gemm.hpp"
#include "kernels.hpp"

namespace dit {

using namespace gemm;

// FC1 epilogue straight from the accumulators.  With the B rows interleaved by 16 (gate rows
// j0 + 16 w + [0, 16) and up rows 14336 + j0 + 16 w + [0, 16) in B's local rows 32 w + [0, 32)),
// lane l of wave (wm, wn) holds in its column blocks 2 jb and 2 jb + 1 the gate and the up
// accumulators of the same y column j0 + 32 wn + 16 jb + l % 16, for its rows
// wm 128 + 16 i + 4 (l / 16) + r.  So h = bf16((acc * s_a) * w1s) and
// y = bf16(bf16(silu(h_gate)) * h_up), as printed, need no LDS staging.  Rows r, r + 1 of a
// column are one packed bf16 pair; lanes l and l ^ 1 swap halves with one DPP move, so each
// lane stores 4 bytes of one row (the staging's pairing).  No LDS and no barrier: G0 runs it
// while G1 finishes its last compute phase.
__device__ __forceinline__ void fc1_epilogue_regs(const Acc& acc, int64_t m0, int64_t M, int j0,
                                                  const float* __restrict__ a_scale, const float* __restrict__ w1s,
                                                  uint16_t* __restrict__ y) {
    const int t = opaque_tid();
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave / kWN, wn = wave % kWN;
    const int cl = lane % 16, rq = lane / 16;
    const int odd = lane & 1;
    const uint32_t sel = odd ? 0x03020706u : 0x05040100u;   // as in stage_tile_bf16
    const int64_t tile_rows = M - m0 < kBM ? M - m0 : kBM;
    // a_scale and y through descriptors over the tile's rows: rows past M read 0, stores dropped
    const __amdgpu_buffer_rsrc_t rrs = make_rsrc(a_scale + m0, (uint32_t)(tile_rows * 4));
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(y + m0 * kInter, (uint32_t)(tile_rows * kInter * 2));
    const int jc = j0 + 32 * wn + cl;               // this lane's y column in block pair 0 (+16: pair 1)
    float sg[2], su[2];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
        sg[jb] = w1s[jc + 16 * jb];
        su[jb] = w1s[kInter + jc + 16 * jb];
    }
#pragma unroll
    for (int i = 0; i < Acc::MB; ++i) {
        const int rb = wm * 128 + i * 16 + 4 * rq;  // this lane's rows rb .. rb + 3
        const u32x4 rsv = buf_ld16(rrs, (uint32_t)(rb * 4));
        float rs[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) rs[r] = __uint_as_float(rsv[r]);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const f32x4 g = acc.v[i][2 * jb], u = acc.v[i][2 * jb + 1];
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
                const uint32_t hg = pack_bf2((g[r] * rs[r]) * sg[jb], (g[r + 1] * rs[r + 1]) * sg[jb]);
                const uint32_t hu = pack_bf2((u[r] * rs[r]) * su[jb], (u[r + 1] * rs[r + 1]) * su[jb]);
                const uint32_t sl = pack_bf2(silu_fast(bf_lo(hg)), silu_fast(bf_hi(hg)));
                const uint32_t yv = pack_bf2(bf_lo(sl) * bf_lo(hu), bf_hi(sl) * bf_hi(hu));
                // quad_perm(1,0,3,2): lane l <- l ^ 1 (every lane active)
                const uint32_t nb = (uint32_t)__builtin_amdgcn_mov_dpp((int)yv, 0xB1, 0xF, 0xF, true);
                const int row = rb + r + odd, col = jc + 16 * jb - odd;
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_amdgcn_perm(nb, yv, sel), ry,
                                                      (int)((row * kInter + col) * 2), 0, 0);
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void k_fc1_swiglu(const uint8_t* __restrict__ a_q, const float* __restrict__ a_scale, int64_t M,
                  const uint8_t* __restrict__ W1, const float* __restrict__ w1s, uint16_t* __restrict__ y, int mt,
                  int nt, uint32_t* tq_ctr) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
    const TileQueue tq(tq_ctr, mt, nt);
    auto tile = [&](int k, TileOps& t, BRowsDefault&) {
        int tm, tn;
        logical_coords(tq.lo + k, mt, nt, tm, tn);
        const int j0 = tn * 128;
        t = TileOps{a_q, kHidden, (int64_t)tm * kBM, M, W1, kHidden, j0, kInter + j0, kHidden / kRowB};
    };
    auto epi = [&](const Acc& acc, const TileOps& t) { fc1_epilogue_regs(acc, t.m0, M, (int)t.nb0, a_scale, w1s, y); };
    persistent_tiles<Mma::kE4m3, true, true, Acc, BRowsDefault>(tq, smem, tile, epi);
}

// y quantisation: one wavefront per row; 14336 = 1792 chunks of 8, 28 per lane.  The row is
// read once into registers: its maximum |y| (on the bf16 bits, as in the MX quantiser), then
// s_y = RN(amax / 448) and the codes.
__global__ __launch_bounds__(256) void k_quant_rows(const uint16_t* __restrict__ y, int64_t M,
                                                    float* __restrict__ y_scale, uint8_t* __restrict__ y_q) {
    const int lane = threadIdx.x & 63;
    const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M) return;
    constexpr int kPerLane = kInter / 8 / 64;    // 28
    const uint16_t* yr = y + m * kInter;
    u32x4 yv[kPerLane];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) yv[j] = ld16(yr + (j * 64 + lane) * 8);
    uint32_t am = 0;
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) am = max(am, amax_bits8(yv[j]));
    const float amax = wave_max(__uint_as_float(am << 16));
    const float s = amax / 448.0f;            // RN(amax / 448)
    const float inv = 1.0f / s;               // RN(1 / s); unused when s == 0
    const bool s_normal = s >= 1.17549435e-38f;   // FLT_MIN
    uint8_t* qr = y_q + m * kInter;
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
        float a[8];
        unpack8(yv[j], a);
        uint2 q;
        if (s == 0.f) {
            q = make_uint2(0u, 0u);
        } else {
            q.x = f2e4m3x2(div_row(a[0], s, inv, s_normal), div_row(a[1], s, inv, s_normal)) |
                  (f2e4m3x2(div_row(a[2], s, inv, s_normal), div_row(a[3], s, inv, s_normal)) << 16);
            q.y = f2e4m3x2(div_row(a[4], s, inv, s_normal), div_row(a[5], s, inv, s_normal)) |
                  (f2e4m3x2(div_row(a[6], s, inv, s_normal), div_row(a[7], s, inv, s_normal)) << 16);
        }
        *reinterpret_cast<uint2*>(qr + (j * 64 + lane) * 8) = q;
    }
    if (lane == 0) y_scale[m] = s;
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void k_fc2_gated(const uint8_t* __restrict__ y_q, const float* __restrict__ y_scale, int64_t M,
                 const uint8_t* __restrict__ W2, const float* __restrict__ w2s, const uint16_t* __restrict__ gate,
                 int64_t gate_rows, int64_t gate_ld, const int64_t* __restrict__ idx, const uint16_t* residual,
                 uint16_t* out, int mt, int nt, uint32_t* tq_ctr) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
    const TileQueue tq(tq_ctr, mt, nt);
    auto tile = [&](int k, TileOps& t, Cols8BRows&) {
        int tm, tn;
        logical_coords(tq.lo + k, mt, nt, tm, tn);
        const int n0 = tn * kBN;
        t = TileOps{y_q, kInter, (int64_t)tm * kBM, M, W2, kInter, n0, n0 + 128, kInter / kRowB};
    };
    auto epi = [&](const AccW& acc, const TileOps& t) {
        gated_epilogue_regs<int64_t, true>(acc, t.m0, M, (int)t.nb0, y_scale, w2s, idx, gate, gate_rows, gate_ld,
                                           residual, out);
    };
    persistent_tiles<Mma::kE4m3, false, true, AccW, Cols8BRows>(tq, smem, tile, epi);
}

hipError_t launch_fc1_swiglu(const uint8_t* a_q, const float* a_scale, int64_t M, const uint8_t* W1,
                             const float* w1s, uint16_t* y, hipStream_t stream) {
    const int mt = (int)((M + kBM - 1) / kBM);
    const int nt = kInter / 128;
    uint32_t* q = nullptr;
    int grid = 0;
    const hipError_t e = tile_queue(stream, &q, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_fc1_swiglu, dim3((unsigned)grid), dim3(kThreads), 0, stream, a_q, a_scale, M, W1, w1s, y,
                       mt, nt, q);
    return hipGetLastError();
}

hipError_t launch_quant_rows(const uint16_t* y, int64_t M, float* y_scale, uint8_t* y_q, hipStream_t stream) {
    hipLaunchKernelGGL(k_quant_rows, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, stream, y, M, y_scale, y_q);
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
