// Row RMSNorm + indexed AdaLN kernels (launch 1 of the bf16 pre-attention stage, kernel A of
// the fp8 MLP block).
//
// FlashInfer "minimax_h3_mlp_fp8_sm120", per-row formula block (its first three lines and the
// per-token activation scale), applied to the pre-attention stage as the
// "minimax_h3_bf16_pre_attention" description orders it (norm, AdaLN, then the workspace the
// QKV GEMM streams).  The adaln_index entry of that page fixes the guard: any int64 outside
// [0, rows) zeroes the row and the tables are never addressed with it.
//
// Mapping: one 64-lane wavefront per row, four rows per 256-thread workgroup.  A 5376-wide
// row is 672 chunks of 8 bf16 (16 bytes); lane l owns chunks l, l+64, ... (11 for lanes
// 0..31, 10 for lanes 32..63), so every load and store is a coalesced 16-byte access and the
// row stays in registers between the sum of squares and the modulation.  HBM-bound: per row
// it reads x (10.5 KiB) and writes the workspace (10.5 KiB, or 5.25 KiB of e4m3 codes); the
// norm weight and the few table rows stay in L2.
#include "common.hpp"
#include "kernels.hpp"
#include "mx.hpp"

namespace dit {

namespace {

constexpr int kChunks = kHidden / 8;          // 672
constexpr int kMaxPerLane = (kChunks + 63) / 64;  // 11

__device__ __forceinline__ bool chunk_ok(int j, int lane) { return j * 64 + lane < kChunks; }

// The row's loads, issued in two groups so that every load not waiting on the index is in
// flight before the guard: at small M each row is a chain of memory latencies (index -> table
// rows), not a stream.  x is read once, so its loads are non-temporal and keep it from
// displacing the tables and the workspace in the caches (10% faster on a cold M = 32760 pass).
// The norm weight, the same for every row, is staged once per workgroup in LDS (stage_weight)
// and read from there chunk by chunk: held in registers beside the row's x, scale and shift it
// took 44 more of them and kept the kernels at 2 waves per SIMD (3 now: bf16 norm -8%).
struct RowRegs {
    u32x4 x[kMaxPerLane], sc[kMaxPerLane], sh[kMaxPerLane];
};

__device__ __forceinline__ void stage_weight(const uint16_t* xw, u32x4* wl) {
    for (int c = threadIdx.x; c < kChunks; c += 256) wl[c] = ld16(xw + c * 8);
}

__device__ __forceinline__ void load_x(const uint16_t* xr, int lane, RowRegs& rg) {
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j)
        if (chunk_ok(j, lane)) rg.x[j] = ld16_nt(xr + (j * 64 + lane) * 8);
}

__device__ __forceinline__ void load_tables(const uint16_t* scr, const uint16_t* shr, int lane, RowRegs& rg) {
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
        if (chunk_ok(j, lane)) {
            rg.sc[j] = ld16(scr + (j * 64 + lane) * 8);
            rg.sh[j] = ld16(shr + (j * 64 + lane) * 8);
        }
    }
}

// r = 1 / sqrt(mean(x^2) + eps) of the row held in registers: an FP32 sum, two squares (exact
// bf16 products) per v_dot2 on the packed values
__device__ __forceinline__ float row_rms(const RowRegs& rg, int lane, float eps) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
        if (chunk_ok(j, lane)) {
#pragma unroll
            for (int e = 0; e < 4; ++e) ss = dot2_bf16(rg.x[j][e], rg.x[j][e], ss);
        }
    }
    ss = wave_sum(ss);
    return 1.0f / sqrtf(ss / (float)kHidden + eps);
}

// a = bf16(shift + n * bf16(1 + scale)),  n = bf16((x * r) * w), for one 8-wide chunk, in FP32
// in the formula block's order: x * r and its product with w each rounded to FP32, then RNE to
// bf16.  1 + scale is exact in FP32 unless |scale| < 2^-16, where every rounding of it gives the
// bf16 1 (one_plus_x8 takes it on the packed scale).  n * bf16(1 + scale) is a product of two
// bf16 values, exact in FP32, so the fma rounds shift + n s1 once to FP32 before the RNE to bf16.
// r is the FP32 reciprocal root.
__device__ __forceinline__ void modulate_chunk(const u32x4& xv, const u32x4& wv, const u32x4& scv,
                                               const u32x4& shv, float r, uint32_t (&out)[4]) {
    float x[8], w[8], sc1[8], sh[8];
    unpack8(xv, x);
    unpack8(wv, w);
    one_plus_x8(scv[0], scv[1], scv[2], scv[3], sc1);
    unpack8(shv, sh);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        // two elements per packed bf16 conversion
        const uint32_t n = pack_bf2((x[2 * k] * r) * w[2 * k], (x[2 * k + 1] * r) * w[2 * k + 1]);
        const uint32_t s1 = pack_bf2(sc1[2 * k], sc1[2 * k + 1]);
        out[k] = pack_bf2(fmaf(bf_lo(n), bf_lo(s1), sh[2 * k]), fmaf(bf_hi(n), bf_hi(s1), sh[2 * k + 1]));
    }
}

}  // namespace

__global__ __launch_bounds__(256) void k_norm_adaln_bf16(const uint16_t* __restrict__ x, int64_t M,
                                                         const uint16_t* __restrict__ xw,
                                                         const uint16_t* __restrict__ scale, int64_t ld_scale,
                                                         const uint16_t* __restrict__ shift, int64_t ld_shift,
                                                         int64_t rows, const int64_t* __restrict__ idx,
                                                         float eps, uint16_t* __restrict__ ws) {
    __shared__ __attribute__((aligned(16))) u32x4 wl[kChunks];
    const int lane = threadIdx.x & 63;
    const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const bool live = m < M;
    stage_weight(xw, wl);
    const int64_t i = live ? idx[m] : -1;
    const bool ok = i >= 0 && i < rows;        // full-width int64 guard
    RowRegs rg;
    if (live) load_x(x + m * kHidden, lane, rg);
    if (ok) load_tables(scale + i * ld_scale, shift + i * ld_shift, lane, rg);
    __syncthreads();                           // the weight staged (every wave, before any exit)
    if (!live) return;
    uint16_t* wr = ws + m * kHidden;
    if (!ok) {
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < kMaxPerLane; ++j)
            if (chunk_ok(j, lane)) st16(wr + (j * 64 + lane) * 8, z);
        return;
    }
    const float r = row_rms(rg, lane, eps);
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
        if (!chunk_ok(j, lane)) continue;
        uint32_t a[4];
        modulate_chunk(rg.x[j], wl[j * 64 + lane], rg.sc[j], rg.sh[j], r, a);
        st16(wr + (j * 64 + lane) * 8, u32x4{a[0], a[1], a[2], a[3]});
    }
}

// MXFP4 pre-attention, launch 1: the same row steps, then a quantised to MXFP4 in registers
// instead of written as bf16.  The 32-value block of chunks 4c .. 4c + 3 belongs to the four
// lanes of one quad (a lane's chunks are 64 apart), so the block maximum is two DPP steps.
// Codes [M, 2688] (4 bytes per lane and chunk); scales in the MX scale layout for R_pad rows
// (rows M .. R_pad write only their zero scales).  Guarded rows quantise a = 0: codes 0, scale 0.
__global__ __launch_bounds__(256) void k_norm_adaln_mxfp4(const uint16_t* __restrict__ x, int64_t M,
                                                          const uint16_t* __restrict__ xw,
                                                          const uint16_t* __restrict__ scale, int64_t ld_scale,
                                                          const uint16_t* __restrict__ shift, int64_t ld_shift,
                                                          int64_t rows, const int64_t* __restrict__ idx, float eps,
                                                          int64_t R_pad, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
    __shared__ __attribute__((aligned(16))) u32x4 wl[kChunks];
    const int lane = threadIdx.x & 63;
    const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    stage_weight(xw, wl);
    const bool live = m < M;
    const int64_t i = live ? idx[m] : -1;
    const bool ok = i >= 0 && i < rows;               // full-width int64 guard
    RowRegs rg;
    if (live) load_x(x + m * kHidden, lane, rg);
    if (ok) load_tables(scale + i * ld_scale, shift + i * ld_shift, lane, rg);
    __syncthreads();                                  // the weight staged (every wave, before any exit)
    if (m >= R_pad) return;
    // scale byte of chunk j's block (b = 16 j + lane / 4) in the MX scale layout: a per-row and a
    // per-lane part plus j * 2048 (b / 8 = 2 j + lane / 32, while b % 2 and (b % 8) / 2 depend on
    // the lane only), mx_scale_offset taken apart for this row length
    static_assert(kHidden % 256 == 0, "whole 256-column scale stages");
    const int64_t rr = m % 128;
    uint8_t* const srow = scales + (m / 128) * (kHidden / 256) * 1024 + 16 * (rr % 32) + 4 * (rr / 32) +
                          (lane / 32) * 1024 + 512 * ((lane / 4) % 2) + (lane / 8) % 4;
    if (!live) {
#pragma unroll
        for (int j = 0; j < kMaxPerLane; ++j)
            if (chunk_ok(j, lane) && (lane & 3) == 0) srow[j * 2048] = 0;
        return;
    }
    // each chunk is quantised as soon as it is modulated (its 32-value block is one quad's
    // chunks), so the modulated row is never held whole; guarded rows quantise a = 0
    const float r = ok ? row_rms(rg, lane, eps) : 0.f;
    uint8_t* cr = codes + m * (kHidden / 2);
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
        if (!chunk_ok(j, lane)) continue;             // whole quads drop out together
        u32x4 av = {0u, 0u, 0u, 0u};
        if (ok) {
            uint32_t a[4];
            modulate_chunk(rg.x[j], wl[j * 64 + lane], rg.sc[j], rg.sh[j], r, a);
            av = u32x4{a[0], a[1], a[2], a[3]};
        }
        uint32_t amax = amax_bits8(av);
        // quad_perm(1,0,3,2) then (2,3,0,1): the maximum over the block's four lanes
        amax = max(amax, (uint32_t)__builtin_amdgcn_mov_dpp((int)amax, 0xB1, 0xF, 0xF, true));
        amax = max(amax, (uint32_t)__builtin_amdgcn_mov_dpp((int)amax, 0x4E, 0xF, 0xF, true));
        const uint32_t E = mx_scale_byte(amax);
        *reinterpret_cast<uint32_t*>(cr + (j * 64 + lane) * 4) = e2m1_pack8(av, E);
        if ((lane & 3) == 0) srow[j * 2048] = (uint8_t)E;
    }
}

// MLP kernel A: the same row steps, then s_a = RN(amax|a| / 448) and a_q = e4m3(a / s_a).
__global__ __launch_bounds__(256) void k_norm_adaln_fp8q(const uint16_t* __restrict__ x, int64_t M,
                                                         const uint16_t* __restrict__ xw,
                                                         const uint16_t* __restrict__ scale, int64_t ld_scale,
                                                         const uint16_t* __restrict__ shift, int64_t ld_shift,
                                                         int64_t rows, const int64_t* __restrict__ idx,
                                                         float eps, uint8_t* __restrict__ a_q,
                                                         float* __restrict__ a_scale) {
    __shared__ __attribute__((aligned(16))) u32x4 wl[kChunks];
    const int lane = threadIdx.x & 63;
    const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const bool live = m < M;
    stage_weight(xw, wl);
    const int64_t i = live ? idx[m] : -1;
    const bool ok = i >= 0 && i < rows;        // full-width int64 guard
    RowRegs rg;
    if (live) load_x(x + m * kHidden, lane, rg);
    if (ok) load_tables(scale + i * ld_scale, shift + i * ld_shift, lane, rg);
    __syncthreads();                           // the weight staged (every wave, before any exit)
    if (!live) return;
    uint8_t* qr = a_q + m * kHidden;
    if (!ok) {
        const uint2 z = {0u, 0u};
#pragma unroll
        for (int j = 0; j < kMaxPerLane; ++j)
            if (chunk_ok(j, lane)) *reinterpret_cast<uint2*>(qr + (j * 64 + lane) * 8) = z;
        if (lane == 0) a_scale[m] = 0.f;
        return;
    }
    const float r = row_rms(rg, lane, eps);
    u32x4 av[kMaxPerLane];
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
        if (!chunk_ok(j, lane)) continue;
        uint32_t ap[4];
        modulate_chunk(rg.x[j], wl[j * 64 + lane], rg.sc[j], rg.sh[j], r, ap);
        av[j] = u32x4{ap[0], ap[1], ap[2], ap[3]};
        float a[8];
        unpack8(av[j], a);
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(a[e]));
    }
    amax = wave_max(amax);
    const float s = amax / 448.0f;             // IEEE division: RN(amax / 448)
    if (lane == 0) a_scale[m] = s;
    uint8_t* const ql = qr + lane * 8;
    if (s == 0.f) {
#pragma unroll
        for (int j = 0; j < kMaxPerLane; ++j)
            if (chunk_ok(j, lane)) *reinterpret_cast<uint2*>(ql + j * 512) = make_uint2(0u, 0u);
    } else if (s >= 1.17549435e-38f) {         // FLT_MIN: RN(1 / s) is finite, div_by applies
        const float inv = 1.0f / s;            // RN(1 / s)
#pragma unroll
        for (int j = 0; j < kMaxPerLane; ++j) {
            if (!chunk_ok(j, lane)) continue;
            float a[8];
            unpack8(av[j], a);
            uint2 q;
            q.x = f2e4m3x2(div_by(a[0], s, inv), div_by(a[1], s, inv)) |
                  (f2e4m3x2(div_by(a[2], s, inv), div_by(a[3], s, inv)) << 16);
            q.y = f2e4m3x2(div_by(a[4], s, inv), div_by(a[5], s, inv)) |
                  (f2e4m3x2(div_by(a[6], s, inv), div_by(a[7], s, inv)) << 16);
            *reinterpret_cast<uint2*>(ql + j * 512) = q;
        }
    } else {                                   // subnormal s: IEEE division
#pragma unroll
        for (int j = 0; j < kMaxPerLane; ++j) {
            if (!chunk_ok(j, lane)) continue;
            float a[8];
            unpack8(av[j], a);
            uint2 q;
            q.x = f2e4m3x2(a[0] / s, a[1] / s) | (f2e4m3x2(a[2] / s, a[3] / s) << 16);
            q.y = f2e4m3x2(a[4] / s, a[5] / s) | (f2e4m3x2(a[6] / s, a[7] / s) << 16);
            *reinterpret_cast<uint2*>(ql + j * 512) = q;
        }
    }
}

hipError_t launch_norm_adaln_bf16(const uint16_t* x, int64_t M, const uint16_t* xw, const uint16_t* scale,
                                  int64_t ld_scale, const uint16_t* shift, int64_t ld_shift, int64_t rows,
                                  const int64_t* idx, float eps, uint16_t* ws, hipStream_t stream) {
    const int64_t blocks = (M + 3) / 4;
    hipLaunchKernelGGL(k_norm_adaln_bf16, dim3((unsigned)blocks), dim3(256), 0, stream, x, M, xw, scale, ld_scale,
                       shift, ld_shift, rows, idx, eps, ws);
    return hipGetLastError();
}

hipError_t launch_norm_adaln_mxfp4(const uint16_t* x, int64_t M, const uint16_t* xw, const uint16_t* scale,
                                   int64_t ld_scale, const uint16_t* shift, int64_t ld_shift, int64_t rows,
                                   const int64_t* idx, float eps, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
    const int64_t R_pad = (M + 127) / 128 * 128;
    hipLaunchKernelGGL(k_norm_adaln_mxfp4, dim3((unsigned)(R_pad / 4)), dim3(256), 0, stream, x, M, xw, scale, ld_scale,
                       shift, ld_shift, rows, idx, eps, R_pad, codes, scales);
    return hipGetLastError();
}

hipError_t launch_norm_adaln_fp8q(const uint16_t* x, int64_t M, const uint16_t* xw, const uint16_t* scale,
                                  int64_t ld_scale, const uint16_t* shift, int64_t ld_shift, int64_t rows,
                                  const int64_t* idx, float eps, uint8_t* a_q, float* a_scale, hipStream_t stream) {
    const int64_t blocks = (M + 3) / 4;
    hipLaunchKernelGGL(k_norm_adaln_fp8q, dim3((unsigned)blocks), dim3(256), 0, stream, x, M, xw, scale, ld_scale,
                       shift, ld_shift, rows, idx, eps, a_q, a_scale);
    return hipGetLastError();
}

}  // namespace dit
