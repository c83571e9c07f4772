// Tiled MFMA GEMM core for gfx950 shared by the QKV, out-projection, FC1 and FC2 kernels.
//
// C[m, n] = sum_k A[m, k] * B[n, k]: both operands are K-contiguous rows (activations
// [M, K], weights [N, K]), FP32 accumulation.
//
// Workgroup: 256 threads = 4 wavefronts (one per SIMD), output tile 256 x 256, wave tile
// 128 x 128 held as 4 x 4 blocks of the 32x32 MFMA (256 FP32 accumulators per lane).  K is
// consumed in tiles of 128 bytes (64 bf16 or 128 e4m3): per K tile every thread fetches
// eight 16-byte chunks of A and eight of B of the next tile into registers, the waves run
// the MFMAs on the current LDS stage, then the fetched chunks are written to the other stage
// (double buffer, 2 x 64 KiB) and one barrier closes the step.  LDS rows are 128 bytes; the 16-byte chunk index is
// XOR-swizzled with the row so that the MFMA operand reads of 8 consecutive rows hit 8
// different bank groups.
//
// bf16: v_mfma_f32_32x32x16_bf16, 4 k-steps per K tile.
// e4m3: v_mfma_f32_32x32x64_f8f6f4 (both operands OCP e4m3), 2 k-steps per K tile.
// A and B fragments take their k values from the same (lane half, byte) positions, so the
// product is the same whatever order the instruction assigns to k inside a fragment.
//
// Rows of A past M are read from row M-1 (always in bounds) and never stored.
#pragma once

#include "common.hpp"

namespace dit {
namespace gemm {

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBKB = 128;                       // K tile, bytes per row
constexpr int kThreads = 256;
constexpr int kTileBytes = 256 * kBKB;          // one operand tile: 32 KiB
constexpr int kStageBytes = 2 * kTileBytes;     // A + B
constexpr int kMainBytes = 2 * kStageBytes;     // double buffer: 128 KiB
constexpr int kEpiPitch = kBN * 2 + 16;         // bf16 epilogue tile, padded row pitch (bytes)
constexpr int kEpiBytes = kBM * kEpiPitch;      // 132 KiB
constexpr int kSmemBytes = kMainBytes > kEpiBytes ? kMainBytes : kEpiBytes;

__device__ __forceinline__ int lds_off(int row, int chunk) { return row * kBKB + ((chunk ^ (row & 7)) << 4); }

// Workgroup id -> (m tile, n tile).  Workgroups are dispatched round-robin over the 8 XCDs,
// so id % 8 names the XCD: each XCD gets one contiguous range of the logical order, and the
// logical order walks groups of 8 m-tiles across all n-tiles (m fastest), so the ~32 tiles
// an XCD runs at once share 8 A panels and 4 B panels in its L2.
__device__ __forceinline__ void tile_coords(int bid, int mt, int nt, int& tm, int& tn) {
    const int G = mt * nt;
    const int xcd = bid & 7, idx = bid >> 3;
    const int per = G >> 3, rem = G & 7;
    const int L = xcd * per + (xcd < rem ? xcd : rem) + idx;
    constexpr int GM = 8;
    const int group = L / (GM * nt);
    const int first_m = group * GM;
    const int gsize = (mt - first_m) < GM ? (mt - first_m) : GM;
    const int in = L - group * GM * nt;
    tm = first_m + in % gsize;
    tn = in / gsize;
}

// MFMA operand fragments of one k-step: 4 A blocks and 4 B blocks of 32 rows.
template <bool kFp8>
struct Frags;
template <>
struct Frags<false> {
    bf16x8 a[4], b[4];
};
template <>
struct Frags<true> {
    i32x8 a[4], b[4];
};

constexpr int ksteps(bool fp8) { return fp8 ? 2 : 4; }

// Reads the fragments of k-step ks from an LDS stage.  bf16: lane l takes 8 consecutive k
// (16 bytes) of row l%32 at k offset 8*(l/32) within the 16-wide step; e4m3: 32 bytes at
// byte offset 32*(l/32) within the 64-wide step.
template <bool kFp8>
__device__ __forceinline__ void load_frags(const uint8_t* __restrict__ stage, int ks, Frags<kFp8>& f) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int r32 = lane & 31, hi = lane >> 5;
    const uint8_t* As = stage;
    const uint8_t* Bs = stage + kTileBytes;
    if constexpr (!kFp8) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            f.a[i] = *reinterpret_cast<const bf16x8*>(As + lds_off(wm * 128 + i * 32 + r32, ks * 2 + hi));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            f.b[j] = *reinterpret_cast<const bf16x8*>(Bs + lds_off(wn * 128 + j * 32 + r32, ks * 2 + hi));
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = wm * 128 + i * 32 + r32;
            const u32x4 lo = *reinterpret_cast<const u32x4*>(As + lds_off(row, ks * 4 + hi * 2));
            const u32x4 up = *reinterpret_cast<const u32x4*>(As + lds_off(row, ks * 4 + hi * 2 + 1));
            f.a[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)up[0], (int)up[1], (int)up[2], (int)up[3]};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = wn * 128 + j * 32 + r32;
            const u32x4 lo = *reinterpret_cast<const u32x4*>(Bs + lds_off(row, ks * 4 + hi * 2));
            const u32x4 up = *reinterpret_cast<const u32x4*>(Bs + lds_off(row, ks * 4 + hi * 2 + 1));
            f.b[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)up[0], (int)up[1], (int)up[2], (int)up[3]};
        }
    }
}

template <bool kFp8>
__device__ __forceinline__ void mma_step(const Frags<kFp8>& f, f32x16 (&acc)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (!kFp8)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
            else
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], 0, 0, 0, 0,
                                                                             0, 0);
        }
}

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSgMfma = 0x008;
constexpr int kSgDsRead = 0x100;

// Orders the scheduling region as n x [mfma_per MFMAs, 1 LDS read].
template <int N, int MfmaPer>
__device__ __forceinline__ void interleave_mfma_ds() {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, MfmaPer, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
    }
}

// Main loop over `ktiles` K tiles.  A rows m0.. (clamped to M-1), B local rows [0,128) are
// global rows nb0.., local rows [128,256) are nb1.. (nb1 = nb0 + 128 for a plain tile).
//
// One iteration, in this order (scheduling barriers keep the compiler from merging phases):
//   1. issue the global loads of K tile kt+1 into registers;
//   2. the MFMAs of every k-step but the last, each interleaved with the LDS reads of the
//      next k-step's fragments (fragments are double-buffered in registers);
//   3. write the registers of tile kt+1 to the other LDS stage; barrier;
//   4. the MFMAs of the last k-step (its fragments are already in registers), interleaved
//      with the LDS reads of the first fragments of tile kt+1.
// The global latency is covered by a K tile of MFMAs and every LDS read by a k-step of them.
// The body has no branches: on the last iteration the loads re-read the last K tile (in
// bounds) and the stage written is never read.  Ends with a barrier, so the caller may reuse
// the LDS.
template <bool kFp8>
__device__ __forceinline__ void mainloop(const uint8_t* __restrict__ A, int64_t lda, int64_t m0, int64_t M,
                                         const uint8_t* __restrict__ B, int64_t ldb, int64_t nb0, int64_t nb1,
                                         int ktiles, uint8_t* smem, f32x16 (&acc)[4][4]) {
    constexpr int KS = ksteps(kFp8);
    constexpr int kReadsPerStep = kFp8 ? 16 : 8;     // ds_read_b128 per k-step per lane
    constexpr int kMfmaPerRead = 16 / kReadsPerStep;
    const int t = threadIdx.x;
    const int lrow = t >> 3, chunk = t & 7;
    const uint8_t* pa[8];
    const uint8_t* pb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = j * 32 + lrow;
        int64_t gm = m0 + r;
        gm = gm < M ? gm : M - 1;
        pa[j] = A + gm * lda + chunk * 16;
        const int64_t gn = r < 128 ? nb0 + r : nb1 + (r - 128);
        pb[j] = B + gn * ldb + chunk * 16;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    u32x4 ra[8], rb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        ra[j] = ld16(pa[j]);
        rb[j] = ld16(pb[j]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        *reinterpret_cast<u32x4*>(smem + lds_off(j * 32 + lrow, chunk)) = ra[j];
        *reinterpret_cast<u32x4*>(smem + kTileBytes + lds_off(j * 32 + lrow, chunk)) = rb[j];
    }
    __syncthreads();
    Frags<kFp8> f[2];
    load_frags<kFp8>(smem, 0, f[0]);

    for (int kt = 0; kt < ktiles; ++kt) {
        const uint8_t* cur = smem + (kt & 1) * kStageBytes;
        uint8_t* nxt = smem + ((kt + 1) & 1) * kStageBytes;
        const int64_t koff = (int64_t)(kt + 1 < ktiles ? kt + 1 : kt) * kBKB;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            ra[j] = ld16(pa[j] + koff);
            rb[j] = ld16(pb[j] + koff);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks + 1 < KS; ++ks) {
            load_frags<kFp8>(cur, ks + 1, f[(ks + 1) & 1]);
            mma_step<kFp8>(f[ks & 1], acc);
        }
        interleave_mfma_ds<(KS - 1) * kReadsPerStep, kMfmaPerRead>();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            *reinterpret_cast<u32x4*>(nxt + lds_off(j * 32 + lrow, chunk)) = ra[j];
            *reinterpret_cast<u32x4*>(nxt + kTileBytes + lds_off(j * 32 + lrow, chunk)) = rb[j];
        }
        __syncthreads();
        load_frags<kFp8>(nxt, 0, f[KS & 1]);
        mma_step<kFp8>(f[(KS - 1) & 1], acc);
        interleave_mfma_ds<kReadsPerStep, kMfmaPerRead>();
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
}

// Epilogue phase 1: tile[row][col] = bf16((acc * rowscale[row]) * colscale[col]) into LDS
// (row pitch kEpiPitch); with scales the products are formed in double and rounded once.
// Accumulator layout of the 32x32 MFMA: lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4
// and column l%32 of its block.  rowscale and colscale are both given or both null (factor 1).
// Must follow a barrier that ends all LDS reads of the main loop.
__device__ __forceinline__ void stage_tile_bf16(const f32x16 (&acc)[4][4], uint8_t* smem, const float* rowscale,
                                                int64_t m0, int64_t M, const float* colscale_lo,
                                                const float* colscale_hi) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int r32 = lane & 31, hi = lane >> 5;
    float cscale[4] = {1.f, 1.f, 1.f, 1.f};
    if (colscale_lo) {
        // local columns [0,128) come from colscale_lo, [128,256) from colscale_hi
        const float* cs = wn == 0 ? colscale_lo : colscale_hi;
#pragma unroll
        for (int j = 0; j < 4; ++j) cscale[j] = cs[j * 32 + r32];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = wm * 128 + i * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
            float rs = 1.f;
            if (rowscale) {
                int64_t gm = m0 + row;
                gm = gm < M ? gm : M - 1;
                rs = rowscale[gm];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = wn * 128 + j * 32 + r32;
                uint32_t b;
                if (rowscale) {
                    // (acc * s_row) * s_col in double, one rounding to bf16
                    b = f2bf_d((double)acc[i][j][r] * (double)rs * (double)cscale[j]);
                } else {
                    b = f2bf(acc[i][j][r]);
                }
                *reinterpret_cast<uint16_t*>(smem + row * kEpiPitch + col * 2) = (uint16_t)b;
            }
        }
    }
}

__device__ __forceinline__ u32x4 epi_ld(const uint8_t* smem, int row, int col) {
    return *reinterpret_cast<const u32x4*>(smem + row * kEpiPitch + col * 2);
}

}  // namespace gemm
}  // namespace dit
