// Tiled MFMA GEMM core for gfx950 shared by the QKV, out-projection, FC1 and FC2 kernels.
//
// C[m, n] = sum_k A[m, k] * B[n, k]: both operands are K-contiguous rows (activations
// [M, K], weights [N, K]), FP32 accumulation.
//
// Workgroup: 256 threads = 4 wavefronts (one per SIMD), output tile 256 x 256, wave tile
// 128 x 128 held as 4 x 4 blocks of the 32x32 MFMA (256 FP32 accumulators per lane, in
// AGPRs).  K is consumed in stages of 64 bytes per row (32 bf16 or 64 e4m3).  Each stage
// (A 256 x 64 B + B 256 x 64 B = 32 KiB) is filled straight from global memory into LDS by
// buffer_load_dwordx4 ... lds (no register staging, no LDS store instructions); four stages
// rotate in 128 KiB of LDS and the loads run three stages ahead of the MFMAs.
//
// Per stage (two halves of 16 bf16 MFMAs, or 8 e4m3 MFMAs, per wave):
//   first half  : MFMAs on fragments already in registers, interleaved with the LDS reads of
//                 the second half's fragments;
//   wait for the next stage's loads (vmcnt), barrier;
//   issue the loads of the stage three ahead into the buffer just released;
//   second half : MFMAs, interleaved with the LDS reads of the next stage's first fragments.
// So every LDS read is covered by MFMAs and global latency by three stages of them.
//
// bf16: v_mfma_f32_32x32x16_bf16 (two k-steps of 16 per stage).
// e4m3: v_mfma_f32_32x32x64_f8f6f4 (one k-step of 64 per stage, split by A blocks).
// A and B fragments take their k values from the same (lane half, byte) positions, so the
// product is the same whatever order the instruction assigns to k inside a fragment.
//
// Rows of A past M read as zeros (buffer descriptor bound) and are never stored.
#pragma once

#include "common.hpp"

namespace dit {
namespace gemm {

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kRowB = 64;                       // bytes of K per row per stage
constexpr int kThreads = 256;
constexpr int kOpBytes = 256 * kRowB;           // one operand of one stage: 16 KiB
constexpr int kStageBytes = 2 * kOpBytes;       // A then B: 32 KiB
constexpr int kStages = 4;
constexpr int kMainBytes = kStages * kStageBytes;   // 128 KiB
constexpr int kEpiPitch = kBN * 2 + 16;         // bf16 epilogue tile, padded row pitch (bytes)
constexpr int kEpiBytes = kBM * kEpiPitch;      // 132 KiB
constexpr int kSmemBytes = kMainBytes > kEpiBytes ? kMainBytes : kEpiBytes;
constexpr int kLoadsPerStage = 8;               // buffer loads per wave per stage (4 A + 4 B)

// LDS layout of an operand within a stage: row r (0..255) holds 64 bytes = 4 chunks of 16;
// chunk c of row r sits at r * 64 + ((c ^ ((r / 4) % 4)) * 16).  An MFMA operand read has 16
// lanes on 16 consecutive rows and one chunk: (r % 4, swizzled chunk) then takes 16 distinct
// values, i.e. 16 distinct 16-byte bank groups of the 64-bank LDS.  The fills are 64 lanes
// writing 1 KiB contiguously, conflict-free.

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

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// s_waitcnt with only a vmcnt limit (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Raw buffer descriptor over [base, base + bytes): loads at offsets >= bytes return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Global -> LDS fill of one stage.  Wave w fills rows [64w, 64w + 64) of A and of B in four
// 1 KiB pieces of 16 rows; lane l of piece j lands at byte 16 l of the piece, i.e. row
// 64w + 16j + l/4, stored chunk l%4, so it loads logical chunk (l%4) ^ ((l/16)%4).
struct StageFill {
    __amdgpu_buffer_rsrc_t ra, rb;
    uint32_t va[4];      // A: row offset of piece j + chunk offset (per lane; bounds-checked)
    uint32_t vb;         // B: row-in-piece offset + chunk offset (per lane)
    uint32_t sb[4];      // B: offset of piece j's first row (uniform)
    uint32_t lds_w;      // this wave's 4 KiB slice within an operand
    __device__ __forceinline__ void issue(uint8_t* smem, int stage, int kt) const {
        lds_u8* S = (lds_u8*)smem + stage * kStageBytes + lds_w;
        const int koff = kt * kRowB;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, S + j * 1024, 16, (int)va[j], koff, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, S + kOpBytes + j * 1024, 16, (int)vb, (int)sb[j] + koff, 0,
                                                     0);
    }
};

// Per-lane LDS offsets of the fragment reads (relative to a stage).  Lane l reads row
// r = l % 32 of each 32-row block; the swizzle depends only on (r / 4) % 4, so block i is an
// immediate i * 2048 and the stage an immediate too.  Slot q: bf16 k-step q reads chunk
// 2q + l/32; e4m3 reads chunks 2(l/32) + q (the two halves of its 32 bytes).
struct FragAddr {
    uint32_t a[2], b[2];
    __device__ __forceinline__ void init(bool fp8) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int wm = wave >> 1, wn = wave & 1;
        const int r32 = lane & 31, hi = lane >> 5;
        const int sw = (r32 >> 2) & 3;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = fp8 ? 2 * hi + q : 2 * q + hi;
            a[q] = (uint32_t)((wm * 128 + r32) * kRowB + ((c ^ sw) << 4));
            b[q] = (uint32_t)(kOpBytes + (wn * 128 + r32) * kRowB + ((c ^ sw) << 4));
        }
    }
};

__device__ __forceinline__ u32x4 lds_ld16(const uint8_t* smem, uint32_t off) {
    return *reinterpret_cast<const u32x4*>(smem + off);
}
__device__ __forceinline__ bf16x8 lds_bf16x8(const uint8_t* smem, uint32_t off) {
    return *reinterpret_cast<const bf16x8*>(smem + off);
}
__device__ __forceinline__ i32x8 lds_i32x8(const uint8_t* smem, uint32_t off0, uint32_t off1) {
    const u32x4 lo = lds_ld16(smem, off0), up = lds_ld16(smem, off1);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)up[0], (int)up[1], (int)up[2], (int)up[3]};
}

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSgMfma = 0x008;
constexpr int kSgDsRead = 0x100;

// Orders the scheduling region as N x [MfmaPer MFMAs, 1 LDS read].
template <int N, int MfmaPer>
__device__ __forceinline__ void interleave_mfma_ds() {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, MfmaPer, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
    }
}
// Orders the scheduling region as N x [1 LDS read, MfmaPer MFMAs] (the reads lead, so the
// last one has MfmaPer MFMAs of time to land before the region ends).
template <int N, int MfmaPer>
__device__ __forceinline__ void interleave_ds_mfma() {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgMfma, MfmaPer, 0);
    }
}

// Stage hand-over: this wave's LDS reads of the stage it is leaving have landed (lgkmcnt 0:
// after the barrier other waves refill that stage by DMA), its loads of the next stage have
// landed (vmcnt), then the workgroup barrier makes every wave's fill visible.
__device__ __forceinline__ void stage_barrier() {
    constexpr int kVm = kLoadsPerStage * (kStages - 2);
    static_assert(kVm < 64, "vmcnt range");
    // s_waitcnt vmcnt(kVm) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_waitcnt((kVm & 15) | ((kVm >> 4) << 14) | (7 << 4) | (0 << 8));
    __syncthreads();
}

// bf16 pipeline.  fA/fB[h]: fragments of k-step h (4 A blocks, 4 B blocks).
struct PipeBf16 {
    bf16x8 a[2][4], b[2][4];
    __device__ __forceinline__ void read(const uint8_t* st, const FragAddr& fa, int h) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[h][i] = lds_bf16x8(st, fa.a[h] + i * 2048);
#pragma unroll
        for (int j = 0; j < 4; ++j) b[h][j] = lds_bf16x8(st, fa.b[h] + j * 2048);
    }
    __device__ __forceinline__ void mma(int h, f32x16 (&acc)[4][4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[h][i], b[h][j], acc[i][j], 0, 0, 0);
    }
    // first half: k-step 0, while reading k-step 1; second half: k-step 1, while reading the
    // next stage's k-step 0
    __device__ __forceinline__ void first(const uint8_t* st, const FragAddr& fa, f32x16 (&acc)[4][4]) {
        read(st, fa, 1);
        mma(0, acc);
        interleave_ds_mfma<8, 2>();
    }
    __device__ __forceinline__ void second(const uint8_t* next, const FragAddr& fa, f32x16 (&acc)[4][4]) {
        read(next, fa, 0);
        mma(1, acc);
        interleave_mfma_ds<8, 2>();
    }
    __device__ __forceinline__ void prime(const uint8_t* st, const FragAddr& fa) { read(st, fa, 0); }
};

// e4m3 pipeline: one 32x32x64 k-step per stage; the first half runs A blocks 0-1, the
// second A blocks 2-3, both against B blocks 0-3.  During the second half the next stage's
// A blocks 0-1 are read first (free since the first half), then each B block is re-read for
// the next stage right after its last two MFMAs, so no fragment needs a second buffer.
struct PipeFp8 {
    i32x8 a[4], b[4];
    __device__ __forceinline__ void read_a(const uint8_t* st, const FragAddr& fa, int i) {
        a[i] = lds_i32x8(st, fa.a[0] + i * 2048, fa.a[1] + i * 2048);
    }
    __device__ __forceinline__ void read_b(const uint8_t* st, const FragAddr& fa, int j) {
        b[j] = lds_i32x8(st, fa.b[0] + j * 2048, fa.b[1] + j * 2048);
    }
    __device__ __forceinline__ void mma(int i, int j, f32x16 (&acc)[4][4]) {
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 0, 0, 0, 0, 0, 0);
    }
    __device__ __forceinline__ void prime(const uint8_t* st, const FragAddr& fa) {
#pragma unroll
        for (int i = 0; i < 2; ++i) read_a(st, fa, i);
#pragma unroll
        for (int j = 0; j < 4; ++j) read_b(st, fa, j);
    }
    __device__ __forceinline__ void first(const uint8_t* st, const FragAddr& fa, f32x16 (&acc)[4][4]) {
        read_a(st, fa, 2);
        read_a(st, fa, 3);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) mma(i, j, acc);
        interleave_ds_mfma<4, 2>();
    }
    __device__ __forceinline__ void second(const uint8_t* next, const FragAddr& fa, f32x16 (&acc)[4][4]) {
        read_a(next, fa, 0);
        read_a(next, fa, 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            mma(2, j, acc);
            mma(3, j, acc);
            read_b(next, fa, j);
        }
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 4, 0);
        interleave_mfma_ds<8, 1>();
    }
};

// Main loop over `ktiles` stages of K.  A rows m0.. (rows past M read as zero), B local rows
// [0,128) are global rows nb0.., local rows [128,256) are nb1.. (nb1 = nb0 + 128 for a
// plain tile).  Ends with all loads drained and a barrier, so the caller may reuse the LDS.
template <bool kFp8>
__device__ __forceinline__ void mainloop(const uint8_t* __restrict__ A, int64_t lda, int64_t m0, int64_t M,
                                         const uint8_t* __restrict__ B, int64_t ldb, int64_t nb0, int64_t nb1,
                                         int ktiles, uint8_t* smem, f32x16 (&acc)[4][4]) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
    StageFill sf;
    const int64_t arows = M - m0 < kBM ? M - m0 : kBM;
    sf.ra = make_rsrc(A + m0 * lda, (uint32_t)(arows * lda));
    sf.rb = make_rsrc(B + nb0 * ldb, (uint32_t)((nb1 - nb0 + 128) * ldb));
    const uint32_t cbyte = (uint32_t)(((lane & 3) ^ ((lane >> 4) & 3)) << 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        sf.va[j] = (uint32_t)((64 * wave + 16 * j + (lane >> 2)) * lda) + cbyte;
        const int64_t r0 = 64 * wave + 16 * j;
        sf.sb[j] = (uint32_t)((r0 < 128 ? r0 : r0 + (nb1 - nb0 - 128)) * ldb);
    }
    sf.vb = (uint32_t)((lane >> 2) * ldb) + cbyte;
    sf.lds_w = (uint32_t)(wave * 4096);
    FragAddr fa;
    fa.init(kFp8);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // prologue: stages 0..3 in flight, wait for stage 0
#pragma unroll
    for (int s = 0; s < kStages; ++s) sf.issue(smem, s, s < ktiles ? s : ktiles - 1);
    wait_vmcnt<kLoadsPerStage * (kStages - 1)>();
    __syncthreads();

    if constexpr (!kFp8) {
        PipeBf16 p;
        p.prime(smem, fa);
        for (int kt = 0; kt < ktiles; ++kt) {
            const int s = kt & (kStages - 1);
            const uint8_t* st = smem + s * kStageBytes;
            const uint8_t* nx = smem + ((kt + 1) & (kStages - 1)) * kStageBytes;
            __builtin_amdgcn_sched_barrier(0);
            p.first(st, fa, acc);
            __builtin_amdgcn_sched_barrier(0);
            stage_barrier();
            const int kl = kt + kStages < ktiles ? kt + kStages : ktiles - 1;
            sf.issue(smem, s, kl);
            __builtin_amdgcn_sched_barrier(0);
            p.second(nx, fa, acc);
        }
    } else {
        PipeFp8 p;
        p.prime(smem, fa);
        for (int kt = 0; kt < ktiles; ++kt) {
            const int s = kt & (kStages - 1);
            const uint8_t* st = smem + s * kStageBytes;
            const uint8_t* nx = smem + ((kt + 1) & (kStages - 1)) * kStageBytes;
            __builtin_amdgcn_sched_barrier(0);
            p.first(st, fa, acc);
            __builtin_amdgcn_sched_barrier(0);
            stage_barrier();
            const int kl = kt + kStages < ktiles ? kt + kStages : ktiles - 1;
            sf.issue(smem, s, kl);
            __builtin_amdgcn_sched_barrier(0);
            p.second(nx, fa, acc);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();
    __syncthreads();
}

// Reads one accumulator out of its AGPR where it is used.  Without this the compiler copies
// all 256 accumulators into VGPRs at the loop exit (the conversions below cannot read AGPRs),
// which does not fit next to the epilogue's own registers.
__device__ __forceinline__ float acc_read(float a) {
    float v;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
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
    // one 32x32 block at a time (the scheduling barrier keeps the compiler from pulling all
    // 256 accumulators into VGPRs at once)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float rs[16];
        if (rowscale) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int64_t gm = m0 + wm * 128 + i * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
                gm = gm < M ? gm : M - 1;
                rs[r] = rowscale[gm];
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = wn * 128 + j * 32 + r32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * 128 + i * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
                const float a = acc_read(acc[i][j][r]);
                uint32_t b;
                if (rowscale) {
                    // (acc * s_row) * s_col in double, one rounding to bf16
                    b = f2bf_d((double)a * (double)rs[r] * (double)cscale[j]);
                } else {
                    b = f2bf(a);
                }
                *reinterpret_cast<uint16_t*>(smem + row * kEpiPitch + col * 2) = (uint16_t)b;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

__device__ __forceinline__ u32x4 epi_ld(const uint8_t* smem, int row, int col) {
    return *reinterpret_cast<const u32x4*>(smem + row * kEpiPitch + col * 2);
}

}  // namespace gemm
}  // namespace dit
