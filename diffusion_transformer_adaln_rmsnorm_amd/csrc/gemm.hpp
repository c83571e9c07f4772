// Tiled MFMA GEMM core for gfx950 shared by the QKV, out-projection, FC1 and FC2 kernels.
//
// C[m, n] = sum_k A[m, k] * B[n, k]: both operands are K-contiguous rows (activations
// [M, K], weights [N, K]), FP32 accumulation.
//
// Workgroup: kWaves wavefronts and one 256 x 256 output tile.  Default 8 waves, two per SIMD,
// each a 128 x 64 wave tile of 4 x 2 blocks of the 32x32 MFMA (128 FP32 accumulators per lane,
// so a wave fits in 256 registers): while one wave of a SIMD waits on its stage-fill loads or
// LDS reads the other issues MFMAs.  4 waves (one per SIMD, 128 x 128 wave tiles, 256
// accumulators in AGPRs) remain selectable with -DDIT_GEMM_WAVES=4.
//
// K is consumed in stages of kRowB bytes per row (128: 64 bf16 or 128 e4m3, one full cache
// line per row).  Each stage (A 256 rows + B 256 rows) is filled straight from
// global memory into LDS by buffer_load_dwordx4 ... lds (no register staging, no LDS store
// instructions); kStages stages rotate in LDS and the loads of a stage are issued as soon as
// its buffer is released.
//
// Per stage:
//   first : the MFMAs of all k-steps but the last, each interleaved with the LDS reads of
//           the next k-step's fragments (fragments double-buffered in registers);
//   wait for the next stage's loads (vmcnt) and this wave's LDS reads, barrier;
//   issue the loads of the stage kStages ahead into the buffer just released;
//   second: the MFMAs of the last k-step, interleaved with the LDS reads of the next stage's
//           first fragments and with the loads just issued.
// So every LDS read is covered by MFMAs and global latency by the stages in flight.
//
// bf16: v_mfma_f32_32x32x16_bf16 (k-steps of 16).
// e4m3: v_mfma_f32_32x32x64_f8f6f4 (k-steps of 64).
// A and B fragments take their k values from the same (lane half, byte) positions, so the
// product is the same whatever order the instruction assigns to k inside a fragment.
//
// Rows of A past M read as zeros (buffer descriptor bound) and are never stored.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace dit {
namespace gemm {

constexpr int kBM = 256;
constexpr int kBN = 256;
#ifndef DIT_GEMM_ROW_BYTES
#define DIT_GEMM_ROW_BYTES 128
#endif
constexpr int kRowB = DIT_GEMM_ROW_BYTES;       // bytes of K per row per stage (64 or 128)
static_assert(kRowB == 64 || kRowB == 128, "stage row width");
#ifndef DIT_GEMM_WAVES
#define DIT_GEMM_WAVES 8
#endif
constexpr int kWaves = DIT_GEMM_WAVES;          // wavefronts per workgroup: 4 (one per SIMD) or 8 (two)
static_assert(kWaves == 4 || kWaves == 8, "wave count");
constexpr int kThreads = 64 * kWaves;
constexpr int kWN = kWaves / 2;                 // waves across n (two across m)
constexpr int kNB = 8 / kWN;                    // 32-column MFMA blocks per wave (4 or 2)
constexpr int kWaveN = 32 * kNB;                // wave tile: 128 rows x kWaveN columns
constexpr int kOpBytes = 256 * kRowB;           // one operand of one stage
constexpr int kStageBytes = 2 * kOpBytes;       // A then B
#ifndef DIT_GEMM_STAGES
#define DIT_GEMM_STAGES (kRowB == 64 ? 4 : 2)
#endif
constexpr int kStages = DIT_GEMM_STAGES;        // LDS stages in the ring (loads run kStages-1 ahead)
constexpr int kMainBytes = kStages * kStageBytes;
constexpr int kEpiPitch = kBN * 2 + 16;         // bf16 epilogue tile, padded row pitch (bytes)
constexpr int kEpiBytes = kBM * kEpiPitch;      // 132 KiB
constexpr int kSmemBytes = kMainBytes > kEpiBytes ? kMainBytes : kEpiBytes;
#ifndef DIT_GEMM_LOAD_AUX
#define DIT_GEMM_LOAD_AUX 0
#endif
constexpr int kLoadAux = DIT_GEMM_LOAD_AUX;     // cache-policy bits of the stage-fill loads
constexpr int kSlots = kRowB / 16;              // 16-byte chunks per row
constexpr int kRowsPerPiece = 1024 / kRowB;     // rows filled by one 1 KiB wave load
constexpr int kFillRows = 256 / kWaves;         // rows of each operand one wave fills per stage
constexpr int kPieces = kFillRows / kRowsPerPiece;   // wave loads per operand per stage
constexpr int kLoadsPerStage = 2 * kPieces;     // buffer loads per wave per stage

// LDS layout of an operand within a stage: row r (0..255) holds kRowB bytes = kSlots chunks
// of 16; chunk c of row r sits at r * kRowB + ((c ^ swz(r)) * 16), swz(r) = (r / 4) % 4 for
// 64-byte rows and (r / 2) % 8 for 128-byte rows.  An MFMA operand read has 16 lanes on 16
// consecutive rows and one chunk, which then land in 16 distinct 16-byte bank groups of the
// 64-bank LDS.  Fills are 64 lanes writing 1 KiB contiguously, conflict-free.
__host__ __device__ constexpr int swz(int r) { return kRowB == 64 ? (r >> 2) & 3 : (r >> 1) & 7; }

// Workgroup id -> (m tile, n tile).  Workgroups are dispatched round-robin over the 8 XCDs,
// so id % 8 names the XCD: each XCD gets one contiguous range of the logical order, and the
// logical order walks groups of 8 m-tiles across all n-tiles (m fastest), so the ~32 tiles
// an XCD runs at once share 8 A panels and 4 B panels in its L2.
__device__ __forceinline__ void tile_coords(int bid, int mt, int nt, int& tm, int& tn) {
    const int G = mt * nt;
    const int xcd = bid & 7, idx = bid >> 3;
    const int per = G >> 3, rem = G & 7;
    const int L = xcd * per + (xcd < rem ? xcd : rem) + idx;
#ifndef DIT_GEMM_GROUP_M
#define DIT_GEMM_GROUP_M 4
#endif
    constexpr int GM = DIT_GEMM_GROUP_M;
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

// Raw buffer descriptor over [base, base + bytes): loads at offsets >= bytes return zeros and
// stores there are dropped (the check covers the per-lane offset, not the scalar one).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Epilogue accesses through descriptors: out-of-range lanes need no branch, so every load of
// an epilogue row is issued unconditionally and the compiler can count the loads in flight
// instead of waiting for all of them where control flow merges.
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ int64_t buf_ld_i64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    return (int64_t)(((uint64_t)(uint32_t)v[1] << 32) | (uint32_t)v[0]);
}
__device__ __forceinline__ int32_t buf_ld_i32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return (int32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_st16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}
constexpr uint32_t kOffNone = 0xFFFFFFF0u;   // an offset past every descriptor's bound

// Global -> LDS fill of one stage.  Wave w fills rows [F w, F w + F) of A and of B
// (F = kFillRows) in kPieces 1 KiB pieces of kRowsPerPiece rows; lane l of piece j lands at
// byte 16 l of the piece, i.e. row F w + j*kRowsPerPiece + l/kSlots, stored chunk l%kSlots,
// so it loads the logical chunk (l % kSlots) ^ swz(row).
// Within a wave's slice the swizzle of a piece's rows depends only on the piece's parity
// (128-byte rows) or not at all (64-byte rows), so B needs kVPat per-lane offsets; A keeps
// the row in the per-lane offset because only that part is checked against the descriptor's
// bound (rows past M).
constexpr int kVPat = kRowB == 128 ? 2 : 1;
struct StageFill {
    __amdgpu_buffer_rsrc_t ra, rb;
    uint32_t va[kPieces];    // A: row + chunk offset of piece j (per lane; bounds-checked)
    uint32_t vb[kVPat];      // B: row-in-piece + chunk offset, by piece parity (per lane)
    uint32_t sb[kPieces];    // B: offset of piece j's first row (uniform)
    uint32_t lds_w;          // this wave's slice within an operand
    // load j of the stage: A piece j for j < kPieces, else B piece j - kPieces
    __device__ __forceinline__ void one(uint8_t* smem, int stage, int kt, int j) const {
        lds_u8* S = (lds_u8*)smem + stage * kStageBytes + lds_w;
        const int koff = kt * kRowB;
        if (j < kPieces) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, S + j * 1024, 16, (int)va[j], koff, 0, kLoadAux);
        } else {
            const int b = j - kPieces;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, S + kOpBytes + b * 1024, 16, (int)vb[b % kVPat],
                                                     (int)sb[b] + koff, 0, kLoadAux);
        }
    }
    __device__ __forceinline__ void issue(uint8_t* smem, int stage, int kt) const {
#pragma unroll
        for (int j = 0; j < kLoadsPerStage; ++j) one(smem, stage, kt, j);
    }
};

// Per-lane LDS offsets of the fragment reads (relative to a stage).  Lane l reads row
// r = l % 32 of each 32-row block; the swizzle of rows r and r + 32i is the same, so block i
// is an immediate (32 * kRowB * i) and the stage an immediate too.  Slot q: bf16 k-step q
// reads chunk 2q + l/32; e4m3 k-step q/2 reads chunks 4(q/2) + 2(l/32) + q%2.
constexpr int kQ = kSlots / 2;                  // fragment slots per operand
constexpr int kBlk = 32 * kRowB;                // bytes of one 32-row block
struct FragAddr {
    uint32_t a[kQ], b[kQ];
    __device__ __forceinline__ void init(bool fp8) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int wm = wave / kWN, wn = wave % kWN;
        const int r32 = lane & 31, hi = lane >> 5;
        const int sw = swz(r32);    // swz has period 16 rows, so rows r32 + 32i share it
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            const int c = fp8 ? 4 * (q >> 1) + 2 * hi + (q & 1) : 2 * q + hi;
            a[q] = (uint32_t)((wm * 128 + r32) * kRowB + ((c ^ sw) << 4));
            b[q] = (uint32_t)(kOpBytes + (wn * kWaveN + r32) * kRowB + ((c ^ sw) << 4));
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
#ifndef DIT_SG_VMEM
#define DIT_SG_VMEM 0x020
#endif
constexpr int kSgVmemRead = DIT_SG_VMEM;
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

// Orders the scheduling region as N k-steps of R LDS reads spread over F MFMAs (each read
// leads its share of the MFMAs).  The group sizes of sched_group_barrier must be constants,
// hence the recursion over the group index.
#ifndef DIT_MFMA_FIRST
#define DIT_MFMA_FIRST 0
#endif
template <int R, int F, int I = 0>
__device__ __forceinline__ void interleave_kstep() {
    if constexpr (I < R) {
        if constexpr (DIT_MFMA_FIRST) {
            __builtin_amdgcn_sched_group_barrier(kSgMfma, F * (I + 1) / R - F * I / R, 0);
            __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
        } else {
            __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSgMfma, F * (I + 1) / R - F * I / R, 0);
        }
        interleave_kstep<R, F, I + 1>();
    }
}
template <int N, int R, int F>
__device__ __forceinline__ void interleave_ksteps() {
    if constexpr (N > 0) {
        interleave_kstep<R, F>();
        interleave_ksteps<N - 1, R, F>();
    }
}
// Orders the scheduling region as F x [its share of V stage loads, its share of R LDS reads,
// 1 MFMA].
template <int V, int R, int F, int I = 0>
__device__ __forceinline__ void interleave_fill() {
    if constexpr (I < F) {
        constexpr int v = V * (I + 1) / F - V * I / F, r = R * (I + 1) / F - R * I / F;
        if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(kSgVmemRead, v, 0);
        if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(kSgDsRead, r, 0);
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        interleave_fill<V, R, F, I + 1>();
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

// bf16 pipeline: kRowB/32 k-steps of 16 per stage, fragments double-buffered in registers.
//   first : k-steps 0..KS-2, each while reading the next k-step's fragments;
//   second: the last k-step, while reading the next stage's k-step 0 (the stage fill issued
//           just before is spread over it).
struct PipeBf16 {
    static constexpr int KS = kRowB / 32;
    static constexpr int R = 4 + kNB;           // fragment reads per k-step
    static constexpr int F = 4 * kNB;           // MFMAs per k-step
    bf16x8 a[2][4], b[2][kNB];
    __device__ __forceinline__ void read(const uint8_t* st, const FragAddr& fa, int ks, int h) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[h][i] = lds_bf16x8(st, fa.a[ks] + i * kBlk);
#pragma unroll
        for (int j = 0; j < kNB; ++j) b[h][j] = lds_bf16x8(st, fa.b[ks] + j * kBlk);
    }
    __device__ __forceinline__ void mma(int h, f32x16 (&acc)[4][kNB]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < kNB; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[h][i], b[h][j], acc[i][j], 0, 0, 0);
    }
    // fragment f of k-step ks into buffer h: A blocks 0..3, then B blocks 0..kNB-1
    __device__ __forceinline__ void read_one(const uint8_t* st, const FragAddr& fa, int ks, int h, int f) {
        if (f < 4) a[h][f] = lds_bf16x8(st, fa.a[ks] + f * kBlk);
        else b[h][f - 4] = lds_bf16x8(st, fa.b[ks] + (f - 4) * kBlk);
    }
    __device__ __forceinline__ void mma_one(int h, int i, f32x16 (&acc)[4][kNB]) {
        const int bi = i / kNB, bj = i % kNB;
        acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[h][bi], b[h][bj], acc[bi][bj], 0, 0, 0);
    }
    __device__ __forceinline__ void prime(const uint8_t* st, const FragAddr& fa) { read(st, fa, 0, 0); }
    __device__ __forceinline__ void first(const uint8_t* st, const FragAddr& fa, f32x16 (&acc)[4][kNB]) {
#pragma unroll
        for (int ks = 0; ks + 1 < KS; ++ks) {
            read(st, fa, ks + 1, (ks + 1) & 1);
            mma(ks & 1, acc);
        }
        if constexpr (kWaves == 4) {
            interleave_ds_mfma<8 * (KS - 1), 2>();
        } else {
            interleave_ksteps<KS - 1, R, F>();
        }
    }
    // The last k-step in F slots, fenced so the order is exactly: stage-fill load i, the next
    // stage's k-step-0 fragment read i (first R slots), MFMA i.
    __device__ __forceinline__ void second_fenced(const uint8_t* next, const FragAddr& fa, f32x16 (&acc)[4][kNB],
                                                  const StageFill& sf, uint8_t* smem, int stage, int kl) {
        static_assert(kLoadsPerStage <= F && R <= F, "slots");
#pragma unroll
        for (int i = 0; i < F; ++i) {
            if (i < kLoadsPerStage) sf.one(smem, stage, kl, i);
            if (i < R) read_one(next, fa, 0, KS & 1, i);
            mma_one((KS - 1) & 1, i, acc);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __device__ __forceinline__ void second(const uint8_t* next, const FragAddr& fa, f32x16 (&acc)[4][kNB]) {
        read(next, fa, 0, KS & 1);
        mma((KS - 1) & 1, acc);
        if constexpr (kWaves == 4) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
#pragma unroll
                for (int v = 0; v < kLoadsPerStage / 8; ++v) __builtin_amdgcn_sched_group_barrier(kSgVmemRead, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
            }
        } else {
            interleave_fill<kLoadsPerStage, R, F>();
        }
    }
};

// e4m3 pipeline for 64-byte rows: one 32x32x64 k-step per stage; the first half runs A
// blocks 0-1, the second A blocks 2-3, both against B blocks 0-3.  During the second half
// the next stage's A blocks 0-1 are read first (free since the first half), then each B
// block is re-read for the next stage right after its last two MFMAs, so no fragment needs a
// second buffer.
struct PipeFp8 {
    static_assert(kWaves == 4 || kRowB != 64, "the 64-byte-row e4m3 pipeline is written for 4 waves");
    i32x8 a[4], b[4];
    __device__ __forceinline__ void read_a(const uint8_t* st, const FragAddr& fa, int i) {
        a[i] = lds_i32x8(st, fa.a[0] + i * kBlk, fa.a[1] + i * kBlk);
    }
    __device__ __forceinline__ void read_b(const uint8_t* st, const FragAddr& fa, int j) {
        b[j] = lds_i32x8(st, fa.b[0] + j * kBlk, fa.b[1] + j * kBlk);
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
        // stage-fill loads, 12 LDS reads, 8 MFMAs
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 4, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSgVmemRead, kLoadsPerStage / 8, 0);
            __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
        }
    }
};

// e4m3 pipeline for 128-byte rows: two 32x32x64 k-steps per stage, fragments
// double-buffered like the bf16 pipeline.
struct PipeFp8K2 {
    static constexpr int R = 2 * (4 + kNB);     // 16-byte LDS reads per k-step
    static constexpr int F = 4 * kNB;           // MFMAs per k-step
    i32x8 a[2][4], b[2][kNB];
    __device__ __forceinline__ void read(const uint8_t* st, const FragAddr& fa, int ks, int h) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[h][i] = lds_i32x8(st, fa.a[2 * ks] + i * kBlk, fa.a[2 * ks + 1] + i * kBlk);
#pragma unroll
        for (int j = 0; j < kNB; ++j) b[h][j] = lds_i32x8(st, fa.b[2 * ks] + j * kBlk, fa.b[2 * ks + 1] + j * kBlk);
    }
    __device__ __forceinline__ void mma(int h, f32x16 (&acc)[4][kNB]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < kNB; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[h][i], b[h][j], acc[i][j], 0, 0, 0, 0,
                                                                             0, 0);
    }
    __device__ __forceinline__ void read_one(const uint8_t* st, const FragAddr& fa, int ks, int h, int f) {
        if (f < 4) a[h][f] = lds_i32x8(st, fa.a[2 * ks] + f * kBlk, fa.a[2 * ks + 1] + f * kBlk);
        else b[h][f - 4] = lds_i32x8(st, fa.b[2 * ks] + (f - 4) * kBlk, fa.b[2 * ks + 1] + (f - 4) * kBlk);
    }
    __device__ __forceinline__ void mma_one(int h, int i, f32x16 (&acc)[4][kNB]) {
        const int bi = i / kNB, bj = i % kNB;
        acc[bi][bj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[h][bi], b[h][bj], acc[bi][bj], 0, 0, 0, 0,
                                                                       0, 0);
    }
    // as in the bf16 pipeline: fill load i, fragment i of the next stage's k-step 0, MFMA i
    __device__ __forceinline__ void second_fenced(const uint8_t* next, const FragAddr& fa, f32x16 (&acc)[4][kNB],
                                                  const StageFill& sf, uint8_t* smem, int stage, int kl) {
        static_assert(kLoadsPerStage <= F && 4 + kNB <= F, "slots");
#pragma unroll
        for (int i = 0; i < F; ++i) {
            if (i < kLoadsPerStage) sf.one(smem, stage, kl, i);
            if (i < 4 + kNB) read_one(next, fa, 0, 0, i);
            mma_one(1, i, acc);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __device__ __forceinline__ void prime(const uint8_t* st, const FragAddr& fa) { read(st, fa, 0, 0); }
    __device__ __forceinline__ void first(const uint8_t* st, const FragAddr& fa, f32x16 (&acc)[4][kNB]) {
        read(st, fa, 1, 1);
        mma(0, acc);
        if constexpr (kWaves == 4) {
            interleave_ds_mfma<16, 1>();
        } else {
            interleave_ksteps<1, R, F>();
        }
    }
    __device__ __forceinline__ void second(const uint8_t* next, const FragAddr& fa, f32x16 (&acc)[4][kNB]) {
        read(next, fa, 0, 0);
        mma(1, acc);
        if constexpr (kWaves == 4) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                __builtin_amdgcn_sched_group_barrier(kSgVmemRead, kLoadsPerStage / 16, 0);
                __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
            }
        } else {
            interleave_fill<kLoadsPerStage, R, F>();
        }
    }
};

template <bool kFp8>
struct PipeOf {
    using type = PipeBf16;
};
template <>
struct PipeOf<true> {
    using type = typename std::conditional<kRowB == 64, PipeFp8, PipeFp8K2>::type;
};

// Main loop over `ktiles` stages of K.  A rows m0.. (rows past M read as zero), B local rows
// [0,128) are global rows nb0.., local rows [128,256) are nb1.. (nb1 = nb0 + 128 for a
// plain tile).  Ends with all loads drained and a barrier, so the caller may reuse the LDS.
template <bool kFp8>
__device__ __forceinline__ void mainloop(const uint8_t* __restrict__ A, int64_t lda, int64_t m0, int64_t M,
                                         const uint8_t* __restrict__ B, int64_t ldb, int64_t nb0, int64_t nb1,
                                         int ktiles, uint8_t* smem, f32x16 (&acc)[4][kNB]) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
    StageFill sf;
    const int64_t arows = M - m0 < kBM ? M - m0 : kBM;
    sf.ra = make_rsrc(A + m0 * lda, (uint32_t)(arows * lda));
    sf.rb = make_rsrc(B + nb0 * ldb, (uint32_t)((nb1 - nb0 + 128) * ldb));
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
        const int rin = j * kRowsPerPiece + lane / kSlots;          // row within the wave's slice
        const int row = kFillRows * wave + rin;
        const uint32_t cbyte = (uint32_t)(((lane % kSlots) ^ swz(row)) << 4);
        sf.va[j] = (uint32_t)(row * lda) + cbyte;
        const int64_t r0 = kFillRows * wave + j * kRowsPerPiece;      // piece's first row (uniform)
        sf.sb[j] = (uint32_t)((r0 < 128 ? r0 : r0 + (nb1 - nb0 - 128)) * ldb);
        if (j < kVPat) sf.vb[j] = (uint32_t)((lane / kSlots) * ldb) + cbyte;
    }
    sf.lds_w = (uint32_t)(wave * kFillRows * kRowB);
    FragAddr fa;
    fa.init(kFp8);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // prologue: every stage of the ring in flight, wait for stage 0
#pragma unroll
    for (int s = 0; s < kStages; ++s) sf.issue(smem, s, s < ktiles ? s : ktiles - 1);
    wait_vmcnt<kLoadsPerStage * (kStages - 1)>();
    __syncthreads();

    typename PipeOf<kFp8>::type p;
    p.prime(smem, fa);
    for (int kt = 0; kt < ktiles; ++kt) {
        const int s = kt % kStages;
        const uint8_t* st = smem + s * kStageBytes;
        const uint8_t* nx = smem + ((kt + 1) % kStages) * kStageBytes;
        __builtin_amdgcn_sched_barrier(0);
        p.first(st, fa, acc);
        __builtin_amdgcn_sched_barrier(0);
        stage_barrier();
        const int kl = kt + kStages < ktiles ? kt + kStages : ktiles - 1;
        if constexpr (kWaves == 8) {
            __builtin_amdgcn_sched_barrier(0);
            p.second_fenced(nx, fa, acc, sf, smem, s, kl);
        } else {
            sf.issue(smem, s, kl);
            p.second(nx, fa, acc);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();
    __syncthreads();
}

// Reads one accumulator out of its AGPR where it is used (4 waves: 256 accumulators per lane,
// in AGPRs).  Without this the compiler copies all of them into VGPRs at the loop exit (the
// conversions below cannot read AGPRs), which does not fit next to the epilogue's registers.
__device__ __forceinline__ float acc_read(float a) {
    if constexpr (kWaves == 4) {
        float v;
        asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
        return v;
    } else {
        return a;   // 128 accumulators per lane: they stay in VGPRs
    }
}

// Epilogue phase 1: tile[row][col] = bf16((acc * rowscale[row]) * colscale[col]) into LDS
// (row pitch kEpiPitch); with scales the products are formed in double and rounded once.
// Accumulator layout of the 32x32 MFMA: lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4
// and column l%32 of its block.  rowscale and colscale are both given or both null (factor 1).
// Must follow a barrier that ends all LDS reads of the main loop.
__device__ __forceinline__ void stage_tile_bf16(const f32x16 (&acc)[4][kNB], uint8_t* smem, const float* rowscale,
                                                int64_t m0, int64_t M, const float* colscale_lo,
                                                const float* colscale_hi) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / kWN, wn = wave % kWN;
    const int r32 = lane & 31, hi = lane >> 5;
    float cscale[kNB];
#pragma unroll
    for (int j = 0; j < kNB; ++j) cscale[j] = 1.f;
    if (colscale_lo) {
        // local columns [0,128) come from colscale_lo, [128,256) from colscale_hi
        const int c0 = wn * kWaveN;
        const float* cs = c0 < 128 ? colscale_lo + c0 : colscale_hi + (c0 - 128);
#pragma unroll
        for (int j = 0; j < kNB; ++j) cscale[j] = cs[j * 32 + r32];
    }
    // one 32x32 block at a time (the scheduling barrier keeps the compiler from pulling all
    // 256 accumulators into VGPRs at once)
    // row scales of block row i + 1 are loaded while block row i converts
    auto load_rs = [&](int i, float (&rs)[16]) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            int64_t gm = m0 + wm * 128 + i * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
            gm = gm < M ? gm : M - 1;
            rs[r] = rowscale[gm];
        }
    };
    float rs[16], rs_nx[16];
    if (rowscale) load_rs(0, rs);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (rowscale && i + 1 < 4) load_rs(i + 1, rs_nx);
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
            const int col = wn * kWaveN + j * 32 + r32;
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
        if (rowscale) {
#pragma unroll
            for (int r = 0; r < 16; ++r) rs[r] = rs_nx[r];
        }
    }
}

__device__ __forceinline__ u32x4 epi_ld(const uint8_t* smem, int row, int col) {
    return *reinterpret_cast<const u32x4*>(smem + row * kEpiPitch + col * 2);
}

}  // namespace gemm
}  // namespace dit
