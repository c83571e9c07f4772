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
// instructions); A and B each rotate through a ring of LDS slots, and the loads of a stage
// are issued as soon as its slots are released.
//
// Per stage:
//   first : the MFMAs of all k-steps but the last, each interleaved with the LDS reads of
//           the next k-step's fragments (fragments double-buffered in registers);
//   wait for the next stage's loads (vmcnt) and this wave's LDS reads, barrier;
//   issue the loads of the stages one ring depth ahead into the slots just released;
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
constexpr int kOpBytes = 256 * kRowB;           // one operand of one stage (an LDS slot)
#ifndef DIT_GEMM_STAGES
#define DIT_GEMM_STAGES (kRowB == 64 ? 4 : 2)
#endif
// A and B each rotate through their own ring of LDS slots; a ring of depth S keeps S - 1
// stages of that operand in flight.
#ifndef DIT_GEMM_STAGES_A
#define DIT_GEMM_STAGES_A DIT_GEMM_STAGES
#endif
#ifndef DIT_GEMM_STAGES_B
#define DIT_GEMM_STAGES_B DIT_GEMM_STAGES
#endif
constexpr int kStagesA = DIT_GEMM_STAGES_A;
constexpr int kStagesB = DIT_GEMM_STAGES_B;
static_assert(kStagesA >= 2 && kStagesB >= 2, "ring depth");
constexpr int kBRing = kStagesA * kOpBytes;     // LDS offset of the B ring
constexpr int kMainBytes = (kStagesA + kStagesB) * kOpBytes;
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
// Within a stage's loads, the operand with the shallower ring goes first: the stage barrier
// then waits for it while the deeper ring's newest stage may still be in flight.
constexpr bool kBFirst = kStagesB < kStagesA;
struct StageFill {
    __amdgpu_buffer_rsrc_t ra, rb;
    uint32_t va[kPieces];    // A: row + chunk offset of piece j (per lane; bounds-checked)
    uint32_t vb[kVPat];      // B: row-in-piece + chunk offset, by piece parity (per lane)
    uint32_t sb[kPieces];    // B: offset of piece j's first row (uniform)
    uint32_t lds_w;          // this wave's slice within an operand
    __device__ __forceinline__ void a_piece(uint8_t* smem, int slot, int kt, int j) const {
        lds_u8* S = (lds_u8*)smem + slot * kOpBytes + lds_w;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, S + j * 1024, 16, (int)va[j], kt * kRowB, 0, kLoadAux);
    }
    __device__ __forceinline__ void b_piece(uint8_t* smem, int slot, int kt, int j) const {
        lds_u8* S = (lds_u8*)smem + kBRing + slot * kOpBytes + lds_w;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, S + j * 1024, 16, (int)vb[j % kVPat], (int)sb[j] + kt * kRowB,
                                                 0, kLoadAux);
    }
    // load j of one step of the fill: stage kta of A into A slot `as`, stage ktb of B into
    // B slot `bs` (with kSkip, a negative kta / ktb skips that operand: prologue only, where
    // the step is a compile-time constant)
    template <bool kSkip = false>
    __device__ __forceinline__ void one(uint8_t* smem, int as, int kta, int bs, int ktb, int j) const {
        const bool first = j < kPieces;
        const int jj = first ? j : j - kPieces;
        if (first != kBFirst) {
            if (!kSkip || kta >= 0) a_piece(smem, as, kta, jj);
        } else {
            if (!kSkip || ktb >= 0) b_piece(smem, bs, ktb, jj);
        }
    }
    template <bool kSkip = false>
    __device__ __forceinline__ void issue(uint8_t* smem, int as, int kta, int bs, int ktb) const {
#pragma unroll
        for (int j = 0; j < kLoadsPerStage; ++j) one<kSkip>(smem, as, kta, bs, ktb, j);
    }
};

// The LDS slots holding one stage of A and of B.
struct Stage {
    const uint8_t* a;
    const uint8_t* b;
};
// One step of the fill: stage kta of A into A slot `as`, stage ktb of B into B slot `bs`.
struct FillStep {
    int as, kta, bs, ktb;
};

// Per-lane LDS offsets of the fragment reads (relative to an operand slot).  Lane l reads row
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
            b[q] = (uint32_t)((wn * kWaveN + r32) * kRowB + ((c ^ sw) << 4));
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

// Load accounting.  Fill step i (issued at the hand-over of main-loop iteration i, or as a
// virtual step i < 0 in the prologue) loads stage i + S_A of A and i + S_B of B, the
// shallower ring's operand first (F, ring depth S_F; the other is G, depth S_G >= S_F).  The
// hand-over of iteration kt needs stage kt + 1 of both, issued in steps kt + 1 - S_F and
// kt + 1 - S_G; loads complete in issue order, so the vmcnt limit is the number of loads
// issued after the younger of the two: the G half of step kt + 1 - S_F and steps
// kt + 2 - S_F .. kt - 1 in full (or, for G, steps kt + 2 - S_G .. kt - 1).
constexpr int kSF = kStagesA < kStagesB ? kStagesA : kStagesB;
constexpr int kSG = kStagesA < kStagesB ? kStagesB : kStagesA;
constexpr int kVmF = kPieces + (kSF - 2) * kLoadsPerStage;
constexpr int kVmG = (kSG - 2) * kLoadsPerStage;
constexpr int kVmSteady = kVmF < kVmG ? kVmF : kVmG;
// Before iteration 0 the prologue (steps -S_G .. -1, each with the loads whose stage is
// >= 0) has to have landed stage 0: after F's stage 0 come the G half of step -S_F and
// steps -S_F + 1 .. -1 in full; after G's stage 0 come, in steps -S_G + 1 .. -1, every G
// load and the F loads of the steps >= -S_F.
constexpr int kVmPrologueF = kPieces + (kSF - 1) * kLoadsPerStage;
constexpr int kVmPrologueG = (kSG - 1) * kPieces + (kSF < kSG - 1 ? kSF : kSG - 1) * kPieces;
constexpr int kVmPrologue = kVmPrologueF < kVmPrologueG ? kVmPrologueF : kVmPrologueG;
static_assert(kVmSteady < 64 && kVmPrologue < 64, "vmcnt range");

// Stage hand-over: this wave's LDS reads of the stage it is leaving have landed (lgkmcnt 0:
// after the barrier other waves refill those slots by DMA), its loads of the next stage have
// landed (vmcnt), then the workgroup barrier makes every wave's fill visible.
__device__ __forceinline__ void stage_barrier() {
    constexpr int kVm = kVmSteady;
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
    __device__ __forceinline__ void read(const Stage& st, const FragAddr& fa, int ks, int h) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[h][i] = lds_bf16x8(st.a, fa.a[ks] + i * kBlk);
#pragma unroll
        for (int j = 0; j < kNB; ++j) b[h][j] = lds_bf16x8(st.b, fa.b[ks] + j * kBlk);
    }
    __device__ __forceinline__ void mma(int h, f32x16 (&acc)[4][kNB]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < kNB; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[h][i], b[h][j], acc[i][j], 0, 0, 0);
    }
    // fragment f of k-step ks into buffer h: A blocks 0..3, then B blocks 0..kNB-1
    __device__ __forceinline__ void read_one(const Stage& st, const FragAddr& fa, int ks, int h, int f) {
        if (f < 4) a[h][f] = lds_bf16x8(st.a, fa.a[ks] + f * kBlk);
        else b[h][f - 4] = lds_bf16x8(st.b, fa.b[ks] + (f - 4) * kBlk);
    }
    __device__ __forceinline__ void mma_one(int h, int i, f32x16 (&acc)[4][kNB]) {
        const int bi = i / kNB, bj = i % kNB;
        acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[h][bi], b[h][bj], acc[bi][bj], 0, 0, 0);
    }
    __device__ __forceinline__ void prime(const Stage& st, const FragAddr& fa) { read(st, fa, 0, 0); }
    __device__ __forceinline__ void first(const Stage& st, const FragAddr& fa, f32x16 (&acc)[4][kNB]) {
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
    __device__ __forceinline__ void second_fenced(const Stage& next, const FragAddr& fa, f32x16 (&acc)[4][kNB],
                                                  const StageFill& sf, uint8_t* smem, const FillStep& fs) {
        static_assert(kLoadsPerStage <= F && R <= F, "slots");
#pragma unroll
        for (int i = 0; i < F; ++i) {
            if (i < kLoadsPerStage) sf.one(smem, fs.as, fs.kta, fs.bs, fs.ktb, i);
            if (i < R) read_one(next, fa, 0, KS & 1, i);
            mma_one((KS - 1) & 1, i, acc);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __device__ __forceinline__ void second(const Stage& next, const FragAddr& fa, f32x16 (&acc)[4][kNB]) {
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
template <int kW = kWaves>
struct PipeFp8Impl {
    static_assert(kW == 4, "the 64-byte-row e4m3 pipeline is written for 4 waves");
    i32x8 a[4], b[4];
    __device__ __forceinline__ void read_a(const Stage& st, const FragAddr& fa, int i) {
        a[i] = lds_i32x8(st.a, fa.a[0] + i * kBlk, fa.a[1] + i * kBlk);
    }
    __device__ __forceinline__ void read_b(const Stage& st, const FragAddr& fa, int j) {
        b[j] = lds_i32x8(st.b, fa.b[0] + j * kBlk, fa.b[1] + j * kBlk);
    }
    __device__ __forceinline__ void mma(int i, int j, f32x16 (&acc)[4][4]) {
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 0, 0, 0, 0, 0, 0);
    }
    __device__ __forceinline__ void prime(const Stage& st, const FragAddr& fa) {
#pragma unroll
        for (int i = 0; i < 2; ++i) read_a(st, fa, i);
#pragma unroll
        for (int j = 0; j < 4; ++j) read_b(st, fa, j);
    }
    __device__ __forceinline__ void first(const Stage& st, const FragAddr& fa, f32x16 (&acc)[4][4]) {
        read_a(st, fa, 2);
        read_a(st, fa, 3);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) mma(i, j, acc);
        interleave_ds_mfma<4, 2>();
    }
    __device__ __forceinline__ void second(const Stage& next, const FragAddr& fa, f32x16 (&acc)[4][4]) {
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
    __device__ __forceinline__ void read(const Stage& st, const FragAddr& fa, int ks, int h) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[h][i] = lds_i32x8(st.a, fa.a[2 * ks] + i * kBlk, fa.a[2 * ks + 1] + i * kBlk);
#pragma unroll
        for (int j = 0; j < kNB; ++j) b[h][j] = lds_i32x8(st.b, fa.b[2 * ks] + j * kBlk, fa.b[2 * ks + 1] + j * kBlk);
    }
    __device__ __forceinline__ void mma(int h, f32x16 (&acc)[4][kNB]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < kNB; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[h][i], b[h][j], acc[i][j], 0, 0, 0, 0,
                                                                             0, 0);
    }
    __device__ __forceinline__ void read_one(const Stage& st, const FragAddr& fa, int ks, int h, int f) {
        if (f < 4) a[h][f] = lds_i32x8(st.a, fa.a[2 * ks] + f * kBlk, fa.a[2 * ks + 1] + f * kBlk);
        else b[h][f - 4] = lds_i32x8(st.b, fa.b[2 * ks] + (f - 4) * kBlk, fa.b[2 * ks + 1] + (f - 4) * kBlk);
    }
    __device__ __forceinline__ void mma_one(int h, int i, f32x16 (&acc)[4][kNB]) {
        const int bi = i / kNB, bj = i % kNB;
        acc[bi][bj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[h][bi], b[h][bj], acc[bi][bj], 0, 0, 0, 0,
                                                                       0, 0);
    }
    // as in the bf16 pipeline: fill load i, fragment i of the next stage's k-step 0, MFMA i
    __device__ __forceinline__ void second_fenced(const Stage& next, const FragAddr& fa, f32x16 (&acc)[4][kNB],
                                                  const StageFill& sf, uint8_t* smem, const FillStep& fs) {
        static_assert(kLoadsPerStage <= F && 4 + kNB <= F, "slots");
#pragma unroll
        for (int i = 0; i < F; ++i) {
            if (i < kLoadsPerStage) sf.one(smem, fs.as, fs.kta, fs.bs, fs.ktb, i);
            if (i < 4 + kNB) read_one(next, fa, 0, 0, i);
            mma_one(1, i, acc);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __device__ __forceinline__ void prime(const Stage& st, const FragAddr& fa) { read(st, fa, 0, 0); }
    __device__ __forceinline__ void first(const Stage& st, const FragAddr& fa, f32x16 (&acc)[4][kNB]) {
        read(st, fa, 1, 1);
        mma(0, acc);
        if constexpr (kWaves == 4) {
            interleave_ds_mfma<16, 1>();
        } else {
            interleave_ksteps<1, R, F>();
        }
    }
    __device__ __forceinline__ void second(const Stage& next, const FragAddr& fa, f32x16 (&acc)[4][kNB]) {
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

using PipeFp8 = PipeFp8Impl<>;

template <bool kFp8>
struct PipeOf {
    using type = PipeBf16;
};
template <>
struct PipeOf<true> {
    using type = typename std::conditional<kRowB == 64, PipeFp8, PipeFp8K2>::type;
};

// Interleaved main loop (every wave fills, reads and multiplies within each stage); the
// 4-wave layout and 64-byte stage rows use it.
template <bool kFp8>
__device__ __forceinline__ void mainloop_interleaved(const uint8_t* __restrict__ A, int64_t lda, int64_t m0, int64_t M,
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

    // prologue: fill steps -S_G .. -1 (every slot of both rings in flight), wait for stage 0
    auto step = [&](int i) -> FillStep {
        const int ka = i + kStagesA, kb = i + kStagesB;
        FillStep f;
        f.as = (i + kStagesA) % kStagesA;
        f.bs = (i + kStagesB) % kStagesB;
        f.kta = ka < 0 ? -1 : (ka < ktiles ? ka : ktiles - 1);
        f.ktb = kb < 0 ? -1 : (kb < ktiles ? kb : ktiles - 1);
        return f;
    };
#pragma unroll
    for (int i = -kSG; i < 0; ++i) {
        const FillStep f = step(i);
        sf.issue<true>(smem, f.as, f.kta, f.bs, f.ktb);
    }
    wait_vmcnt<kVmPrologue>();
    __syncthreads();

    auto slots = [&](int kt) -> Stage {
        return Stage{smem + (kt % kStagesA) * kOpBytes, smem + kBRing + (kt % kStagesB) * kOpBytes};
    };
    typename PipeOf<kFp8>::type p;
    p.prime(slots(0), fa);
    for (int kt = 0; kt < ktiles; ++kt) {
        const Stage st = slots(kt);
        const Stage nx = slots(kt + 1);
        __builtin_amdgcn_sched_barrier(0);
        p.first(st, fa, acc);
        __builtin_amdgcn_sched_barrier(0);
        stage_barrier();
        const FillStep f = step(kt);
        if constexpr (kWaves == 8) {
            __builtin_amdgcn_sched_barrier(0);
            p.second_fenced(nx, fa, acc, sf, smem, f);
        } else {
            sf.issue(smem, f.as, f.kta, f.bs, f.ktb);
            p.second(nx, fa, acc);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();
    __syncthreads();
}

// ---------------------------------------------------------------------------------------
// Ping-pong main loop (8 waves, 128-byte stage rows, two slots per operand).
//
// Group G0 = waves 0-3 (tile rows 0-127) and group G1 = waves 4-7 (rows 128-255); waves w
// and w + 4 share a SIMD.  Each wave alternates a memory phase (read every fragment of one
// stage from LDS into registers) and a compute phase (that stage's MFMAs, from registers
// only).  G1 runs one phase behind G0, so on every SIMD one wave issues MFMAs back to back
// while the other waits on LDS; a workgroup barrier ends every phase.  G1 enters one extra
// barrier before its first phase and G0 one after its last, so both groups pass the same
// number of barriers.
//
// Phase 2s: G0 memory(s), G1 compute(s-1).  Phase 2s+1: G0 compute(s), G1 memory(s).
// Stage s sits in slot s % 2.  All fill loads are issued in memory phases (a compute phase
// is MFMAs only: a wave issues in order, so a fill load that waits for the memory pipeline
// would hold back the MFMAs behind it), and every wave refills only rows whose readers are
// done:
//   A rows 0-127 are read by G0 alone: at the start of its memory phase for stage s, G0 wave
//     w refills rows 32w.. of the other slot (stage s-1, read in its previous memory phase)
//     with stage s+1;
//   A rows 128-255 likewise by G1, at the start of its memory phase for stage s;
//   B rows 64c.. are read by waves c and 4+c only: G1 wave 4+c refills them in its slot of
//     stage s with stage s+2 at the end of its memory phase for s, once its own reads have
//     landed (wave c read them a phase earlier).
// Each group waits for its A rows of stage s+1 before the barrier that ends its compute phase
// for s, and G1 for the B rows of stage s+1 before the barrier that ends its memory phase for
// s; those are the last barriers before the first reads.  Loads for stages past the end go
// through a zero-length descriptor (no memory read, zeros into a slot with no reader left),
// so every phase issues the same loads and the vmcnt limits hold throughout.
constexpr int kPPAPieces = 32 / kRowsPerPiece;      // A: 32 rows per wave
constexpr int kPPBPieces = 64 / kRowsPerPiece;      // B: 64 rows per G1 wave

struct PPFill {
    __amdgpu_buffer_rsrc_t ra, rb;
    __amdgpu_buffer_rsrc_t rnull;   // zero records: every load through it is out of range
    uint32_t va[kPPAPieces];  // A: row + chunk offset of piece j (per lane; bounds-checked)
    uint32_t vb[kVPat];       // B: row-in-piece + chunk offset, by piece parity (per lane)
    uint32_t sb[kPPBPieces];  // B: offset of piece j's first row (uniform)
    uint32_t lds_a, lds_b;    // this wave's rows within an A slot / a B slot
    // Stage kt of this wave's rows into `slot`.  A load past the last stage (live false) goes
    // through rnull: it reads no memory and writes zeros into a slot that has no reader left,
    // but still counts in vmcnt, so every phase issues the same number of loads.
    __device__ __forceinline__ void a_rows(uint8_t* smem, int slot, int kt, bool live) const {
        lds_u8* S = (lds_u8*)smem + slot * kOpBytes + lds_a;
        const __amdgpu_buffer_rsrc_t r = live ? ra : rnull;
#pragma unroll
        for (int j = 0; j < kPPAPieces; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, S + j * 1024, 16, (int)va[j], kt * kRowB, 0, kLoadAux);
    }
    __device__ __forceinline__ void b_rows(uint8_t* smem, int slot, int kt, bool live) const {
        lds_u8* S = (lds_u8*)smem + 2 * kOpBytes + slot * kOpBytes + lds_b;
        const __amdgpu_buffer_rsrc_t r = live ? rb : rnull;
#pragma unroll
        for (int j = 0; j < kPPBPieces; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, S + j * 1024, 16, (int)vb[j % kVPat], (int)sb[j] + kt * kRowB,
                                                     0, kLoadAux);
    }
};

// Every fragment of one stage in registers: bf16 has kRowB/32 k-steps of 16, e4m3 kRowB/64
// k-steps of 64 (each fragment then two 16-byte reads).
template <bool kFp8>
struct PPFrags;
template <>
struct PPFrags<false> {
    static constexpr int KS = kRowB / 32;
    bf16x8 a[KS][4], b[KS][kNB];
    __device__ __forceinline__ void read(const Stage& st, const FragAddr& fa) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int i = 0; i < 4; ++i) a[ks][i] = lds_bf16x8(st.a, fa.a[ks] + i * kBlk);
#pragma unroll
            for (int j = 0; j < kNB; ++j) b[ks][j] = lds_bf16x8(st.b, fa.b[ks] + j * kBlk);
        }
    }
    __device__ __forceinline__ void mma(f32x16 (&acc)[4][kNB]) const {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < kNB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks][i], b[ks][j], acc[i][j], 0, 0, 0);
    }
};
template <>
struct PPFrags<true> {
    static constexpr int KS = kRowB / 64;
    i32x8 a[KS][4], b[KS][kNB];
    __device__ __forceinline__ void read(const Stage& st, const FragAddr& fa) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int i = 0; i < 4; ++i) a[ks][i] = lds_i32x8(st.a, fa.a[2 * ks] + i * kBlk, fa.a[2 * ks + 1] + i * kBlk);
#pragma unroll
            for (int j = 0; j < kNB; ++j)
                b[ks][j] = lds_i32x8(st.b, fa.b[2 * ks] + j * kBlk, fa.b[2 * ks + 1] + j * kBlk);
        }
    }
    __device__ __forceinline__ void mma(f32x16 (&acc)[4][kNB]) const {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < kNB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[ks][i], b[ks][j], acc[i][j], 0, 0, 0,
                                                                                 0, 0, 0);
    }
};

// Phase-ending barrier: wait for vmcnt(kVm) and lgkmcnt(0), then a bare s_barrier.  These
// waits are all the hand-over needs, so younger fill loads stay in flight across it (the
// __syncthreads() fence would drain them).  The asm's memory clobber keeps the compiler from
// moving memory accesses across the barrier.
template <int kVm>
__device__ __forceinline__ void pp_barrier() {
    static_assert(kVm >= 0 && kVm < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((kVm & 15) | ((kVm >> 4) << 14) | (7 << 4) | (0 << 8));
    asm volatile("s_barrier" ::: "memory");
}

template <bool kFp8>
__device__ __forceinline__ void mainloop_pp(const uint8_t* __restrict__ A, int64_t lda, int64_t m0, int64_t M,
                                            const uint8_t* __restrict__ B, int64_t ldb, int64_t nb0, int64_t nb1,
                                            int ktiles, uint8_t* smem, f32x16 (&acc)[4][kNB]) {
    static_assert(kWaves == 8 && kRowB == 128, "ping-pong layout");
    static_assert(4 * kOpBytes <= kSmemBytes, "two slots per operand");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
    const bool g0 = wave < 4;
    const int c = wave & 3;                          // B rows 64c.. (G1 fills them)
    PPFill sf;
    const int64_t arows = M - m0 < kBM ? M - m0 : kBM;
    sf.ra = make_rsrc(A + m0 * lda, (uint32_t)(arows * lda));
    sf.rb = make_rsrc(B + nb0 * ldb, (uint32_t)((nb1 - nb0 + 128) * ldb));
    sf.rnull = make_rsrc(B, 0u);
#pragma unroll
    for (int j = 0; j < kPPAPieces; ++j) {
        const int row = 32 * wave + j * kRowsPerPiece + lane / kSlots;
        sf.va[j] = (uint32_t)(row * lda) + (uint32_t)(((lane % kSlots) ^ swz(row)) << 4);
    }
#pragma unroll
    for (int j = 0; j < kPPBPieces; ++j) {
        const int64_t r0 = 64 * c + j * kRowsPerPiece;               // piece's first row (uniform)
        sf.sb[j] = (uint32_t)((r0 < 128 ? r0 : r0 + (nb1 - nb0 - 128)) * ldb);
        if (j < kVPat) {
            const int row = (int)r0 + lane / kSlots;
            sf.vb[j] = (uint32_t)((lane / kSlots) * ldb) + (uint32_t)(((lane % kSlots) ^ swz(row)) << 4);
        }
    }
    sf.lds_a = (uint32_t)(32 * wave * kRowB);
    sf.lds_b = (uint32_t)(64 * c * kRowB);
    FragAddr fa;
    fa.init(kFp8);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    auto slot = [&](int kt) -> Stage {
        const int s = kt & 1;
        return Stage{smem + s * kOpBytes, smem + 2 * kOpBytes + s * kOpBytes};
    };
    PPFrags<kFp8> fr;

    // prologue: A of stage 0 (each wave its rows), B of stages 0 and 1 (G1).  Only stage 0 must
    // have landed here; B of stage 1 is first read in phase 2, after G1's memory-phase barrier
    // (whose vmcnt limit counts only younger loads).
    sf.a_rows(smem, 0, 0, true);
    if (!g0) {
        sf.b_rows(smem, 0, 0, true);
        sf.b_rows(smem, 1, 1, ktiles > 1);
        pp_barrier<kPPBPieces>();
        pp_barrier<63>();            // G1 starts one phase behind
    } else {
        pp_barrier<0>();
    }
    for (int kt = 0; kt < ktiles; ++kt) {
        const int s = kt & 1;
        // memory phase.  First this wave's A rows of stage kt+1 into the other slot: its
        // group read them (stage kt-1) in its last memory phase.
        __builtin_amdgcn_sched_barrier(0);
        sf.a_rows(smem, s ^ 1, kt + 1, kt + 1 < ktiles);
        __builtin_amdgcn_sched_barrier(0);
        fr.read(slot(kt), fa);
        __builtin_amdgcn_sched_barrier(0);
        if (g0) {
            pp_barrier<63>();
        } else {
            // B rows 64c.. of this slot, stage kt+2: the partner G0 wave read them in the
            // last phase, this wave's reads land here
            __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));    // lgkmcnt(0)
            sf.b_rows(smem, s, kt + 2, kt + 2 < ktiles);
            // landed: B of stage kt+1 (issued before the A rows and B rows of this phase)
            pp_barrier<kPPAPieces + kPPBPieces>();
        }
        // compute phase: MFMAs only
        __builtin_amdgcn_sched_barrier(0);
        fr.mma(acc);
        __builtin_amdgcn_sched_barrier(0);
        if (g0) {
            pp_barrier<0>();                 // G0: A rows of stage kt+1 landed
        } else {
            pp_barrier<kPPBPieces>();        // G1: A rows of stage kt+1 landed (B of kt+2 may fly)
        }
    }
    if (g0) pp_barrier<63>();        // G1's last compute phase
    __syncthreads();
}

// Main loop over `ktiles` stages of K.  A rows m0.. (rows past M read as zero), B local rows
// [0,128) are global rows nb0.., local rows [128,256) are nb1.. (nb1 = nb0 + 128 for a
// plain tile).  Ends with all loads drained and a barrier, so the caller may reuse the LDS.
#ifndef DIT_GEMM_PINGPONG
#define DIT_GEMM_PINGPONG (kWaves == 8 && kRowB == 128)
#endif
template <bool kFp8>
__device__ __forceinline__ void mainloop(const uint8_t* __restrict__ A, int64_t lda, int64_t m0, int64_t M,
                                         const uint8_t* __restrict__ B, int64_t ldb, int64_t nb0, int64_t nb1,
                                         int ktiles, uint8_t* smem, f32x16 (&acc)[4][kNB]) {
    if constexpr (DIT_GEMM_PINGPONG) {
        mainloop_pp<kFp8>(A, lda, m0, M, B, ldb, nb0, nb1, ktiles, smem, acc);
    } else {
        mainloop_interleaved<kFp8>(A, lda, m0, M, B, ldb, nb0, nb1, ktiles, smem, acc);
    }
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
// (row pitch kEpiPitch); with scales the product of the three fp32 values is rounded once.
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
            for (int r = 0; r < 16; r += 2) {
                // registers r and r + 1 hold rows R and R + 1 of the column
                const int row = wm * 128 + i * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
                const float a0 = acc_read(acc[i][j][r]), a1 = acc_read(acc[i][j][r + 1]);
                uint32_t b;
                if (rowscale) {
                    // (acc * s_row) * s_col, one rounding to bf16
                    b = pack_bf2(mul3_odd32(a0, rs[r], cscale[j]), mul3_odd32(a1, rs[r + 1], cscale[j]));
                } else {
                    b = pack_bf2(a0, a1);
                }
                *reinterpret_cast<uint16_t*>(smem + row * kEpiPitch + col * 2) = (uint16_t)b;
                *reinterpret_cast<uint16_t*>(smem + (row + 1) * kEpiPitch + col * 2) = (uint16_t)(b >> 16);
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
