// Tiled MFMA GEMM core for gfx950 shared by the QKV, out-projection, FC1 and FC2 kernels.
//
// C[m, n] = sum_k A[m, k] * B[n, k]: both operands are K-contiguous rows (activations
// [M, K], weights [N, K]), FP32 accumulation.
//
// Workgroup: 8 waves, two per SIMD, and one 256 x 256 output tile; each wave owns a 128 x 64
// wave tile, or 64 x 128 (128 FP32 accumulators per lane, so a wave fits in 256 registers):
//   bf16:  8 x 4 blocks of 16 x 16, v_mfma_f32_16x16x32_bf16, two k-steps per stage;
//   e4m3:  8 x 4 blocks of 16 x 16, v_mfma_f32_16x16x128_f8f6f4 (the scaled builtin with zero
//          scale operands, which the compiler emits as the unscaled instruction), one k-step per
//          stage;
//   mxfp4: 4 x 2 blocks of 32 x 32, v_mfma_scale_f32_32x32x64_f8f6f4 on E2M1 operands with
//          their E8M0 block scales, four k-steps per stage.
// Under a full-chip load the shader clock is set by power.  For the same MACs the 16x16 forms
// move fewer register bytes than the 32x32 ones (bf16: operands plus accumulator read and
// write, 0.5 against 0.625 bytes per MAC), and a register-only MFMA loop sustains about 12%
// (bf16) and 7% (e4m3) more FLOP/s with them.  The scaled MFMA is the exception: while one
// wave of a SIMD issues the 16x16x128 scaled form, the other wave's fill and LDS-read
// instructions issue at about half their usual rate (a memory phase of ~1430 cycles against
// ~980), and the 32x32x64 form, half as many instructions for the same work, removes that.
// A and B fragments take their k values from the same (lane group, byte) positions, so the
// product is the same whatever order the instruction assigns to k inside a fragment.
//
// K is consumed in stages of 128 bytes per row (64 bf16, 128 e4m3 or 256 E2M1, one cache
// line).  Each stage (A 256 rows + B 256 rows) is filled straight from global memory into LDS
// by buffer_load_dwordx4 ... lds (no register staging, no LDS store instructions), into two A
// slots and a ring of three B slots.  Rows of A past M read as zeros (buffer descriptor bound)
// and are never stored.
#pragma once

#include "common.hpp"

namespace dit {
namespace gemm {

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kRowB = 128;                      // bytes of K per row per stage
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kWN = 4;                          // waves across n (two across m)
constexpr int kWaveN = kBN / kWN;               // wave tile: 128 rows x 64 columns
constexpr int kOpBytes = 256 * kRowB;           // one operand of one stage (an LDS slot)
constexpr int kEpiPitch = kBN * 2 + 16;         // bf16 epilogue tile, padded row pitch (bytes)
constexpr int kEpiBytes = kBM * kEpiPitch;      // 132 KiB
// main loop: two A slots and a ring of three B slots, all of gfx950's 160 KiB of LDS
constexpr int kMainBytes = 5 * kOpBytes;
constexpr int kSmemBytes = kMainBytes > kEpiBytes ? kMainBytes : kEpiBytes;
constexpr int kSlots = kRowB / 16;              // 16-byte chunks per row
constexpr int kRowsPerPiece = 1024 / kRowB;     // rows filled by one 1 KiB wave load

// LDS layout of an operand within a stage: row r (0..255) holds 8 chunks of 16 bytes; chunk
// c of row r sits at r * 128 + ((c ^ swz(r)) * 16), swz(r) = (r / 2) % 8.  An MFMA operand
// read has 16 lanes on 16 consecutive rows and one chunk, which then land in 16 distinct
// 16-byte bank groups of the 64-bank LDS.  Fills are 64 lanes writing 1 KiB contiguously,
// conflict-free.
__host__ __device__ constexpr int swz(int r) { return (r >> 1) & 7; }

// What the operands hold: bf16 values, e4m3 codes, or MXFP4 (E2M1 codes, two per byte, with
// E8M0 scales of 32-value blocks in the MX scale layout below).
enum class Mma { kBf16, kE4m3, kMxFp4 };

// MX scale layout.  For a matrix of R rows (padded to a multiple of 128) and K values per row
// (a multiple of 256), the E8M0 scale of row r, block b (values 32 b .. 32 b + 31) is the byte
//   ((r / 128) (K / 256) + b / 8) 1024 + 16 l + 4 ((r % 128) / 32) + (b % 8) / 2,
//   l = r % 32 + 32 (b % 2).
// So each 128 rows x 256 values (one GEMM stage of a wave-row of 128) own 1 KiB, in which lane
// l's 16 bytes are the scales it hands the MFMA: the 32x32x64 instruction takes the scale of
// row l % 32 and block l / 32 of a 32 x 64 operand from lane l; register I of the four holds
// the 32-row block I, byte q the stage's k-step q.

// Logical tile order -> (m tile, n tile): groups of 4 m-tiles across all n-tiles, m fastest.
__device__ __forceinline__ void logical_coords(int L, int mt, int nt, int& tm, int& tn) {
    constexpr int GM = 4;
    const int group = L / (GM * nt);
    const int first_m = group * GM;
    const int gsize = (mt - first_m) < GM ? (mt - first_m) : GM;
    const int in = L - group * GM * nt;
    tm = first_m + in % gsize;
    tn = in / gsize;
}

// Workgroup id -> (m tile, n tile) for a launch of one workgroup per tile.  Workgroups are
// dispatched round-robin over the 8 XCDs, so id % 8 names the XCD: each XCD gets one contiguous
// range of the logical order, and the ~32 tiles an XCD runs at once share 4 A panels and 8 B
// panels in its L2.
constexpr int kXcds = 8;
__device__ __forceinline__ void xcd_range(int xcd, int G, int& lo, int& cnt) {
    const int per = G / kXcds, rem = G % kXcds;
    lo = xcd * per + (xcd < rem ? xcd : rem);
    cnt = per + (xcd < rem ? 1 : 0);
}
__device__ __forceinline__ void tile_coords(int bid, int mt, int nt, int& tm, int& tn) {
    int lo, cnt;
    xcd_range(bid % kXcds, mt * nt, lo, cnt);
    logical_coords(lo + bid / kXcds, mt, nt, tm, tn);
}

// Persistent launches: one workgroup per CU, which runs tile after tile.  Workgroup b runs on
// XCD b % 8 (the dispatcher's round robin), and the workgroups of an XCD claim the tiles of the
// same contiguous range of the logical order as above one at a time, from a counter of that
// XCD: a tile keeps its place in the order (and the L2 window with it), and the CUs of an XCD
// balance their work among themselves.  The counters (one per XCD, zero when the launch
// starts) are claimed by one lane with a global atomic add; the index reaches the other waves
// through an LDS word just past the staged epilogue tile, which no main loop or epilogue holds
// at the two points it is used: after the main loop (claim) and after the epilogue's closing
// barrier (read).  A counter set is kTileQueueWords words: the kXcds tile counters, a count of
// finished workgroups and, from kReadyBase, the ready counters of a launch that hands work
// between its workgroups (the fused FC2).  The workgroup that finishes last puts the set back to
// zero for its next launch (finish()): every other workgroup has made its last claim, and read
// its last ready counter, before it counted itself finished.
constexpr int kReadyBase = 16;
constexpr int kMaxReady = 144;
constexpr int kTileQueueWords = kReadyBase + kMaxReady;
struct TileQueue {
    uint32_t* set;     // the launch's counter set
    uint32_t* ctr;     // this XCD's counter
    int xcd;           // the XCD (range) this workgroup works on: blockIdx.x % kXcds
    int lo, cnt;       // this XCD's range of the logical order
    __device__ __forceinline__ TileQueue(uint32_t* counters, int mt, int nt) {
        xcd = (int)(blockIdx.x % kXcds);
        set = counters;
        ctr = counters + xcd;
        xcd_range(xcd, mt * nt, lo, cnt);
    }
    // after the workgroup's last claim: count it finished; the last one zeroes the set (the tile
    // counters, the finished count and the first nready ready counters)
    __device__ __forceinline__ void finish(int nready = 0) const {
        if (threadIdx.x == 0 && atomicAdd(set + kXcds, 1u) == gridDim.x - 1) {
#pragma unroll
            for (int i = 0; i <= kXcds; ++i) __hip_atomic_store(set + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int i = 0; i < nready; ++i)
                __hip_atomic_store(set + kReadyBase + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    static __device__ __forceinline__ uint32_t* slot(uint8_t* smem) {
        return reinterpret_cast<uint32_t*>(smem + kEpiBytes);
    }
    // thread 0 claims the next index (the caller's LDS use must leave the slot free)
    __device__ __forceinline__ void claim(uint8_t* smem) const {
        if (threadIdx.x == 0) *slot(smem) = atomicAdd(ctr, 1u);
    }
    // the index claimed last, after a barrier that follows claim()
    __device__ __forceinline__ int claimed(uint8_t* smem) const {
        return __builtin_amdgcn_readfirstlane((int)*slot(smem));
    }
    // The claim of persistent_tiles: thread 0 marks the slot empty once the tile's main loop no
    // longer writes it (mark_empty) and, past a barrier, claims into it (claim_wait); the waves
    // wait on the slot itself, not on a barrier, for the claimed index (wait_claimed).  A counter
    // never reaches kEmpty (it grows by at most one per claim past its range's length).
    static constexpr uint32_t kEmpty = 0xFFFFFFFFu;
    __device__ __forceinline__ void mark_empty(uint8_t* smem) const {
        if (threadIdx.x == 0) *slot(smem) = kEmpty;
    }
    __device__ __forceinline__ int wait_claimed(uint8_t* smem) const {
        volatile uint32_t* w = slot(smem);
        uint32_t v = *w;
        while (v == kEmpty) {           // thread 0 of this workgroup writes it once its atomic returns
            __builtin_amdgcn_s_sleep(1);
            v = *w;
        }
        return __builtin_amdgcn_readfirstlane((int)v);
    }
    __device__ __forceinline__ int claim_wait(uint8_t* smem) const {
        if (threadIdx.x == 0) *(volatile uint32_t*)slot(smem) = atomicAdd(ctr, 1u);
        return wait_claimed(smem);
    }
};
static_assert(kSmemBytes >= kEpiBytes + 4, "tile queue slot");

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// threadIdx.x through an empty volatile asm.  The persistent kernels run the same main loop and
// epilogue tile after tile; per-lane setup computed from a plain threadIdx.x would be hoisted out
// of that loop and kept live across it, and the registers it holds pushed the epilogues into
// spilling.  A volatile asm is never moved out of the loop, so what derives from its value is
// recomputed per tile, where it is used.
__device__ __forceinline__ int opaque_tid() {
    int t = (int)threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
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
// The GEMM epilogues' output stores carry the non-temporal cache policy (the nt bit of the
// buffer instruction's cache-policy operand): a launch writes each output once and never reads it.
// Measured: MXFP4 pre-attention -6% (its short tiles store 4x as often per flop as the bf16 ones),
// out-projection -0.3%, bf16 QKV unchanged; the L2-miss reads (FETCH_SIZE) stay the same, so the
// gain is on the write path.  FC1's y is read back at once by FC2 and keeps the default policy,
// and so do the e4m3 output mode's 4- and 8-byte stores: streamed, their partial lines reached
// HBM as separate writes (WRITE_SIZE +26%, time +0.4%).
constexpr int kStoreNt = 2;
__device__ __forceinline__ void buf_st16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kStoreNt);
}
constexpr uint32_t kOffNone = 0xFFFFFFF0u;   // an offset past every descriptor's bound
// Cache-policy operand of the buffer instructions: nt (non-temporal: streamed through the caches
// without being kept), for data a kernel touches once.
constexpr int kCpolNt = 2;

// Within a wave's slice the swizzle of a fill piece's rows depends only on the piece's
// parity, so B needs two per-lane offsets; A keeps the row in the per-lane offset because only
// that part is checked against the descriptor's bound (rows past M).
constexpr int kVPat = 2;

// The LDS slots holding one stage of A and of B.
struct Stage {
    const uint8_t* a;
    const uint8_t* b;
};

// Accumulators of one wave: MB x NB blocks of 16 x 16.  Lane l, register r of a block holds
// row 4 (l / 16) + r and column l % 16.  Acc: a 128 x 64 wave tile (two waves across m, four
// across n); AccW: 64 x 128 (four across m, two across n), so that one wave holds whole
// 128-column blocks of its rows.  Waves 0-3 hold tile rows 0-127 in both.
template <int kMB, int kNB>
struct AccN {
    static constexpr int MB = kMB, NB = kNB;
    static constexpr int kRows = 16 * kMB;              // rows of the wave tile
    static constexpr int kWavesN = kBN / (16 * kNB);    // waves across n
    f32x4 v[MB][NB];
};
using Acc = AccN<8, 4>;
using AccW = AccN<4, 8>;
// MXFP4: 4 x 2 blocks of 32 x 32.  Lane l, register r of a block holds row
// 8 (r / 4) + 4 (l / 32) + r % 4 and column l % 32.
struct AccMx {
    static constexpr int MB = 4, NB = 2;
    f32x16 w[MB][NB];
};

// Per-lane LDS offsets of the fragment reads (relative to an operand slot).  Lane l reads row
// l % 16 of each 16-row block and, in lane group g = l / 16, chunks g and g + 4 of it:
//   bf16, 16x16x32:  chunk 4 q + g (8 bf16 of k) is the fragment of k-step q = 0, 1;
//   e4m3, 16x16x128: chunks g and g + 4 together (32 bytes of k) are the fragment of the one
//         k-step.  Any assignment of a stage's 128 bytes to (lane group, byte) serves, as long
//         as A and B use the same one; this one reads like the bf16 path, and in both the 16
//         lanes of a group hit 16 distinct bank groups (contiguous chunks 2 g, 2 g + 1 would
//         put two lane groups of a read on the same banks).
// swz has period 16 rows, so one offset serves every block of a wave (blocks are immediates).
// A and B rows of a lane differ only by the wave's row bases, so the B offsets are the A offsets
// plus a wave-uniform difference (bdelta, a scalar added to the B slot's base).
constexpr int kBlk = 16 * kRowB;                // bytes between 16-row blocks
template <class AccT>
struct FragAddrN {
    uint32_t a[2];
    int bdelta;
    __device__ __forceinline__ void init() {
        const int tid = opaque_tid();
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int wm = wave / AccT::kWavesN, wn = wave % AccT::kWavesN;
        const int r = lane % 16, g = lane / 16;
        const int sw = swz(r);      // wave row bases are multiples of 16
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = 4 * q + g;
            a[q] = (uint32_t)((wm * AccT::kRows + r) * kRowB + ((c ^ sw) << 4));
        }
        bdelta = (wn * 16 * AccT::NB - wm * AccT::kRows) * kRowB;
    }
};
using FragAddr = FragAddrN<Acc>;

// MXFP4 (32x32x64): lane l reads row l % 32 of each 32-row block and, for k-step q, chunk
// 2 q + l / 32 (32 E2M1 values).  The 16 lanes of a read quarter sit on 16 consecutive rows of
// one chunk, so the swizzle keeps them on 16 distinct bank groups.
struct FragAddrMx {
    uint32_t a[4];
    int bdelta;
    __device__ __forceinline__ void init() {
        const int tid = opaque_tid();
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int wm = wave / kWN, wn = wave % kWN;
        const int r = lane % 32, h = lane / 32;
        const int sw = swz(r);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = 2 * q + h;
            a[q] = (uint32_t)((wm * 128 + r) * kRowB + ((c ^ sw) << 4));
        }
        bdelta = (wn * kWaveN - wm * 128) * kRowB;
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

// v_mfma_scale_f32_32x32x64_f8f6f4 on E2M1 operands (4 registers each, format 4 for both),
// scale_a / scale_b the E8M0 bytes OA / OB of the lanes' scale words.  The four-register form
// of the intrinsic is named directly: the builtin only takes the eight-register (fp8) operands.
extern "C" __device__ f32x16 __dit_mfma_scale_f4_32(i32x4 a, i32x4 b, f32x16 c, int cbsz, int blgp, int opsel_a,
                                                    int scale_a, int opsel_b, int scale_b)
    __asm("llvm.amdgcn.mfma.scale.f32.32x32x64.f8f6f4.v4i32.v4i32");
// byte selectors as immediates: q is a constant once the MFMA loop is unrolled, and each case
// passes literal ones
__device__ __forceinline__ f32x16 mfma_mxfp4(const i32x4& a, const i32x4& b, const f32x16& c, uint32_t sa,
                                             uint32_t sb, int q) {
    switch (q) {
        case 0: return __dit_mfma_scale_f4_32(a, b, c, 4, 4, 0, (int)sa, 0, (int)sb);
        case 1: return __dit_mfma_scale_f4_32(a, b, c, 4, 4, 1, (int)sa, 1, (int)sb);
        case 2: return __dit_mfma_scale_f4_32(a, b, c, 4, 4, 2, (int)sa, 2, (int)sb);
        default: return __dit_mfma_scale_f4_32(a, b, c, 4, 4, 3, (int)sa, 3, (int)sb);
    }
}

// Every fragment of one stage in registers (24 16-byte reads, 96 registers; MXFP4 adds its 24
// bytes of scales, which the main loop loads from global memory).
template <Mma kKind, class AccT>
struct PPFrags;
template <class AccT>
struct PPFrags<Mma::kBf16, AccT> {
    static constexpr int MB = AccT::MB, NB = AccT::NB;
    bf16x8 a[2][MB], b[2][NB];
    __device__ __forceinline__ void read(const Stage& st, const FragAddrN<AccT>& fa) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int i = 0; i < MB; ++i) a[ks][i] = lds_bf16x8(st.a, fa.a[ks] + i * kBlk);
#pragma unroll
            for (int j = 0; j < NB; ++j) b[ks][j] = lds_bf16x8(st.b + fa.bdelta, fa.a[ks] + j * kBlk);
        }
    }
    __device__ __forceinline__ void mma(AccT& acc) const {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc.v[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks][i], b[ks][j], acc.v[i][j], 0, 0, 0);
    }
};
template <class AccT>
struct PPFrags<Mma::kE4m3, AccT> {
    static constexpr int MB = AccT::MB, NB = AccT::NB;
    i32x8 a[MB], b[NB];
    __device__ __forceinline__ void read(const Stage& st, const FragAddrN<AccT>& fa) {
#pragma unroll
        for (int i = 0; i < MB; ++i) a[i] = lds_i32x8(st.a, fa.a[0] + i * kBlk, fa.a[1] + i * kBlk);
#pragma unroll
        for (int j = 0; j < NB; ++j) b[j] = lds_i32x8(st.b + fa.bdelta, fa.a[0] + j * kBlk, fa.a[1] + j * kBlk);
    }
    __device__ __forceinline__ void mma(AccT& acc) const {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
                acc.v[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i], b[j], acc.v[i][j], 0, 0, 0, 0, 0, 0);
    }
};
// MXFP4: a 128-byte stage row is 256 E2M1 values, four k-steps of 64; lane l reads 16 bytes
// (32 values, block 2 q + l / 32) of its row.  Scale byte q of the lane's A record I belongs
// to block row I, k-step q (B: record J).
template <>
struct PPFrags<Mma::kMxFp4, AccMx> {
    static constexpr int MB = AccMx::MB, NB = AccMx::NB;
    i32x4 a[4][MB], b[4][NB];
    u32x4 sa;      // this lane's E8M0 scale records of the stage (loaded by the main loop)
    u32x2 sb;
    __device__ __forceinline__ void read(const Stage& st, const FragAddrMx& fa) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int i = 0; i < MB; ++i) a[q][i] = __builtin_bit_cast(i32x4, lds_ld16(st.a, fa.a[q] + i * 2 * kBlk));
#pragma unroll
            for (int j = 0; j < NB; ++j)
                b[q][j] = __builtin_bit_cast(i32x4, lds_ld16(st.b + fa.bdelta, fa.a[q] + j * 2 * kBlk));
        }
    }
    __device__ __forceinline__ void mma(AccMx& acc) const {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j) acc.w[i][j] = mfma_mxfp4(a[q][i], b[q][j], acc.w[i][j], sa[i], sb[j], q);
    }
};

// Keeps a compute phase's MFMAs between its two barriers.  The MFMA builtins touch no memory,
// so passes that move pure operations may otherwise carry them across the s_barrier statements
// (whose memory clobber binds only memory accesses): in one build all 64 MFMAs of a phase sank
// past the barrier that ends it into the loop latch, so the two waves of a SIMD issued MFMAs at
// the same time and the ping-pong was lost.  An empty volatile asm that reads and writes every
// accumulator, placed after the opening barrier and after the MFMAs, orders them: volatile asm
// statements keep their program order, and the MFMAs consume the first one's outputs and feed the
// second one's inputs.
template <int kMB, int kNB>
__device__ __forceinline__ void pin_acc(AccN<kMB, kNB>& acc) {
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j) asm volatile("" : "+v"(acc.v[i][j]));
}
__device__ __forceinline__ void pin_acc(AccMx& acc) {
#pragma unroll
    for (int i = 0; i < AccMx::MB; ++i)
#pragma unroll
        for (int j = 0; j < AccMx::NB; ++j) asm volatile("" : "+v"(acc.w[i][j]));
}

// Fragment-address type of an operand kind and accumulator layout.
template <Mma kKind, class AccT>
struct KindTypes {
    using FragAddrT = FragAddrN<AccT>;
};
template <>
struct KindTypes<Mma::kMxFp4, AccMx> {
    using FragAddrT = FragAddrMx;
};

// B row order of a tile.  BRowsDefault: the local rows [0, 128) are global rows nb0.. and
// [128, 256) are nb1.. (or interleaved by 16, kInterleaveB).  A map with kMapped set instead
// names, for each local row L of the B slot, its global row nb0 + row(L) (row(L) in [0, 256),
// nb1 = nb0 + 128), so the columns of the wave tiles can follow another order.  The fills keep
// their form (per lane: the row within the 8-row piece, by piece parity; per piece: a uniform
// base), so the map must satisfy, for every wave w and k < 8,
//   row(32 w + 8 p + k) - row(32 w + 8 p)  the same for pieces p and p + 2.
struct BRowsDefault {
    static constexpr bool kMapped = false;
    __device__ __forceinline__ int row(int L) const { return L; }
};
// Compile-time check of a row map given as a constexpr function of L: a permutation of [0, 256)
// with the fill form above.
template <class RowFn>
constexpr bool brow_map_ok(RowFn row) {
    bool seen[256] = {};
    for (int L = 0; L < 256; ++L) {
        const int g = row(L);
        if (g < 0 || g >= 256 || seen[g]) return false;
        seen[g] = true;
    }
    for (int L0 = 0; L0 < 256; L0 += 32)
        for (int p = 0; p < 2; ++p)
            for (int k = 0; k < 8; ++k)
                if (row(L0 + 8 * p + k) - row(L0 + 8 * p) != row(L0 + 8 * (p + 2) + k) - row(L0 + 8 * (p + 2)))
                    return false;
    return true;
}
// The map that gives each lane of a 64 x 128 wave tile (AccW) 8 contiguous columns: local row
// L = 128 h + 16 j + c is row 128 h + 8 c + j, so lane column c of block j holds column 8 c + j of
// its 128-column half.
__host__ __device__ constexpr int cols8_brow(int L) { return 128 * (L >> 7) + 8 * (L & 15) + ((L >> 4) & 7); }
struct Cols8BRows {
    static constexpr bool kMapped = true;
    __device__ __forceinline__ int row(int L) const { return cols8_brow(L); }
};
static_assert(brow_map_ok([](int L) { return cols8_brow(L); }), "8-column B row order");

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

// Barrier after the accumulators are staged in LDS: waits for this wave's LDS writes only
// (lgkmcnt(0)), not for its global loads.  The epilogues request their global operands (cos/sin
// rows, residual chunks, row indices) before staging, to be in flight across the barrier;
// __syncthreads() would drain them there (its fence waits for vmcnt(0) too).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));    // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}

// MXFP4 scale arrays of A and B in the MX scale layout, and their sizes in bytes (unused for
// the other operand kinds).
struct MxScales {
    const uint8_t* a = nullptr;
    uint32_t a_bytes = 0;
    const uint8_t* b = nullptr;
    uint32_t b_bytes = 0;
};

// ---------------------------------------------------------------------------------------
// Ping-pong main loop (8 waves, 128-byte stage rows; two A slots and a ring of three B slots).
//
// Group G0 = waves 0-3 (tile rows 0-127) and group G1 = waves 4-7 (rows 128-255); waves w
// and w + 4 share a SIMD.  Each wave alternates a memory phase (refill, then read every
// fragment of one stage from LDS into registers) and a compute phase (that stage's MFMAs, from
// registers only).  G1 runs one phase behind G0, so on every SIMD one wave issues MFMAs back
// to back while the other works on LDS; a workgroup barrier ends every phase.  G1 enters one
// extra barrier before its first phase and G0 one after its last, so both groups pass the
// same number of barriers.
//
// Phase 2s: G0 memory(s), G1 compute(s-1).  Phase 2s+1: G0 compute(s), G1 memory(s).
// A stage s sits in A slot s % 2 and B slot s % 3.  The B slot a wave refills with stage s+2
// held stage s-1, which both groups finished reading before the barrier that opens stage s's
// first phase, so every wave refills as soon as its memory phase starts, before its own
// fragment reads, and both groups move the same bytes: each wave fills its 32 rows of A (stage
// s+1; its group alone reads them, and read stage s-1 from that slot a phase earlier) and its
// 32 rows of B (stage s+2), 8 KiB in 8 loads.  (With two B slots a B slot is free only after
// the second group's reads, so one group moved three quarters of the stage's fills after its
// reads.)  All fills are issued in memory phases: a wave issues in order, so a load that waits
// for the memory pipeline would hold back the MFMAs behind it.  Loads for stages past the end
// go through a zero-length descriptor (no memory read, zeros into a slot with no reader left),
// so every phase issues the same loads and the vmcnt limits hold throughout.
//
// MXFP4: the E8M0 scales of a stage are not staged in LDS (the five slots fill it): in the MX
// scale layout each wave's scales for a stage are one contiguous 1 KiB record of its group, 16
// bytes per lane for A and 8 for B, which it loads straight into the registers the MFMAs take
// them from, right after the compute phase that used the previous ones.
//
// Each wave waits only for its own loads before a barrier (per wave and stage: 8 fills, and
// for MXFP4 2 scale loads after the MFMAs):
//   G0, end of its compute phase for s:  A(s+1) and B(s+1) landed, B(s+2) (and the scales of
//                                        s+1) may fly;
//   G1, end of its memory phase for s:   B(s+1) landed (G0 reads it next phase); MXFP4: the
//                                        scales of s landed;
//   G0, end of its memory phase for s:   MXFP4: the scales of s landed;
//   G1, end of its compute phase for s:  A(s+1) landed (its next memory phase).
// G0's rows of A and B are read by G1 one phase after G0 has waited for them, and G1's rows
// of B by G0 one phase after G1 has.
constexpr int kPPAPieces = 32 / kRowsPerPiece;      // rows per wave and operand: 4 loads of 1 KiB

struct PPFill {
    __amdgpu_buffer_rsrc_t ra, rb, rnull;
    uint32_t va[kPPAPieces];  // A: row + chunk offset of piece j (per lane; bounds-checked)
    uint32_t vb[kVPat];       // B: row-in-piece + chunk offset, by piece parity (per lane)
    uint32_t sb[kPPAPieces];  // B: offset of piece j's first row (uniform)
    uint32_t lds_rows;        // this wave's 32 rows within an A or B slot
    // MXFP4: this wave's scale records (A: its group's rows; B: the 128-row group holding its
    // columns), and this lane's bytes in them
    __amdgpu_buffer_rsrc_t rsa, rsb;
    uint32_t vsa, vsb;
    __device__ __forceinline__ void a_rows(uint8_t* smem, int slot, int kt, bool live) const {
        lds_u8* S = (lds_u8*)smem + slot * kOpBytes + lds_rows;
        const __amdgpu_buffer_rsrc_t r = live ? ra : rnull;
#pragma unroll
        for (int j = 0; j < kPPAPieces; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, S + j * 1024, 16, (int)va[j], kt * kRowB, 0, 0);
    }
    __device__ __forceinline__ void b_rows(uint8_t* smem, int slot, int kt, bool live) const {
        lds_u8* S = (lds_u8*)smem + (2 + slot) * kOpBytes + lds_rows;
        const __amdgpu_buffer_rsrc_t r = live ? rb : rnull;
#pragma unroll
        for (int j = 0; j < kPPAPieces; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, S + j * 1024, 16, (int)vb[j % kVPat], (int)sb[j] + kt * kRowB,
                                                     0, 0);
    }
    // MXFP4 scales of stage kt into the fragment registers (through rnull past the last stage)
    __device__ __forceinline__ void scales(u32x4& sa, u32x2& sbv, int kt, bool live) const {
        sa = __builtin_amdgcn_raw_buffer_load_b128(live ? rsa : rnull, (int)(vsa + kt * 1024), 0, 0);
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(live ? rsb : rnull, (int)(vsb + kt * 1024), 0, 0);
        sbv = u32x2{(uint32_t)v[0], (uint32_t)v[1]};
    }
};

// The operands of one tile's main loop: A rows m0.. of its M rows (rows past M read as zero),
// B local rows [0, 128) from global row nb0 and [128, 256) from nb1 (nb1 = nb0 + 128 for a plain
// tile; for MXFP4 both multiples of 128), unless kInterleaveB or a row map orders them; ktiles
// stages of kRowB bytes per row.
struct TileOps {
    const uint8_t* A;
    int64_t lda, m0, M;
    const uint8_t* B;
    int64_t ldb, nb0, nb1;
    int ktiles;
};

// The fill descriptors and per-lane offsets of wave `wave`'s 32 rows of A and B (lane `lane`).
template <bool kInterleaveB, class BMap>
__device__ __forceinline__ void fill_setup(PPFill& sf, const TileOps& t, int wave, int lane, const BMap& bmap) {
    constexpr bool kMapped = BMap::kMapped;
    static_assert(!(kMapped && kInterleaveB), "one B row order");
    const int64_t arows = t.M - t.m0 < kBM ? t.M - t.m0 : kBM;
    sf.ra = make_rsrc(t.A + t.m0 * t.lda, (uint32_t)(arows * t.lda));
    sf.rb = make_rsrc(t.B + t.nb0 * t.ldb, (uint32_t)((t.nb1 - t.nb0 + 128) * t.ldb));
    sf.rnull = make_rsrc(t.B, 0u);
#pragma unroll
    for (int j = 0; j < kPPAPieces; ++j) {
        const int row = 32 * wave + j * kRowsPerPiece + lane / kSlots;
        sf.va[j] = (uint32_t)(row * t.lda) + (uint32_t)(((lane % kSlots) ^ swz(row)) << 4);
        const int64_t r0 = 32 * wave + j * kRowsPerPiece;                // piece's first row (uniform)
        if constexpr (kMapped) {
            sf.sb[j] = (uint32_t)(bmap.row((int)r0) * t.ldb);
        } else if constexpr (kInterleaveB) {
            static_assert(kPPAPieces == 4 && kRowsPerPiece == 8, "two pieces per 16-row half");
            const int64_t g = j < 2 ? 16 * wave + 8 * j : (t.nb1 - t.nb0) + 16 * wave + 8 * (j - 2);
            sf.sb[j] = (uint32_t)(g * t.ldb);
        } else {
            sf.sb[j] = (uint32_t)((r0 < 128 ? r0 : r0 + (t.nb1 - t.nb0 - 128)) * t.ldb);
        }
        if (j < kVPat) {
            const int brow = (int)r0 + lane / kSlots;
            const int in_piece = kMapped ? bmap.row(brow) - bmap.row((int)r0) : lane / kSlots;
            sf.vb[j] = (uint32_t)(in_piece * t.ldb) + (uint32_t)(((lane % kSlots) ^ swz(brow)) << 4);
        }
    }
    sf.lds_rows = (uint32_t)(32 * wave * kRowB);
}

// kInterleaveB: B local rows 32 w + [0, 16) are global rows nb0 + 16 w + [0, 16) and 32 w + [16,
// 32) are nb1 + 16 w + [0, 16) (w = 0..7), so each wave's 16-column blocks alternate between the
// two halves and a lane holds matching columns of both in adjacent blocks.  kPersist: the tile is
// one of a persistent workgroup's run (persistent_tiles).  Then, when `prefilled`, its prologue
// fills (A(0), B(0), B(1), all 256 rows) were issued by G0 during the previous tile's boundary
// and have landed behind a barrier; each group waits for every load of its last phase that issues
// any (the dead ones past the end included) before that phase's barrier, so that once G0 has left
// the loop no fill of the tile is in flight; and the loop returns after each wave's last in-loop
// barrier, without the closing barrier: the caller then owes G0 one barrier (the one that ends
// G1's last compute phase).
// AccT: the wave tile (Acc or AccW; AccMx for MXFP4).  bmap: the B row order (BRowsDefault).
template <Mma kKind, bool kInterleaveB, bool kPersist, class AccT, class BMap>
__device__ __forceinline__ void mainloop_pp(const uint8_t* __restrict__ A, int64_t lda, int64_t m0, int64_t M,
                                            const uint8_t* __restrict__ B, int64_t ldb, int64_t nb0, int64_t nb1,
                                            int ktiles, uint8_t* smem, AccT& acc, const MxScales& mxs,
                                            const BMap& bmap, bool prefilled = false) {
    static_assert(kWaves == 8 && kRowB == 128, "ping-pong layout");
    constexpr bool kMx = kKind == Mma::kMxFp4;
    constexpr int kFills = 2 * kPPAPieces;          // fill loads per wave and memory phase
    constexpr int kScl = kMx ? 2 : 0;               // scale loads per wave, after its MFMAs
    const int tid = opaque_tid();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const bool g0 = wave < 4;
    static_assert(!(BMap::kMapped && kMx), "one B row order");
    static_assert(!(kPersist && kMx), "persistent runs take register epilogues (no MXFP4 scales)");
    PPFill sf;
    fill_setup<kInterleaveB>(sf, TileOps{A, lda, m0, M, B, ldb, nb0, nb1, ktiles}, wave, lane, bmap);
    if constexpr (kMx) {
        // A: the 128-row group of this wave's rows (the last m tile's second group may lie past
        // the array: zero records, scales read as 0); B: the group of this wave's 64 columns
        const int wm = wave / kWN, wn = wave % kWN;
        const int64_t group_bytes = (int64_t)ktiles * 1024;
        const int64_t ga = m0 / 128 + wm;
        const int64_t a_rest = (int64_t)mxs.a_bytes - ga * group_bytes;
        sf.rsa = make_rsrc(mxs.a + (a_rest > 0 ? ga * group_bytes : 0), (uint32_t)(a_rest > 0 ? a_rest : 0));
        const int64_t gb = (wn < 2 ? nb0 : nb1) / 128;
        sf.rsb = make_rsrc(mxs.b + gb * group_bytes, (uint32_t)((int64_t)mxs.b_bytes - gb * group_bytes));
        sf.vsa = (uint32_t)(lane * 16);
        sf.vsb = (uint32_t)(lane * 16 + (wn % 2) * 8);
    }
    typename KindTypes<kKind, AccT>::FragAddrT fa;
    fa.init();
    if constexpr (kMx) {
#pragma unroll
        for (int i = 0; i < AccMx::MB; ++i)
#pragma unroll
            for (int j = 0; j < AccMx::NB; ++j) acc.w[i][j] = 0.f;
    } else {
#pragma unroll
        for (int i = 0; i < AccT::MB; ++i)
#pragma unroll
            for (int j = 0; j < AccT::NB; ++j) acc.v[i][j] = 0.f;
    }

    PPFrags<kKind, AccT> fr;
    if (!(kPersist && prefilled)) {
        // prologue: this wave's rows of A(0), B(0) (and the scales of stage 0), then B(1).  A(0)
        // and B(0) must land before the first reads; B(1) before this wave's first wait that
        // covers it (G1: the end of its first memory phase; G0: the end of its first compute phase)
        sf.a_rows(smem, 0, 0, true);
        sf.b_rows(smem, 0, 0, true);
        if constexpr (kMx) sf.scales(fr.sa, fr.sb, 0, true);
        sf.b_rows(smem, 1, 1, ktiles > 1);
        pp_barrier<kPPAPieces + kScl>();
    }
    if (!g0) pp_barrier<63>();       // G1 starts one phase behind
    int sb_read = 0;                 // B slot of stage kt (kt % 3)
    // Not unrolled or peeled: in a peeled copy the scheduler reordered the MFMAs of the two
    // k-steps and the register allocator then spilled accumulators to scratch.
#pragma nounroll
    for (int kt = 0; kt < ktiles; ++kt) {
        const int sa = kt & 1;
        const int sb_fill = sb_read == 0 ? 2 : sb_read - 1;              // (kt + 2) % 3
        // memory phase: refill first (A of stage kt+1, B of stage kt+2), then read stage kt
        __builtin_amdgcn_sched_barrier(0);
        sf.a_rows(smem, sa ^ 1, kt + 1, kt + 1 < ktiles);
        sf.b_rows(smem, sb_fill, kt + 2, kt + 2 < ktiles);
        __builtin_amdgcn_sched_barrier(0);
        fr.read(Stage{smem + sa * kOpBytes, smem + (2 + sb_read) * kOpBytes}, fa);
        __builtin_amdgcn_sched_barrier(0);
        if (g0) {
            pp_barrier<kMx ? kFills : 63>();         // MXFP4: the scales of stage kt landed
        } else if (!kPersist || kt + 1 < ktiles) {
            pp_barrier<kFills>();                    // B(kt+1) (and the scales of kt) landed
        } else {
            pp_barrier<0>();                         // the last one: its dead fills landed too
        }
        // compute phase: MFMAs only, then the next stage's scales into the registers they used
        __builtin_amdgcn_sched_barrier(0);
        pin_acc(acc);
        fr.mma(acc);
        pin_acc(acc);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kMx) sf.scales(fr.sa, fr.sb, kt + 1, kt + 1 < ktiles);
        __builtin_amdgcn_sched_barrier(0);
        if (!kPersist || kt + 1 < ktiles || !g0) {
            pp_barrier<kPPAPieces + kScl>();         // A(kt+1) (G0: and B(kt+1)) landed
        } else {
            pp_barrier<0>();                         // G0's last: its dead fills landed too
        }
        sb_read = sb_read == 2 ? 0 : sb_read + 1;
    }
    if constexpr (!kPersist) {
        if (g0) pp_barrier<63>();    // G1's last compute phase
        // drain every load (the dead ones too: they write zeros into the slots the caller reuses)
        __syncthreads();
    }
}

// Main loop over `ktiles` stages of K for one tile (TileOps).  Ends with all loads drained and a
// barrier, so the caller may reuse the LDS (kSmemBytes).
template <Mma kKind, bool kInterleaveB = false, class AccT, class BMap = BRowsDefault>
__device__ __forceinline__ void mainloop(const uint8_t* __restrict__ A, int64_t lda, int64_t m0, int64_t M,
                                         const uint8_t* __restrict__ B, int64_t ldb, int64_t nb0, int64_t nb1,
                                         int ktiles, uint8_t* smem, AccT& acc, const MxScales& mxs = MxScales{},
                                         const BMap& bmap = BMap{}) {
    mainloop_pp<kKind, kInterleaveB, false, AccT, BMap>(A, lda, m0, M, B, ldb, nb0, nb1, ktiles, smem, acc, mxs,
                                                         bmap);
}

// G0 wave w issues a tile's prologue fills for its own rows and for those of wave w + 4 (G1):
// A(0) and B(0) first (16 loads), then B(1) (8 loads; through the null descriptor for a one-stage
// tile).
template <bool kInterleaveB, class BMap>
__device__ __forceinline__ void prefill(const TileOps& t, uint8_t* smem, const BMap& bmap) {
    const int tid = opaque_tid();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    PPFill f0, f1;
    fill_setup<kInterleaveB>(f0, t, wave, lane, bmap);
    fill_setup<kInterleaveB>(f1, t, wave + 4, lane, bmap);
    f0.a_rows(smem, 0, 0, true);
    f1.a_rows(smem, 0, 0, true);
    f0.b_rows(smem, 0, 0, true);
    f1.b_rows(smem, 0, 0, true);
    f0.b_rows(smem, 1, 1, t.ktiles > 1);
    f1.b_rows(smem, 1, 1, t.ktiles > 1);
}

// A persistent workgroup's run over the tiles it claims from tq, for the kernels whose epilogue
// works from the accumulators (no LDS).  tile(k, TileOps&, BMap&) names the operands of claimed
// tile k; epi(acc, TileOps) writes the tile out.  At each tile boundary G0 runs its epilogue while
// G1 finishes its last compute phase; past the barrier that ends that phase, G1 runs its epilogue
// while G0 claims the next tile.  kPrefill: G0 then also issues the next tile's prologue fills for
// all 256 rows, so their latency hides behind G1's epilogue instead of following it, and the next
// main loop starts with its first memory phase.  That pays where the clock has headroom (the e4m3
// GEMMs: MLP -0.85%); the bf16 GEMMs run at the power limit, where a shorter idle gap only lowers
// the clock (QKV and out-projection +0.2-0.3%, within noise), and load their own prologue.  The
// barrier after both epilogues drains every load.
template <Mma kKind, bool kInterleaveB, bool kPrefill, class AccT, class BMap, class TileFn, class EpiFn>
__device__ __forceinline__ void persistent_tiles(const TileQueue& tq, uint8_t* smem, TileFn tile, EpiFn epi) {
    tq.claim(smem);
    __syncthreads();
    const bool g0 = __builtin_amdgcn_readfirstlane(opaque_tid() >> 6) < 4;
    bool prefilled = false;
    int k = tq.claimed(smem);
    while (k < tq.cnt) {
        TileOps t;
        BMap bm;
        tile(k, t, bm);
        AccT acc;
        mainloop_pp<kKind, kInterleaveB, true, AccT, BMap>(t.A, t.lda, t.m0, t.M, t.B, t.ldb, t.nb0, t.nb1,
                                                            t.ktiles, smem, acc, MxScales{}, bm, prefilled);
        int kn;
        if (g0) {
            // no fill is in flight (the main loop's last barriers waited for them all, the dead
            // ones that write the claim word's rows included), so the slot keeps what is written
            tq.mark_empty(smem);
            epi(acc, t);
            pp_barrier<63>();   // the barrier that ends G1's last compute phase
            kn = tq.claim_wait(smem);
            if (kPrefill && kn < tq.cnt) {
                TileOps tn;
                BMap bmn;
                tile(kn, tn, bmn);
                prefill<kInterleaveB>(tn, smem, bmn);
            }
        } else {
            epi(acc, t);
            kn = tq.wait_claimed(smem);
        }
        // every wave's loads drained (the next tile's prologue fills landed) and every read of the
        // claim word done before the next tile's first fill of its row
        __builtin_amdgcn_s_waitcnt(0x0F70);         // vmcnt(0)
        __syncthreads();
        k = kn;
        prefilled = kPrefill;
    }
    tq.finish();
}

// Epilogue phase 1: tile[row][col] = bf16((acc * rowscale[row]) * colscale[col]) into LDS
// (row pitch kEpiPitch), the products in fp32 as printed, then RNE to bf16.
// rowscale and colscale are both given or both null (factor 1).  Registers r and r + 1 of a
// block hold rows R and R + 1 of one column c = l % 16, packed as one bf16 pair; lanes l and
// l ^ 1 (columns c and c ^ 1) swap halves with one DPP move, so that the even lane holds row R,
// columns c, c + 1 and the odd lane row R + 1, columns c - 1, c: one 32-bit LDS write each.
// Must follow a barrier that ends all LDS reads of the main loop.
__device__ __forceinline__ void stage_tile_bf16(const Acc& acc, uint8_t* smem, const float* rowscale, int64_t m0,
                                                int64_t M, const float* colscale_lo, const float* colscale_hi) {
    const int tid = opaque_tid();
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / kWN, wn = wave % kWN;
    const int col_in = lane % 16, row_in = (lane / 16) * 4;
    const int odd = lane & 1;
    // v_perm selector on (neighbour pair, own pair): even lane (own.lo, nb.lo), odd lane
    // (nb.hi, own.hi)
    const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
    float cscale[Acc::NB];
#pragma unroll
    for (int j = 0; j < Acc::NB; ++j) cscale[j] = 1.f;
    if (colscale_lo) {
        // local columns [0,128) come from colscale_lo, [128,256) from colscale_hi
        const int c0 = wn * kWaveN;
        const float* cs = c0 < 128 ? colscale_lo + c0 : colscale_hi + (c0 - 128);
#pragma unroll
        for (int j = 0; j < Acc::NB; ++j) cscale[j] = cs[j * 16 + col_in];
    }
    // row scales of block row i + 1 are loaded while block row i converts: the lane's four rows
    // are consecutive, one 16-byte load through a descriptor over the tile's rows (rows past M
    // read 0; their accumulators are 0 and never stored)
    const __amdgpu_buffer_rsrc_t rrs =
        make_rsrc(rowscale + (rowscale ? m0 : 0), (uint32_t)((M - m0 < kBM ? M - m0 : kBM) * 4));
    auto load_rs = [&](int i, float (&rs)[4]) {
        const u32x4 v = buf_ld16(rrs, (uint32_t)((wm * 128 + i * 16 + row_in) * 4));
#pragma unroll
        for (int r = 0; r < 4; ++r) rs[r] = __uint_as_float(v[r]);
    };
    float rs[4], rs_nx[4];
    if (rowscale) load_rs(0, rs);
#pragma unroll
    for (int i = 0; i < Acc::MB; ++i) {
        if (rowscale && i + 1 < Acc::MB) load_rs(i + 1, rs_nx);
#pragma unroll
        for (int j = 0; j < Acc::NB; ++j) {
            const int col = wn * kWaveN + j * 16 + col_in - odd;
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
                const int row = wm * 128 + i * 16 + row_in + r + odd;
                const float a0 = acc.v[i][j][r], a1 = acc.v[i][j][r + 1];
                uint32_t b;
                if (rowscale) {
                    b = pack_bf2((a0 * rs[r]) * cscale[j], (a1 * rs[r + 1]) * cscale[j]);
                } else {
                    b = pack_bf2(a0, a1);
                }
                // quad_perm(1,0,3,2): lane l <- l ^ 1 (every lane active, the source always exists)
                const uint32_t nb = (uint32_t)__builtin_amdgcn_mov_dpp((int)b, 0xB1, 0xF, 0xF, true);
                *reinterpret_cast<uint32_t*>(smem + row * kEpiPitch + col * 2) = __builtin_amdgcn_perm(nb, b, sel);
            }
        }
        if (rowscale) {
#pragma unroll
            for (int r = 0; r < 4; ++r) rs[r] = rs_nx[r];
        }
    }
}

// The same staging (no scales) for the 32 x 32 blocks of the MXFP4 accumulators: registers
// r and r + 1 (r even) of a block again hold rows R and R + 1 of one column, so the lane-pair
// swap is the same.
__device__ __forceinline__ void stage_tile_bf16(const AccMx& acc, uint8_t* smem) {
    const int tid = opaque_tid();
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / kWN, wn = wave % kWN;
    const int col_in = lane % 32, row_in = (lane / 32) * 4;
    const int odd = lane & 1;
    const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
#pragma unroll
    for (int i = 0; i < AccMx::MB; ++i) {
#pragma unroll
        for (int j = 0; j < AccMx::NB; ++j) {
            const int col = wn * kWaveN + j * 32 + col_in - odd;
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const int row = wm * 128 + i * 32 + 8 * (r / 4) + row_in + r % 4 + odd;
                const uint32_t b = pack_bf2(acc.w[i][j][r], acc.w[i][j][r + 1]);
                const uint32_t nb = (uint32_t)__builtin_amdgcn_mov_dpp((int)b, 0xB1, 0xF, 0xF, true);
                *reinterpret_cast<uint32_t*>(smem + row * kEpiPitch + col * 2) = __builtin_amdgcn_perm(nb, b, sel);
            }
        }
    }
}

__device__ __forceinline__ u32x4 epi_ld(const uint8_t* smem, int row, int col) {
    return *reinterpret_cast<const u32x4*>(smem + row * kEpiPitch + col * 2);
}

}  // namespace gemm
}  // namespace dit
