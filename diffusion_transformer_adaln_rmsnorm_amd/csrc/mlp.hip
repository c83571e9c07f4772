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
// accumulators.  The y quantisation then reads each row of y once, takes its maximum |y| for s_y
// and writes y_q, and FC2 consumes y_q: where the m tiles split into whole groups per XCD, FC2
// quantises y itself, a group ahead of its GEMM tiles, behind ready counters
// (k_fc2_gated_fused); otherwise a launch of its own does it, and stream order separates the
// three launches.
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

// y quantisation of row m by one wavefront: 14336 = 1792 chunks of 8, 28 per lane.  The row is
// read once into registers: its maximum |y| (on the bf16 bits, as in the MX quantiser), then
// s_y = RN(amax / 448) and the codes.  kNt: y is read with the non-temporal cache policy (inside
// FC2, so that the stream does not evict the GEMM tiles' operands from L2).
template <bool kNt = false>
__device__ __forceinline__ void quant_y_row(const uint16_t* __restrict__ y, int64_t m, float* __restrict__ y_scale,
                                            uint8_t* __restrict__ y_q, int lane) {
    constexpr int kPerLane = kInter / 8 / 64;    // 28
    const uint16_t* yr = y + m * kInter;
    u32x4 yv[kPerLane];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) yv[j] = kNt ? ld16_nt(yr + (j * 64 + lane) * 8) : ld16(yr + (j * 64 + lane) * 8);
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

// y quantisation as a launch of its own: one wavefront per row.
__global__ __launch_bounds__(256) void k_quant_rows(const uint16_t* __restrict__ y, int64_t M,
                                                    float* __restrict__ y_scale, uint8_t* __restrict__ y_q) {
    const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M) return;
    quant_y_row(y, m, y_scale, y_q, threadIdx.x & 63);
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

// FC2 with the y quantisation in the same launch, as the MLP page's FC2 quantises y for its own
// tiles and publishes tile-ready flags (description under its formula block).  Used when the m
// tiles split into the XCDs' ranges as whole groups of kQGroupTiles m tiles (mt a multiple of
// 4 x 8), so that every row of a group is quantised and consumed on one XCD.  Each XCD's queue
// interleaves quant units (32 rows of y -> y_q and s_y, 4 rows per wave) with its GEMM tiles: the
// 32 units of its first group, then each group's 84 tiles in four chunks of 21, each chunk
// followed by 8 of the next group's units, so that a group's units run one group ahead, beside
// GEMM tiles, and the y stream overlaps the MFMA work.
//
// Hand-over: a unit's waves wait for their stores, then its workgroup adds one to the group's
// ready counter; a GEMM tile of the group (or G0, before it issues the tile's prologue fills)
// waits until the counter holds all 32 units.  Producer and consumer work on the same range, so
// they run on the same XCD: the dispatcher deals workgroups to the XCDs round robin, and workgroup
// b takes range b % 8, so every workgroup of a range sits on XCD b % (XCDs of the device), which
// holds for a device of 8, 4, 2 or 1 XCDs.  The codes and scales are therefore in the L2 both
// use, and no CU has read those rows' codes or scales earlier in the launch (each L1 starts
// empty), so no L1 holds stale copies.  Every unit a tile waits for was claimed earlier by a
// running workgroup and waits for nothing itself, so the wait ends.
constexpr int kQGroupTiles = 4;                               // m tiles per group (the logical order's)
constexpr int kQUnitRows = kWaves * 4;                        // rows of y per quant unit
constexpr int kQUnits = kQGroupTiles * kBM / kQUnitRows;      // units per group: 32
constexpr int kQNt = kHidden / kBN;                           // FC2's n tiles: 21
constexpr int kQGroupN = kQGroupTiles * kQNt;                 // GEMM tiles per group: 84
constexpr int kQChunks = 4;
constexpr int kQChunkTiles = kQGroupN / kQChunks;             // 21
constexpr int kQChunkUnits = kQUnits / kQChunks;              // 8
constexpr int kQChunk = kQChunkTiles + kQChunkUnits;          // 29
constexpr int kQSpan = kQGroupN + kQUnits;                    // items per group: 116
static_assert(kQGroupN % kQChunks == 0 && kQUnits % kQChunks == 0, "chunks");

// Item i of an XCD's queue (ng groups): a unit (group g, unit idx) or a GEMM tile (group g, tile
// idx of the group, in the logical order).
struct QItem {
    bool unit;
    int g, idx;
};
__host__ __device__ constexpr QItem q_item(int i, int ng) {
    if (i < kQUnits) return QItem{true, 0, i};
    i -= kQUnits;
    if (i < kQSpan * (ng - 1)) {
        const int g = i / kQSpan, r = i - g * kQSpan, c = r / kQChunk, p = r - c * kQChunk;
        return p < kQChunkTiles ? QItem{false, g, kQChunkTiles * c + p}
                                : QItem{true, g + 1, kQChunkUnits * c + (p - kQChunkTiles)};
    }
    return QItem{false, ng - 1, i - kQSpan * (ng - 1)};
}
// Every tile and unit of ng groups appears once, and a group's units all precede its first tile.
constexpr bool q_order_ok(int ng) {
    int units_seen[32] = {}, tiles_seen[32] = {};
    bool tile_seen[32 * kQGroupN] = {}, unit_seen[32 * kQUnits] = {};
    for (int i = 0; i < kQSpan * ng; ++i) {
        const QItem it = q_item(i, ng);
        if (it.g < 0 || it.g >= ng) return false;
        if (it.unit) {
            if (it.idx < 0 || it.idx >= kQUnits || unit_seen[it.g * kQUnits + it.idx]) return false;
            if (tiles_seen[it.g] != 0) return false;
            unit_seen[it.g * kQUnits + it.idx] = true;
            ++units_seen[it.g];
        } else {
            if (it.idx < 0 || it.idx >= kQGroupN || tile_seen[it.g * kQGroupN + it.idx]) return false;
            if (units_seen[it.g] != kQUnits) return false;
            tile_seen[it.g * kQGroupN + it.idx] = true;
            ++tiles_seen[it.g];
        }
    }
    for (int g = 0; g < ng; ++g)
        if (units_seen[g] != kQUnits || tiles_seen[g] != kQGroupN) return false;
    return true;
}
static_assert(q_order_ok(1) && q_order_ok(2) && q_order_ok(4) && q_order_ok(7) && q_order_ok(18), "quant unit order");
static_assert(kMaxReady >= kXcds * 18, "ready counters for the largest fused launch");

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void k_fc2_gated_fused(const uint16_t* __restrict__ y, float* __restrict__ y_scale, uint8_t* __restrict__ y_q,
                       int64_t M, const uint8_t* __restrict__ W2, const float* __restrict__ w2s,
                       const uint16_t* __restrict__ gate, int64_t gate_rows, int64_t gate_ld,
                       const int64_t* __restrict__ idx, const uint16_t* residual, uint16_t* out, int mt,
                       uint32_t* tq_ctr) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
    const int ng = mt / (kQGroupTiles * kXcds);                    // groups per XCD
    const TileQueue tq(tq_ctr, kXcds * kQSpan * ng, 1);            // kQSpan ng items per range
    const int gx = tq.xcd * ng;                                    // this range's first group
    uint32_t* const ready = tq.set + kReadyBase;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const bool g0 = wave < 4;
    auto tile = [&](const QItem& it, TileOps& to) {
        int tm, tn;
        logical_coords((gx + it.g) * kQGroupN + it.idx, mt, kQNt, tm, tn);
        const int n0 = tn * kBN;
        to = TileOps{y_q, kInter, (int64_t)tm * kBM, M, W2, kInter, n0, n0 + 128, kInter / kRowB};
    };
    // until every unit of group g has been counted (read at L2: the load skips the L1)
    auto wait_ready = [&](int g) {
        const uint32_t* r = ready + gx + g;
        while (__hip_atomic_load(r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)kQUnits)
            __builtin_amdgcn_s_sleep(2);
    };
    tq.claim(smem);
    __syncthreads();
    int k = tq.claimed(smem);
    bool prefilled = false;
    while (k < tq.cnt) {
        const QItem it = q_item(k, ng);
        if (it.unit) {
            const int64_t r0 = (int64_t)(gx + it.g) * (kQGroupTiles * kBM) + it.idx * kQUnitRows + 4 * wave;
            for (int q = 0; q < 4; ++q)
                if (r0 + q < M) quant_y_row<true>(y, r0 + q, y_scale, y_q, threadIdx.x & 63);
            __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0): this wave's codes and scale are in L2
            __syncthreads();
            if (threadIdx.x == 0) atomicAdd(ready + gx + it.g, 1u);
            tq.claim(smem);
            __syncthreads();
            k = tq.claimed(smem);
            prefilled = false;
            continue;
        }
        TileOps to;
        tile(it, to);
        if (!prefilled) wait_ready(it.g);
        AccW acc;
        mainloop_pp<Mma::kE4m3, false, true, AccW, Cols8BRows>(to.A, to.lda, to.m0, to.M, to.B, to.ldb, to.nb0,
                                                               to.nb1, to.ktiles, smem, acc, MxScales{},
                                                               Cols8BRows{}, prefilled);
        int kn;
        if (g0) {
            tq.mark_empty(smem);
            gated_epilogue_regs<int64_t, true>(acc, to.m0, M, (int)to.nb0, y_scale, w2s, idx, gate, gate_rows, gate_ld,
                                               residual, out);
            pp_barrier<63>();   // the barrier that ends G1's last compute phase
            kn = tq.claim_wait(smem);
            if (kn < tq.cnt) {
                const QItem nx = q_item(kn, ng);
                if (!nx.unit) {
                    wait_ready(nx.g);
                    TileOps tn;
                    tile(nx, tn);
                    prefill<false>(tn, smem, Cols8BRows{});
                }
            }
        } else {
            gated_epilogue_regs<int64_t, true>(acc, to.m0, M, (int)to.nb0, y_scale, w2s, idx, gate, gate_rows, gate_ld,
                                               residual, out);
            kn = tq.wait_claimed(smem);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);         // vmcnt(0): the prologue fills landed
        __syncthreads();
        prefilled = kn < tq.cnt && !q_item(kn, ng).unit;
        k = kn;
    }
    tq.finish(kXcds * ng);
}

bool fc2_fused_fits(int64_t M) {
    const int64_t mt = (M + kBM - 1) / kBM;
    return mt % (kQGroupTiles * kXcds) == 0 && mt / kQGroupTiles <= kMaxReady;
}

hipError_t launch_fc2_fused(const uint16_t* y, float* y_scale, uint8_t* y_q, int64_t M, const uint8_t* W2,
                            const float* w2s, const uint16_t* gate, int64_t gate_rows, int64_t gate_ld,
                            const int64_t* idx, const uint16_t* residual, uint16_t* out, hipStream_t stream) {
    if (!fc2_fused_fits(M)) return hipErrorInvalidValue;
    const int mt = (int)((M + kBM - 1) / kBM);
    uint32_t* q = nullptr;
    int grid = 0;
    const hipError_t e = tile_queue(stream, &q, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_fc2_gated_fused, dim3((unsigned)grid), dim3(kThreads), 0, stream, y, y_scale, y_q, M, W2, w2s,
                       gate, gate_rows, gate_ld, idx, residual, out, mt, q);
    return hipGetLastError();
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
