// QKV projection with the fused Q/K RMSNorm, RoPE and pack epilogue (launch 2 of the bf16
// pre-attention stage).
//
// FlashInfer "minimax_h3_bf16_pre_attention": description (GEMM streams the workspace, the
// epilogue applies the per-head Q/K RMSNorm, partial split-half NeoX RoPE and the
// destination-major pack) and Parameters (qkv_weight row order [q_all | k_all | v_all] x 56
// heads x 128, q/k_norm_weight [128], rope_cos_sin [S, 96] with cos in columns [0,48) and sin
// in [48,96), rope_positions clamped to [0, S) or the identity, out [P, M, 56 / P, 3, 128] for
// P = ulysses_degree destinations, destination p holding heads [p 56/P, (p+1) 56/P)).
//
// A 256-wide n tile is exactly two heads of one kind (7168 = 28 x 256), so each tile owns
// whole heads and needs nothing from its neighbours.
//
// bf16 operands: 64 x 128 wave tiles, so a wave holds one head of its 64 rows, with the weight
// rows loaded in an order (QkvBRows) that gives each lane 4 contiguous dims and their RoPE
// partners; the epilogue works from the accumulators (qkv_epilogue_regs).  The epilogue is
// bound by VALU issue, so the layout is chosen to keep its per-element instruction count low.
//
// MXFP4 operands: 128 x 64 wave tiles; after the main loop the tile is rounded to bf16 into LDS,
// then the 16 lanes of one DPP row own one (row, head), 8 dims each (qk_norm_rope), and each
// lane writes 16 contiguous bytes of out.
#include "common.hpp"
#include "gemm.hpp"
#include "kernels.hpp"
#include "qk_epi.hpp"

namespace dit {

using namespace gemm;

// a / s rounded to nearest (div_by), except that quotients far beyond the largest e4m3 value
// (which saturate either way) skip the correction, which an infinite first guess would turn
// into NaN
__device__ __forceinline__ float div_sat(float a, float s, float y) {
    const float q0 = a * y;
    return fabsf(q0) > 1024.0f ? q0 : div_by(a, s, y);
}

// Head dim held by lane column c (= l % 16) in column block j of a wave of the register
// epilogue: in a Q/K tile lanes c < 12 hold dims 4 c .. 4 c + 3 (blocks 0-3) and their RoPE
// partners 48 + 4 c .. (blocks 4-7), so each pair (d, d + 48) sits in one lane, and lanes 12-15
// the pass-through dims 96 + 8 (c - 12) + j; in a V tile lane c holds dims 8 c + j.
__host__ __device__ constexpr int qkv_dim(int j, int c, bool rope) {
    const int rot = (j < 4 ? 4 * c : kNFreq + 4 * c) + (j & 3);
    const int pass = kRopeCols + 8 * (c - 12) + j;
    return rope ? (c < 12 ? rot : pass) : 8 * c + j;      // selects, no branches
}

// The B row order that produces that layout with the 64 x 128 wave tiles (AccW): local row
// L = 128 h + 16 j + c of the B slot is weight row n0 + 128 h + qkv_dim(j, c).
__host__ __device__ constexpr int qkv_brow(int L, bool rope) {
    return 128 * (L >> 7) + qkv_dim((L >> 4) & 7, L & 15, rope);
}
struct QkvBRows {
    static constexpr bool kMapped = true;
    bool rope;
    __device__ __forceinline__ int row(int L) const { return qkv_brow(L, rope); }
};
// The order is a permutation of the tile's 256 rows, and it keeps the fills' form: within each
// 8-row fill piece the rows step from the piece's first row the same way in pieces p and p + 2
// of a wave (by 4 for rotated dims, by 8 for pass-through and V dims).
static_assert(brow_map_ok([](int L) { return qkv_brow(L, true); }) &&
                  brow_map_ok([](int L) { return qkv_brow(L, false); }),
              "QKV B row order");

// e4m3 output mode ("minimax_h3_nvfp4_pre_attention", Parameters: out_mode "e4m3" with
// per-tensor q/k/v dequantization scales): 4 bf16 values (two packed pairs) become
// e4m3(fl32(v / ds)), saturating at 448, little-endian in one word; y = RN(1 / ds).
__device__ __forceinline__ uint32_t e4m3_codes4(uint32_t p0, uint32_t p1, float ds, float y) {
    return f2e4m3x2(div_sat(bf_lo(p0), ds, y), div_sat(bf_hi(p0), ds, y)) |
           (f2e4m3x2(div_sat(bf_lo(p1), ds, y), div_sat(bf_hi(p1), ds, y)) << 16);
}

// The QKV epilogue of one 256 x 256 tile straight from the accumulators (AccW, B rows in
// QkvBRows order): wave (wm, h) holds rows 64 wm + 16 i + 4 (l / 16) + r (i, r = 0..3) of the
// tile's head h, lane l the 8 dims qkv_dim(j, l % 16) of each.  The 16 lanes of a DPP row hold
// the same 4 rows, so a row's sum of squares over the head is one 4-step DPP reduction, and
// RoPE pairs need no lane exchange.  No LDS and no barrier: G0 runs it while G1 finishes its
// last compute phase.  Per row: u = bf16((v w) r2) with r2 = rsqrt(mean(v^2) + qk_eps), then
// o_d = u_d c - u_(d+48) s, o_(d+48) = u_(d+48) c + u_d s for d < 48, with c, s the cos and sin
// of frequency d at the row's position; V as is.  Stores: 4 contiguous dims at a time (Q/K) or
// 8 (V), into out[dst, m, hl, kind, :].
template <bool kE4m3>
__device__ __forceinline__ void qkv_epilogue_regs(const AccW& acc, int64_t m0, int64_t M, int n0,
                                                  const uint16_t* __restrict__ qw, const uint16_t* __restrict__ kw,
                                                  const uint16_t* __restrict__ cs, int64_t S,
                                                  const int64_t* __restrict__ pos, float qk_eps, int hpd, float dq,
                                                  float dk, float dv, void* __restrict__ out) {
    const int t = opaque_tid();
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // uniform: the output descriptor uses it
    const int wm = wave / AccW::kWavesN, h = wave % AccW::kWavesN;
    const int c = lane & 15, rq = lane >> 4;
    const int kind = n0 / kAttnWidth;              // 0 q, 1 k, 2 v (uniform)
    const bool rope = kind < 2;
    const bool rot = rope && c < 12;               // this lane's dims are rotated
    const int head = (n0 % kAttnWidth) / kHeadDim + h;
    const int dst = head / hpd, hl = head - dst * hpd;
    const int64_t tile_rows = M - m0 < kBM ? M - m0 : kBM;
    constexpr int kElemB = kE4m3 ? 1 : 2;
    constexpr int kGroup = 3 * kHeadDim;           // elements of one (token, head): q, k, v
    const int row_el = hpd * kGroup;               // elements of one row of a destination
    // destination dst's rows of this tile, out[dst, m0 .., :, :, :] (rows past M dropped)
    uint8_t* const obase = static_cast<uint8_t*>(out) + ((int64_t)dst * M + m0) * row_el * kElemB;
    const __amdgpu_buffer_rsrc_t rout = make_rsrc(obase, (uint32_t)(tile_rows * row_el * kElemB));
    const int d0 = qkv_dim(0, c, rope), d1 = qkv_dim(4, c, rope);   // dims of blocks 0-3, 4-7
    const int rbase = wm * AccW::kRows + 4 * rq;    // + 16 i + r: this lane's rows
    // byte offsets of this lane's two 4-dim pieces in its first row; a row adds row_el elements
    const int ohead = (hl * 3 + kind) * kHeadDim;
    const uint32_t vo0 = (uint32_t)((rbase * row_el + ohead + d0) * kElemB);
    const uint32_t vo1 = (uint32_t)((rbase * row_el + ohead + d1) * kElemB);
    const float ds = kind == 0 ? dq : (kind == 1 ? dk : dv);
    const float ds_inv = kE4m3 ? 1.0f / ds : 0.0f;

    // The 16 lanes of a DPP row share their 16 rows: lane c takes the position of row
    // (i, r) = (c / 4, c % 4) of them, clamped to [0, S), as the byte offset of its cos/sin row
    // (requested first: the cos/sin loads depend on it), and hands it to the others
    // (ds_bpermute).
    const int64_t prow = m0 + rbase + 16 * (c >> 2) + (c & 3);
    uint32_t csrow_own = 0u;
    if (rope) {
        int64_t p = prow;                                 // identity positions: the row
        if (pos != nullptr) {
            const __amdgpu_buffer_rsrc_t rpos = make_rsrc(pos, (uint32_t)(M * 8));
            p = buf_ld_i64(rpos, (uint32_t)(prow * 8));
        }
        const int64_t pc = p < 0 ? 0 : (p > S - 1 ? S - 1 : p);
        csrow_own = (uint32_t)pc * (uint32_t)(kRopeCols * 2);
    }
    // norm weights of the lane's dims, bf16 pairs with one half zeroed
    u32x4 nwlo, nwhi;
    {
        const uint16_t* nw = kind == 0 ? qw : kw;
        u32x2 w0 = {0u, 0u}, w1 = {0u, 0u};
        if (rope) {
            w0 = *reinterpret_cast<const u32x2*>(nw + d0);
            w1 = *reinterpret_cast<const u32x2*>(nw + d1);
        }
        const uint32_t wv[4] = {w0.x, w0.y, w1.x, w1.y};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            nwlo[e] = wv[e] & 0xFFFFu;
            nwhi[e] = wv[e] & 0xFFFF0000u;
        }
    }
    // The phases below are kept in this order (scheduling barriers): the accumulators become
    // packed bf16 before the cos/sin rows are requested, so the two never hold registers at once.
    __builtin_amdgcn_sched_barrier(0);
    // the rows as bf16 (the GEMM output), packed: vp[i][r][e] = (v_2e, v_2e+1), blocks 2e, 2e+1
    u32x4 vp[AccW::MB][4];
#pragma unroll
    for (int i = 0; i < AccW::MB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) vp[i][r][e] = pack_bf2(acc.v[i][2 * e][r], acc.v[i][2 * e + 1][r]);

    if (!rope) {
#pragma unroll
        for (int i = 0; i < AccW::MB; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t e0 = vo0 + (uint32_t)((16 * i + r) * row_el * kElemB);
                if constexpr (kE4m3) {
                    const u32x2 q = {e4m3_codes4(vp[i][r][0], vp[i][r][1], ds, ds_inv),
                                     e4m3_codes4(vp[i][r][2], vp[i][r][3], ds, ds_inv)};
                    __builtin_amdgcn_raw_buffer_store_b64(q, rout, (int)e0, 0, 0);
                } else {
                    buf_st16(rout, e0, vp[i][r]);
                }
            }
        return;
    }

    // this lane's cos (frequencies d0 .. d0 + 3) and sin of a row block's 4 rows, requested one
    // block ahead (the 16 rows' at once would not fit in the registers beside the values).
    // Pass-through lanes rotate by the identity: cos 1 (set below), sin 0 (no load: zeros).
    const __amdgpu_buffer_rsrc_t rcs = make_rsrc(cs, (uint32_t)(S * kRopeCols * 2));
    const uint32_t cs_col = (uint32_t)(d0 * 2);
    const uint32_t one = rot ? 0u : 0x3F803F80u;
    auto load_cs = [&](int i, u32x2 (&cv)[4], u32x2 (&sv)[4]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            // the cos/sin row of row (i, r), from lane 4 i + r of this DPP row
            const uint32_t oc =
                (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (16 * rq + 4 * i + r), (int)csrow_own) + cs_col;
            const auto cw = __builtin_amdgcn_raw_buffer_load_b64(rcs, (int)(rot ? oc : kOffNone), 0, 0);
            const auto sw = __builtin_amdgcn_raw_buffer_load_b64(rcs, (int)(rot ? oc + kNFreq * 2 : kOffNone), 0, 0);
            cv[r] = u32x2{(uint32_t)cw[0], (uint32_t)cw[1]};
            sv[r] = u32x2{(uint32_t)sw[0], (uint32_t)sw[1]};
        }
    };
    u32x2 cv_nx[4], sv_nx[4];
    load_cs(0, cv_nx, sv_nx);
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int i = 0; i < AccW::MB; ++i) {
        u32x2 cvi[4], svi[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            cvi[r] = cv_nx[r];
            svi[r] = sv_nx[r];
        }
        if (i + 1 < AccW::MB) load_cs(i + 1, cv_nx, sv_nx);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const u32x4& v = vp[i][r];
            // 1 / rms over the head: this lane's 8 squares (exact bf16 products, accumulated by
            // v_dot2), then the 16 lanes of the DPP row
            const float sq = dot2_bf16(v[3], v[3], dot2_bf16(v[2], v[2], dot2_bf16(v[1], v[1], dot2_bf16(v[0], v[0]))));
            const float r2 = __builtin_amdgcn_rsqf(row16_sum(sq) * (1.0f / kHeadDim) + qk_eps);
            // u = bf16((v w) r2): v w exact (v_dot2 with one half of w zeroed)
            float vw[8], u[8];
            dot2x4_zero(v[0], nwlo[0], v[0], nwhi[0], v[1], nwlo[1], v[1], nwhi[1], *reinterpret_cast<float(*)[4]>(vw));
            dot2x4_zero(v[2], nwlo[2], v[2], nwhi[2], v[3], nwlo[3], v[3], nwhi[3],
                        *reinterpret_cast<float(*)[4]>(vw + 4));
#pragma unroll
            for (int e = 0; e < 8; ++e) u[e] = vw[e] * r2;
            // RoPE on the bf16 u: pairs (u_e, u_4+e) of dims (d0 + e, d1 + e) against (c_e, s_e)
            uint32_t ua[4], ub[4], csp[4];
            const uint32_t cw0 = cvi[r].x | one, cw1 = cvi[r].y | one;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ua[e] = pack_bf2(u[e], u[4 + e]);
                ub[e] = pack_bf2(u[4 + e], u[e]);
                const uint32_t sel = (e & 1) ? kPermHi : kPermLo;
                csp[e] = __builtin_amdgcn_perm(e < 2 ? svi[r].x : svi[r].y, e < 2 ? cw0 : cw1, sel);
            }
            float o[8];
            rope_dot2x8(ua, ub, csp, o);
            const u32x4 res = pack8(o);
            const uint32_t roff = (uint32_t)((16 * i + r) * row_el * kElemB);
            if constexpr (kE4m3) {
                __builtin_amdgcn_raw_buffer_store_b32(e4m3_codes4(res[0], res[1], ds, ds_inv), rout, (int)(vo0 + roff),
                                                      0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(e4m3_codes4(res[2], res[3], ds, ds_inv), rout, (int)(vo1 + roff),
                                                      0, 0);
            } else {
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{res[0], res[1]}, rout, (int)(vo0 + roff), 0, kStoreNt);
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{res[2], res[3]}, rout, (int)(vo1 + roff), 0, kStoreNt);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The QKV epilogue of one MXFP4 tile (acc of this wave, 128 x 64 wave tiles) through LDS: Q/K
// RMSNorm, RoPE and the pack into bf16 out, or V as is.  The 16 lanes of one DPP row own one
// (row, head), 8 dims each, and a 4-step DPP reduction gives the head's sum of squares.  The
// chunks are placed so that the RoPE partner (pairs (j, j+48), i.e. chunk c and c + 6 for c < 6)
// is always 8 lanes away: lanes 0-5 hold chunks 0-5, lanes 8-13 chunks 6-11, and lanes 6, 7,
// 14, 15 the pass-through chunks 12-15.  One row rotation by 8 then fetches every partner, with
// no lane-dependent choice (a DPP move must run with its source lanes active, which a select
// lowered to a branch would break).  Each lane writes 16 contiguous bytes of out, so the 16
// lanes of a head store its 256 bytes in one piece.
__device__ __forceinline__ void qkv_epilogue_staged(AccMx& acc, uint8_t* smem, int64_t m0, int64_t M, int n0,
                                                    const uint16_t* __restrict__ qw,
                                                    const uint16_t* __restrict__ kw, const uint16_t* __restrict__ cs,
                                                    int64_t S, const int64_t* __restrict__ pos, float qk_eps,
                                                    int hpd, void* __restrict__ out) {
    const int t = opaque_tid();
    const int li = t & 15;              // lane within the (row, head) group
    // 8-dim chunk of the head held by this lane (partner chunk q +/- 6 sits at lane li ^ 8)
    const int q = chunk_of_lane(li);
    const int hh = (t >> 4) & 1;        // which of the tile's two heads
    const int rsub = t >> 5;            // 0..kThreads/32-1
    const int kind = n0 / kAttnWidth;   // 0 q, 1 k, 2 v
    const int head = (n0 % kAttnWidth) / kHeadDim + hh;
    // destination-major pack: destination dst takes heads [dst * hpd, (dst + 1) * hpd) of every
    // token (hpd = 56 / P), out[dst, m, hl, kind, :]
    const int dst = head / hpd, hl = head - dst * hpd;
    const int d0 = q * 8;
    const int j0 = (q % 6) * 8;         // frequency index of this chunk (q < 12)

    // Every global operand of the epilogue is requested before it is needed, so the loop
    // below pays one memory latency per tile rather than one per row: the positions of this
    // thread's kIters rows now (they land while the accumulators are staged), the cos/sin
    // rows right after the staging.  All epilogue loads and stores go through buffer descriptors and are
    // issued unconditionally (out-of-range lanes read zeros, stores past M are dropped).
    constexpr int kRowsPerPass = kThreads / 32;
    constexpr int kIters = kBM / kRowsPerPass;
    const bool need_cs = kind < 2 && q < 12;
    const __amdgpu_buffer_rsrc_t rcs = make_rsrc(cs, kind < 2 ? (uint32_t)(S * kRopeCols * 2) : 0u);
    const __amdgpu_buffer_rsrc_t rpos = make_rsrc(pos, pos ? (uint32_t)(M * 8) : 0u);
    const int64_t tile_rows = M - m0 < kBM ? M - m0 : kBM;
    constexpr int64_t kOutRow = (int64_t)kHeads * 3 * kHeadDim;        // elements per token
    constexpr int64_t kElemB = 2;                                     // bytes per output element
    uint8_t* const out8 = static_cast<uint8_t*>(out);
    const __amdgpu_buffer_rsrc_t rout = make_rsrc(out8 + m0 * kOutRow * kElemB,
                                                  (uint32_t)(tile_rows * kOutRow * kElemB));
    // P = 1: byte offset (within the tile's rows) of this lane's 8 elements in the first pass;
    // each pass moves kRowsPerPass rows on
    const uint32_t o1 = (uint32_t)((((rsub * kHeads + head) * 3 + kind) * kHeadDim + d0) * kElemB);
    constexpr uint32_t kPassB = (uint32_t)(kRowsPerPass * kOutRow * kElemB);
    u32x4 nwv = {0u, 0u, 0u, 0u};       // this lane's 8 q/k norm weights
    if (kind < 2) nwv = ld16((kind == 0 ? qw : kw) + d0);
    int64_t praw[kIters];               // raw positions (read only when pos is given)
    if (pos != nullptr && kind < 2) {
#pragma unroll
        for (int it = 0; it < kIters; ++it)
            praw[it] = buf_ld_i64(rpos, (uint32_t)((m0 + it * kRowsPerPass + rsub) * 8));
    }

    stage_tile_bf16(acc, smem);
    // the cos/sin rows are requested once the accumulators are free and before the barrier, so
    // they are in flight while the other waves finish staging
    // this lane's half of the row's cos/sin: the cos chunk (q < 6) or the sin chunk (6 <= q < 12)
    const int cs_col = q < 6 ? j0 : kNFreq + j0;
    u32x4 csv[kIters];
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
        const int64_t m = m0 + it * kRowsPerPass + rsub;
        const int64_t p = pos != nullptr ? praw[it] : m;      // identity positions: the row
        const int64_t pc = p < 0 ? 0 : (p > S - 1 ? S - 1 : p);
        csv[it] = buf_ld16(rcs, need_cs ? (uint32_t)((pc * kRopeCols + cs_col) * 2) : kOffNone);
    }
    lds_barrier();

    u32x4 nwlo, nwhi;                   // the norm weights, one bf16 of each pair kept
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        nwlo[e] = nwv[e] & 0xFFFFu;
        nwhi[e] = nwv[e] & 0xFFFF0000u;
    }

#pragma unroll
    for (int it = 0; it < kIters; ++it) {
        const int row = it * kRowsPerPass + rsub;
        const u32x4 vp = epi_ld(smem, row, hh * 128 + d0);
        u32x4 o = vp;
        if (kind < 2) o = qk_norm_rope(vp, nwlo, nwhi, qk_eps, q, csv[it]);
        // one destination: rows past M fall outside rout and are dropped; else out[dst, m, hl, ...]
        const uint32_t e1 = o1 + (uint32_t)it * kPassB;
        const int64_t m = m0 + row;
        const int64_t eP = (((dst * M + m) * hpd + hl) * 3 + kind) * kHeadDim + d0;
        if (hpd == kHeads) {
            buf_st16(rout, e1, o);
        } else if (m < M) {
            st16_nt(out8 + eP * 2, o);
        }
    }
}

// kE4m3: out holds e4m3 codes (one byte per element) of the bf16 results divided by the
// descale of their kind (dq, dk, dv); else bf16 values (the descales are unused).
// Persistent: tiles are claimed from the queue tq (see TileQueue).
template <bool kE4m3>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void k_qkv_gemm(const uint16_t* __restrict__ ws, int64_t M, const uint16_t* __restrict__ W,
                const uint16_t* __restrict__ qw, const uint16_t* __restrict__ kw,
                const uint16_t* __restrict__ cs, int64_t S, const int64_t* __restrict__ pos, float qk_eps,
                int hpd, float dq, float dk, float dv, void* __restrict__ out, int mt, int nt, uint32_t* tq_ctr) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
    const TileQueue tq(tq_ctr, mt, nt);
    auto tile = [&](int k, TileOps& t, QkvBRows& bm) {
        int tm, tn;
        logical_coords(tq.lo + k, mt, nt, tm, tn);
        const int n0 = tn * kBN;
        t = TileOps{reinterpret_cast<const uint8_t*>(ws), kHidden * 2, (int64_t)tm * kBM, M,
                    reinterpret_cast<const uint8_t*>(W), kHidden * 2, n0, n0 + 128, kHidden * 2 / kRowB};
        bm = QkvBRows{n0 < 2 * kAttnWidth};
    };
    auto epi = [&](const AccW& acc, const TileOps& t) {
        qkv_epilogue_regs<kE4m3>(acc, t.m0, M, (int)t.nb0, qw, kw, cs, S, pos, qk_eps, hpd, dq, dk, dv, out);
    };
    persistent_tiles<Mma::kBf16, false, false, AccW, QkvBRows>(tq, smem, tile, epi);
}

// The same tile on MXFP4 operands: the workspace's and the weight's E2M1 codes ([M, 2688],
// [21504, 2688]) with their scales in the MX scale layout; bf16 output.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void k_qkv_gemm_mxfp4(const uint8_t* __restrict__ ws_codes, const uint8_t* __restrict__ ws_scales, uint32_t ws_sbytes,
                      int64_t M, const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales,
                      uint32_t w_sbytes, const uint16_t* __restrict__ qw, const uint16_t* __restrict__ kw,
                      const uint16_t* __restrict__ cs, int64_t S, const int64_t* __restrict__ pos, float qk_eps,
                      int hpd, void* __restrict__ out, int mt, int nt, uint32_t* tq_ctr) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmemBytes];
    MxScales mxs;
    mxs.a = ws_scales;
    mxs.a_bytes = ws_sbytes;
    mxs.b = w_scales;
    mxs.b_bytes = w_sbytes;
    constexpr int kRowBytes = kHidden / 2;
    const TileQueue tq(tq_ctr, mt, nt);
    tq.claim(smem);
    __syncthreads();
    for (int k = tq.claimed(smem); k < tq.cnt; k = tq.claimed(smem)) {
        int tm, tn;
        logical_coords(tq.lo + k, mt, nt, tm, tn);
        const int64_t m0 = (int64_t)tm * kBM;
        const int n0 = tn * kBN;
        AccMx acc;
        mainloop<Mma::kMxFp4>(ws_codes, kRowBytes, m0, M, w_codes, kRowBytes, n0, n0 + 128, kRowBytes / kRowB, smem,
                              acc, mxs);
        tq.claim(smem);
        qkv_epilogue_staged(acc, smem, m0, M, n0, qw, kw, cs, S, pos, qk_eps, hpd, out);
        __syncthreads();
    }
    tq.finish();
}

hipError_t launch_qkv_gemm(const uint16_t* ws, int64_t M, const uint16_t* W, const uint16_t* qw,
                           const uint16_t* kw, const uint16_t* cs, int64_t S, const int64_t* pos, float qk_eps,
                           int P, uint16_t* out, hipStream_t stream) {
    // up to 16 rows the weight stream bounds the launch: spread it over one workgroup per head
    if (M <= 16) return launch_qkv_small(ws, M, W, qw, kw, cs, S, pos, qk_eps, P, out, stream);
    const int mt = (int)((M + kBM - 1) / kBM);
    const int nt = kQkvRows / kBN;
    uint32_t* q = nullptr;
    int grid = 0;
    const hipError_t e = tile_queue(stream, &q, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_qkv_gemm<false>, dim3((unsigned)grid), dim3(kThreads), 0, stream, ws, M, W, qw, kw, cs, S,
                       pos, qk_eps, kHeads / P, 1.0f, 1.0f, 1.0f, out, mt, nt, q);
    return hipGetLastError();
}

hipError_t launch_qkv_gemm_mxfp4(const uint8_t* ws_codes, const uint8_t* ws_scales, int64_t M, const uint8_t* w_codes,
                                 const uint8_t* w_scales, const uint16_t* qw, const uint16_t* kw, const uint16_t* cs,
                                 int64_t S, const int64_t* pos, float qk_eps, int P, uint16_t* out,
                                 hipStream_t stream) {
    const int mt = (int)((M + kBM - 1) / kBM);
    const int nt = kQkvRows / kBN;
    const uint32_t a_sb = (uint32_t)mx_scale_bytes(M, kHidden);
    const uint32_t w_sb = (uint32_t)mx_scale_bytes(kQkvRows, kHidden);
    uint32_t* q = nullptr;
    int grid = 0;
    const hipError_t e = tile_queue(stream, &q, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_qkv_gemm_mxfp4, dim3((unsigned)grid), dim3(kThreads), 0, stream, ws_codes, ws_scales, a_sb, M,
                       w_codes, w_scales, w_sb, qw, kw, cs, S, pos, qk_eps, kHeads / P, out, mt, nt, q);
    return hipGetLastError();
}

hipError_t launch_qkv_gemm_e4m3(const uint16_t* ws, int64_t M, const uint16_t* W, const uint16_t* qw,
                                const uint16_t* kw, const uint16_t* cs, int64_t S, const int64_t* pos,
                                float qk_eps, int P, float dq, float dk, float dv, uint8_t* out, hipStream_t stream) {
    const int mt = (int)((M + kBM - 1) / kBM);
    const int nt = kQkvRows / kBN;
    uint32_t* q = nullptr;
    int grid = 0;
    const hipError_t e = tile_queue(stream, &q, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_qkv_gemm<true>, dim3((unsigned)grid), dim3(kThreads), 0, stream, ws, M, W, qw, kw, cs, S, pos,
                       qk_eps, kHeads / P, dq, dk, dv, out, mt, nt, q);
    return hipGetLastError();
}

}  // namespace dit
