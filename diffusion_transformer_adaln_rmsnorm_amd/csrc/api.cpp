// C ABI entry points: host-side contract checks, then the kernel launches, all on the
// caller's stream.  Nothing here allocates, copies, or synchronises.
#include <hip/hip_runtime_api.h>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include "../../include/dit.h"
#include "kernels.hpp"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool eps_ok(float e) { return isfinite(e) && e > 0.f; }
// A per-tensor e4m3 descale divides each output; its reciprocal must be a finite float, which
// every normal float has (1 / FLT_MIN = 2^126) and some subnormals do not.
bool descale_ok(float d) { return isfinite(d) && d >= FLT_MIN; }

dit_status check_table(const dit_bf16_table& t) {
    if (!t.ptr) return DIT_ERR_NULL;
    if (!aligned(t.ptr, 16)) return DIT_ERR_ALIGN;
    if (t.rows < 1 || t.rows > INT32_MAX) return DIT_ERR_SHAPE;      // row numbers fit 32 bits on the device
    if (t.row_stride < DIT_HIDDEN || (t.row_stride & 7) != 0) return DIT_ERR_STRIDE;
    return DIT_OK;
}

dit_status launched(hipError_t e) { return e == hipSuccess ? DIT_OK : DIT_ERR_LAUNCH; }

// Upper row bound: keeps every grid below 2^32 work-items (x alone is 180 GB at this M).
constexpr int64_t kMaxRows = (int64_t)1 << 24;
// Upper bound on the rows S of the [S, 96] bf16 cos/sin cache: the QKV epilogue reads it
// through one buffer descriptor, whose byte range and offsets are 32-bit (S * 192 < 2^32).
constexpr int64_t kMaxRopeRows = (int64_t)0xFFFFFFFF / (DIT_ROPE_COLS * 2);

}  // namespace

extern "C" {

const char* dit_status_string(int s) {
    switch (s) {
        case DIT_OK: return "ok";
        case DIT_ERR_NULL: return "required pointer is NULL";
        case DIT_ERR_SHAPE: return "size out of range";
        case DIT_ERR_ALIGN: return "pointer not aligned";
        case DIT_ERR_STRIDE: return "bad table row stride";
        case DIT_ERR_UNSUPPORTED: return "unsupported argument value";
        case DIT_ERR_LAUNCH: return "kernel launch failed";
        case DIT_ERR_VALUE: return "invalid scalar argument";
        default: return "unknown status";
    }
}

int dit_abi_version(void) { return 100; }

int64_t dit_mlp_fp8_flags_elems(int64_t M) {
    (void)M;
    return 0;
}

dit_status dit_norm_adaln_bf16(const void* x, int64_t M, const void* x_norm_weight, dit_bf16_table adaln_scale,
                               dit_bf16_table adaln_shift, const int64_t* adaln_index, float eps, void* workspace,
                               void* stream) {
    if (!eps_ok(eps)) return DIT_ERR_VALUE;
    if (M < 0 || M > kMaxRows) return DIT_ERR_SHAPE;
    if (!x || !x_norm_weight || !adaln_index || !workspace) return DIT_ERR_NULL;
    dit_status st = check_table(adaln_scale);
    if (st != DIT_OK) return st;
    st = check_table(adaln_shift);
    if (st != DIT_OK) return st;
    if (adaln_scale.rows != adaln_shift.rows) return DIT_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(x_norm_weight, 16) || !aligned(workspace, 16) || !aligned(adaln_index, 8))
        return DIT_ERR_ALIGN;
    if (M == 0) return DIT_OK;
    return launched(dit::launch_norm_adaln_bf16(
        static_cast<const uint16_t*>(x), M, static_cast<const uint16_t*>(x_norm_weight),
        static_cast<const uint16_t*>(adaln_scale.ptr), adaln_scale.row_stride,
        static_cast<const uint16_t*>(adaln_shift.ptr), adaln_shift.row_stride, adaln_scale.rows, adaln_index, eps,
        static_cast<uint16_t*>(workspace), static_cast<hipStream_t>(stream)));
}

// Checks and launch of the QKV GEMM (launch 2), bf16 output (descales null) or e4m3 codes.
static dit_status qkv_rope_pack(const void* workspace, int64_t M, const void* qkv_weight, const void* q_norm_weight,
                                const void* k_norm_weight, const void* rope_cos_sin, int64_t S,
                                const int64_t* rope_positions, int ulysses_degree, float qk_eps, const float* descale,
                                void* out, void* stream) {
    if (ulysses_degree != 1 && ulysses_degree != 2 && ulysses_degree != 4 && ulysses_degree != 8)
        return DIT_ERR_VALUE;
    if (!eps_ok(qk_eps)) return DIT_ERR_VALUE;
    if (descale && (!descale_ok(descale[0]) || !descale_ok(descale[1]) || !descale_ok(descale[2])))
        return DIT_ERR_VALUE;
    if (M < 0 || M > kMaxRows) return DIT_ERR_SHAPE;
    if (!workspace || !qkv_weight || !q_norm_weight || !k_norm_weight || !rope_cos_sin || !out) return DIT_ERR_NULL;
    if (!aligned(workspace, 16) || !aligned(qkv_weight, 16) || !aligned(q_norm_weight, 16) ||
        !aligned(k_norm_weight, 16) || !aligned(rope_cos_sin, 16) || !aligned(out, 16) ||
        (rope_positions && !aligned(rope_positions, 8)))
        return DIT_ERR_ALIGN;
    if (S < 1 || S > kMaxRopeRows) return DIT_ERR_SHAPE;
    if (!rope_positions && S < M) return DIT_ERR_SHAPE;
    if (M == 0) return DIT_OK;
    const uint16_t* ws = static_cast<const uint16_t*>(workspace);
    const uint16_t* W = static_cast<const uint16_t*>(qkv_weight);
    const uint16_t* qw = static_cast<const uint16_t*>(q_norm_weight);
    const uint16_t* kw = static_cast<const uint16_t*>(k_norm_weight);
    const uint16_t* cs = static_cast<const uint16_t*>(rope_cos_sin);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (descale)
        return launched(dit::launch_qkv_gemm_e4m3(ws, M, W, qw, kw, cs, S, rope_positions, qk_eps, ulysses_degree,
                                                  descale[0], descale[1], descale[2], static_cast<uint8_t*>(out),
                                                  st));
    return launched(dit::launch_qkv_gemm(ws, M, W, qw, kw, cs, S, rope_positions, qk_eps, ulysses_degree,
                                         static_cast<uint16_t*>(out), st));
}

// Both launches; every argument is checked before either is enqueued.
static dit_status pre_attn(const void* x, int64_t M, const void* x_norm_weight, dit_bf16_table adaln_scale,
                           dit_bf16_table adaln_shift, const int64_t* adaln_index, const void* qkv_weight,
                           const void* q_norm_weight, const void* k_norm_weight, const void* rope_cos_sin, int64_t S,
                           const int64_t* rope_positions, int ulysses_degree, float eps, float qk_eps,
                           const float* descale, void* workspace, void* out, void* stream) {
    if (ulysses_degree != 1 && ulysses_degree != 2 && ulysses_degree != 4 && ulysses_degree != 8)
        return DIT_ERR_VALUE;
    if (!eps_ok(eps) || !eps_ok(qk_eps)) return DIT_ERR_VALUE;
    if (descale && (!descale_ok(descale[0]) || !descale_ok(descale[1]) || !descale_ok(descale[2])))
        return DIT_ERR_VALUE;
    if (M < 0 || M > kMaxRows) return DIT_ERR_SHAPE;
    if (!x || !x_norm_weight || !adaln_index || !qkv_weight || !q_norm_weight || !k_norm_weight ||
        !rope_cos_sin || !workspace || !out)
        return DIT_ERR_NULL;
    dit_status st = check_table(adaln_scale);
    if (st != DIT_OK) return st;
    st = check_table(adaln_shift);
    if (st != DIT_OK) return st;
    if (adaln_scale.rows != adaln_shift.rows) return DIT_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(x_norm_weight, 16) || !aligned(qkv_weight, 16) || !aligned(q_norm_weight, 16) ||
        !aligned(k_norm_weight, 16) || !aligned(rope_cos_sin, 16) || !aligned(workspace, 16) || !aligned(out, 16) ||
        !aligned(adaln_index, 8) || (rope_positions && !aligned(rope_positions, 8)))
        return DIT_ERR_ALIGN;
    if (S < 1 || S > kMaxRopeRows) return DIT_ERR_SHAPE;
    if (!rope_positions && S < M) return DIT_ERR_SHAPE;
    if (M == 0) return DIT_OK;
    st = dit_norm_adaln_bf16(x, M, x_norm_weight, adaln_scale, adaln_shift, adaln_index, eps, workspace, stream);
    if (st != DIT_OK) return st;
    return qkv_rope_pack(workspace, M, qkv_weight, q_norm_weight, k_norm_weight, rope_cos_sin, S, rope_positions,
                         ulysses_degree, qk_eps, descale, out, stream);
}

dit_status dit_qkv_rope_pack_bf16(const void* workspace, int64_t M, const void* qkv_weight,
                                  const void* q_norm_weight, const void* k_norm_weight, const void* rope_cos_sin,
                                  int64_t S, const int64_t* rope_positions, int ulysses_degree, float qk_eps,
                                  void* out, void* stream) {
    return qkv_rope_pack(workspace, M, qkv_weight, q_norm_weight, k_norm_weight, rope_cos_sin, S, rope_positions,
                         ulysses_degree, qk_eps, nullptr, out, stream);
}

dit_status dit_qkv_rope_pack_e4m3(const void* workspace, int64_t M, const void* qkv_weight,
                                  const void* q_norm_weight, const void* k_norm_weight, const void* rope_cos_sin,
                                  int64_t S, const int64_t* rope_positions, int ulysses_degree, float qk_eps,
                                  float q_descale, float k_descale, float v_descale, void* out, void* stream) {
    const float d[3] = {q_descale, k_descale, v_descale};
    return qkv_rope_pack(workspace, M, qkv_weight, q_norm_weight, k_norm_weight, rope_cos_sin, S, rope_positions,
                         ulysses_degree, qk_eps, d, out, stream);
}

dit_status dit_pre_attn_bf16(const void* x, int64_t M, const void* x_norm_weight, dit_bf16_table adaln_scale,
                             dit_bf16_table adaln_shift, const int64_t* adaln_index, const void* qkv_weight,
                             const void* q_norm_weight, const void* k_norm_weight, const void* rope_cos_sin,
                             int64_t S, const int64_t* rope_positions, int ulysses_degree, float eps, float qk_eps,
                             void* workspace, void* out, void* stream) {
    return pre_attn(x, M, x_norm_weight, adaln_scale, adaln_shift, adaln_index, qkv_weight, q_norm_weight,
                    k_norm_weight, rope_cos_sin, S, rope_positions, ulysses_degree, eps, qk_eps, nullptr, workspace, out,
                    stream);
}

dit_status dit_pre_attn_e4m3(const void* x, int64_t M, const void* x_norm_weight, dit_bf16_table adaln_scale,
                             dit_bf16_table adaln_shift, const int64_t* adaln_index, const void* qkv_weight,
                             const void* q_norm_weight, const void* k_norm_weight, const void* rope_cos_sin,
                             int64_t S, const int64_t* rope_positions, int ulysses_degree, float eps, float qk_eps,
                             float q_descale, float k_descale, float v_descale, void* workspace, void* out,
                             void* stream) {
    const float d[3] = {q_descale, k_descale, v_descale};
    return pre_attn(x, M, x_norm_weight, adaln_scale, adaln_shift, adaln_index, qkv_weight, q_norm_weight,
                    k_norm_weight, rope_cos_sin, S, rope_positions, ulysses_degree, eps, qk_eps, d, workspace, out,
                    stream);
}

dit_status dit_out_proj_gated_bf16(const void* attn_out, int64_t M, const void* o_weight, dit_bf16_table gate,
                                   const int32_t* gate_index, const void* residual, void* out, void* stream) {
    if (M < 0 || M > kMaxRows) return DIT_ERR_SHAPE;
    if (!attn_out || !o_weight || !gate_index || !residual || !out) return DIT_ERR_NULL;
    dit_status st = check_table(gate);
    if (st != DIT_OK) return st;
    if (!aligned(attn_out, 16) || !aligned(o_weight, 16) || !aligned(residual, 16) || !aligned(out, 16) ||
        !aligned(gate_index, 4))
        return DIT_ERR_ALIGN;
    if (M == 0) return DIT_OK;
    return launched(dit::launch_out_proj_gemm(
        static_cast<const uint16_t*>(attn_out), M, static_cast<const uint16_t*>(o_weight),
        static_cast<const uint16_t*>(gate.ptr), gate.rows, gate.row_stride, gate_index,
        static_cast<const uint16_t*>(residual), static_cast<uint16_t*>(out), static_cast<hipStream_t>(stream)));
}

dit_status dit_pre_attn_mxfp4(const void* x, int64_t M, const void* x_norm_weight, dit_bf16_table adaln_scale,
                              dit_bf16_table adaln_shift, const int64_t* adaln_index, const uint8_t* w_codes,
                              const uint8_t* w_scales, const void* q_norm_weight, const void* k_norm_weight,
                              const void* rope_cos_sin, int64_t S, const int64_t* rope_positions, int ulysses_degree,
                              float eps, float qk_eps, uint8_t* ws_codes, uint8_t* ws_scales, void* out,
                              void* stream) {
    if (ulysses_degree != 1 && ulysses_degree != 2 && ulysses_degree != 4 && ulysses_degree != 8)
        return DIT_ERR_VALUE;
    if (!eps_ok(eps) || !eps_ok(qk_eps)) return DIT_ERR_VALUE;
    if (M < 0 || M > kMaxRows) return DIT_ERR_SHAPE;
    if (!x || !x_norm_weight || !adaln_index || !w_codes || !w_scales || !q_norm_weight || !k_norm_weight ||
        !rope_cos_sin || !ws_codes || !ws_scales || !out)
        return DIT_ERR_NULL;
    dit_status st = check_table(adaln_scale);
    if (st != DIT_OK) return st;
    st = check_table(adaln_shift);
    if (st != DIT_OK) return st;
    if (adaln_scale.rows != adaln_shift.rows) return DIT_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(x_norm_weight, 16) || !aligned(w_codes, 16) || !aligned(w_scales, 16) ||
        !aligned(q_norm_weight, 16) || !aligned(k_norm_weight, 16) || !aligned(rope_cos_sin, 16) ||
        !aligned(ws_codes, 16) || !aligned(ws_scales, 16) || !aligned(out, 16) || !aligned(adaln_index, 8) ||
        (rope_positions && !aligned(rope_positions, 8)))
        return DIT_ERR_ALIGN;
    if (S < 1 || S > kMaxRopeRows) return DIT_ERR_SHAPE;
    if (!rope_positions && S < M) return DIT_ERR_SHAPE;
    if (M == 0) return DIT_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = launched(dit::launch_norm_adaln_mxfp4(
        static_cast<const uint16_t*>(x), M, static_cast<const uint16_t*>(x_norm_weight),
        static_cast<const uint16_t*>(adaln_scale.ptr), adaln_scale.row_stride,
        static_cast<const uint16_t*>(adaln_shift.ptr), adaln_shift.row_stride, adaln_scale.rows, adaln_index, eps,
        ws_codes, ws_scales, s));
    if (st != DIT_OK) return st;
    return launched(dit::launch_qkv_gemm_mxfp4(ws_codes, ws_scales, M, w_codes, w_scales,
                                               static_cast<const uint16_t*>(q_norm_weight),
                                               static_cast<const uint16_t*>(k_norm_weight),
                                               static_cast<const uint16_t*>(rope_cos_sin), S, rope_positions, qk_eps,
                                               ulysses_degree, static_cast<uint16_t*>(out), s));
}

int64_t dit_mx_scale_bytes(int64_t rows, int64_t K) {
    if (rows < 0 || K < 0) return 0;
    return dit::mx_scale_bytes(rows, K);
}

dit_status dit_mx_quant_fp4(const void* x, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales, void* stream) {
    if (rows < 0 || K < 256 || K % 256 != 0) return DIT_ERR_SHAPE;
    // one thread per 32-value block of the padded rows: the grid must fit 2^31 threads
    if ((rows + 127) / 128 * 128 > ((int64_t)1 << 31) / (K / 32)) return DIT_ERR_SHAPE;
    if (!x || !codes || !scales) return DIT_ERR_NULL;
    if (!aligned(x, 16) || !aligned(codes, 16)) return DIT_ERR_ALIGN;
    if (rows == 0) return DIT_OK;
    return launched(dit::launch_mx_quant_fp4(static_cast<const uint16_t*>(x), rows, K, codes, scales,
                                             static_cast<hipStream_t>(stream)));
}

dit_status dit_out_proj_gated_mxfp4(const void* attn_out, int64_t M, const uint8_t* w_codes, const uint8_t* w_scales,
                                    dit_bf16_table gate, const int32_t* gate_index, const void* residual,
                                    uint8_t* act_codes, uint8_t* act_scales, void* out, void* stream) {
    if (M < 0 || M > kMaxRows) return DIT_ERR_SHAPE;
    if (!attn_out || !w_codes || !w_scales || !gate_index || !residual || !act_codes || !act_scales || !out)
        return DIT_ERR_NULL;
    dit_status st = check_table(gate);
    if (st != DIT_OK) return st;
    if (!aligned(attn_out, 16) || !aligned(w_codes, 16) || !aligned(residual, 16) || !aligned(out, 16) ||
        !aligned(act_codes, 16) || !aligned(w_scales, 16) || !aligned(act_scales, 16) || !aligned(gate_index, 4))
        return DIT_ERR_ALIGN;
    if (M == 0) return DIT_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = launched(dit::launch_mx_quant_fp4(static_cast<const uint16_t*>(attn_out), M, DIT_ATTN_WIDTH, act_codes,
                                           act_scales, s));
    if (st != DIT_OK) return st;
    return launched(dit::launch_out_proj_mxfp4(act_codes, act_scales, M, w_codes, w_scales,
                                               static_cast<const uint16_t*>(gate.ptr), gate.rows, gate.row_stride,
                                               gate_index, static_cast<const uint16_t*>(residual),
                                               static_cast<uint16_t*>(out), s));
}

dit_status dit_mlp_fp8(const void* x, int64_t M, const void* x_norm_weight, dit_bf16_table adaln_scale,
                       dit_bf16_table adaln_shift, dit_bf16_table gate, const int64_t* adaln_index,
                       const void* residual, const uint8_t* fc1_q, const float* fc1_scale, const uint8_t* fc2_q,
                       const float* fc2_scale, float eps, uint8_t* ws_a_q, float* ws_a_scale, void* ws_y,
                       uint8_t* ws_y_q, float* ws_y_scale, int32_t* ws_flags, void* out, void* stream) {
    (void)ws_flags;
    if (!eps_ok(eps)) return DIT_ERR_VALUE;
    if (M < 1 || M > DIT_MLP_MAX_M) return DIT_ERR_SHAPE;
    if (!x || !x_norm_weight || !adaln_index || !residual || !fc1_q || !fc1_scale || !fc2_q || !fc2_scale ||
        !ws_a_q || !ws_a_scale || !ws_y || !ws_y_q || !ws_y_scale || !out)
        return DIT_ERR_NULL;
    dit_status st;
    if ((st = check_table(adaln_scale)) != DIT_OK) return st;
    if ((st = check_table(adaln_shift)) != DIT_OK) return st;
    if ((st = check_table(gate)) != DIT_OK) return st;
    if (adaln_scale.rows != adaln_shift.rows || adaln_scale.rows != gate.rows) return DIT_ERR_SHAPE;
    if (adaln_scale.row_stride != adaln_shift.row_stride) return DIT_ERR_STRIDE;
    if (!aligned(x, 16) || !aligned(x_norm_weight, 16) || !aligned(residual, 16) || !aligned(fc1_q, 16) ||
        !aligned(fc2_q, 16) || !aligned(ws_a_q, 16) || !aligned(ws_y, 16) || !aligned(ws_y_q, 16) ||
        !aligned(out, 16) || !aligned(adaln_index, 8) || !aligned(fc1_scale, 4) || !aligned(fc2_scale, 4) ||
        !aligned(ws_a_scale, 4) || !aligned(ws_y_scale, 4))
        return DIT_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint16_t* xs = static_cast<const uint16_t*>(x);
    st = launched(dit::launch_norm_adaln_fp8q(
        xs, M, static_cast<const uint16_t*>(x_norm_weight), static_cast<const uint16_t*>(adaln_scale.ptr),
        adaln_scale.row_stride, static_cast<const uint16_t*>(adaln_shift.ptr), adaln_shift.row_stride,
        adaln_scale.rows, adaln_index, eps, ws_a_q, ws_a_scale, s));
    if (st != DIT_OK) return st;
    st = launched(dit::launch_fc1_swiglu(ws_a_q, ws_a_scale, M, fc1_q, fc1_scale, static_cast<uint16_t*>(ws_y), s));
    if (st != DIT_OK) return st;
    if (dit::fc2_fused_fits(M))
        return launched(dit::launch_fc2_fused(static_cast<const uint16_t*>(ws_y), ws_y_scale, ws_y_q, M, fc2_q,
                                              fc2_scale, static_cast<const uint16_t*>(gate.ptr), gate.rows,
                                              gate.row_stride, adaln_index, static_cast<const uint16_t*>(residual),
                                              static_cast<uint16_t*>(out), s));
    st = launched(dit::launch_quant_rows(static_cast<const uint16_t*>(ws_y), M, ws_y_scale, ws_y_q, s));
    if (st != DIT_OK) return st;
    return launched(dit::launch_fc2_gated(ws_y_q, ws_y_scale, M, fc2_q, fc2_scale,
                                          static_cast<const uint16_t*>(gate.ptr), gate.rows, gate.row_stride,
                                          adaln_index, static_cast<const uint16_t*>(residual),
                                          static_cast<uint16_t*>(out), s));
}

}  // extern "C"
