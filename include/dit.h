/*
 * dit.h - C ABI of the MI355X (gfx950) MiniMax-H3 AdaLN-modulated projection stages.
 *
 * Three operations, each following the tensor contract of one FlashInfer diffusion_ops page:
 *   dit_pre_attn_bf16       "minimax_h3_bf16_pre_attention" (description, Parameters, Notes),
 *                           and its e4m3 output mode dit_pre_attn_e4m3 ("minimax_h3_nvfp4_pre_attention",
 *                           Parameters: out_mode, q/k/v_descale); its W4A4 form dit_pre_attn_mxfp4
 *                           (that page's description, OCP MXFP4 in place of NVFP4)
 *   dit_out_proj_gated_bf16 "minimax_h3_nvfp4_out_proj" gated-residual epilogue, bf16 operands,
 *                           and its W4A4 form dit_out_proj_gated_mxfp4 (same page's description,
 *                           with OCP MXFP4 in place of NVFP4; quantiser dit_mx_quant_fp4)
 *   dit_mlp_fp8             "minimax_h3_mlp_fp8_sm120" (per-row formula block, Parameters)
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is caller-owned DEVICE memory on the current HIP device.  The
 *    library never allocates, frees, copies to or from the host, or synchronises.
 *  - bf16 tensors are passed as raw 16-bit patterns (void*); e4m3 tensors as uint8 codes of
 *    OCP float8_e4m3fn; indices as int64 or int32 as stated.  All matrices are row-major and
 *    contiguous except the AdaLN/gate tables, which are dit_bf16_table views.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the call
 *    returns immediately.  Results are ready when the stream reaches them.
 *  - Host-side contract checks run before anything is launched; a failed check returns its
 *    status and launches nothing.  Malformed index or position VALUES are not errors: they
 *    are guarded on the device (zero rows, zero gates, clamped positions) as the pages state.
 *  - Calls that share output or workspace buffers must not overlap in time.
 *  - Every GEMM launch is persistent: one workgroup per CU claims tiles from per-XCD
 *    counters.  The counters come from a static per-GPU pool of 4096 sets, taken in rotation,
 *    and the launch's last workgroup leaves its set at zero for the set's next use.  Calls in
 *    flight at the same time get distinct sets while fewer than 4096 are in flight.  The one
 *    exception is two replays of a single captured HIP graph: they reuse the set fixed at
 *    capture and must not overlap.
 *  - Launch failures reported by the HIP runtime return DIT_ERR_LAUNCH.
 */
#ifndef DIT_H
#define DIT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DIT_HIDDEN 5376       /* model width */
#define DIT_HEADS 56          /* attention heads */
#define DIT_HEAD_DIM 128      /* per-head dimension */
#define DIT_QKV_ROWS 21504    /* 3 * 56 * 128 */
#define DIT_ATTN_WIDTH 7168   /* 56 * 128 */
#define DIT_ROPE_COLS 96      /* 48 cos + 48 sin per cache row */
#define DIT_INTER 14336       /* MLP intermediate width */
#define DIT_FC1_ROWS 28672    /* gate | up */
#define DIT_MLP_MAX_M 149796  /* row limit of the fp8 MLP page */
#define DIT_MAX_ROWS 16777216 /* 2^24: row limit of the pre-attention and out-projection calls
                                 (keeps every launch grid below 2^32 work-items) */
#define DIT_MAX_ROPE_ROWS 22369621 /* floor((2^32 - 1) / 192): rows of the [S, 96] bf16 cos/sin
                                      cache, whose byte offsets are 32-bit on the device */

typedef enum {
    DIT_OK = 0,
    DIT_ERR_NULL = 1,        /* a required pointer is NULL */
    DIT_ERR_SHAPE = 2,       /* a size is out of range (M, rows, S, S < M with identity positions);
                                M <= DIT_MAX_ROWS and S <= DIT_MAX_ROPE_ROWS wherever they apply */
    DIT_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned (8 for int64 vectors, 4 for int32/f32) */
    DIT_ERR_STRIDE = 4,      /* table row stride < 5376 or not a multiple of 8 elements, or mismatched */
    DIT_ERR_UNSUPPORTED = 5, /* a valid argument this build does not implement (none at present) */
    DIT_ERR_LAUNCH = 6,      /* the HIP runtime rejected a kernel launch */
    DIT_ERR_VALUE = 7        /* a scalar is invalid (eps <= 0 or not finite, ulysses_degree not 1/2/4/8,
                                an e4m3 descale below FLT_MIN or not finite) */
} dit_status;

/*
 * A bf16 [rows, 5376] table view with unit column stride, as the pre-attention page's
 * adaln_scale/adaln_shift entries allow: row r starts at ptr + r * row_stride ELEMENTS.
 * row_stride >= 5376 and a multiple of 8; 1 <= rows <= 2^31 - 1; ptr 16-byte aligned.  A column chunk of a wider
 * [rows, 6 * 5376] modulation matrix is passed as-is (ptr = chunk start, row_stride = 32256).
 */
typedef struct {
    const void* ptr;
    int64_t rows;
    int64_t row_stride;
} dit_bf16_table;

/* Human-readable name of a status code (static string). */
const char* dit_status_string(int status);

/* ABI version of this library (major * 100 + minor). */
int dit_abi_version(void);

/*
 * BF16 pre-attention stage ("minimax_h3_bf16_pre_attention": description and Parameters).
 *
 * For each row m of x [M, 5376]:
 *   i = adaln_index[m]; if i is outside [0, rows) the workspace row is all +0 (and so is the
 *   output row), without reading the tables;
 *   n = bf16(x[m] * rsqrt(mean(x[m]^2) + eps) * x_norm_weight)       (FP32 sum of squares)
 *   a = bf16(adaln_shift[i] + n * bf16(1 + adaln_scale[i]))  -> workspace[m, :]
 *   qkv = bf16(a @ qkv_weight^T)                       (qkv_weight [21504, 5376], rows in
 *                                                       [q_all | k_all | v_all] x 56 x 128)
 *   per q and k head: u = bf16(v * rsqrt(mean(v^2) + qk_eps) * {q,k}_norm_weight)
 *   p = rope_positions ? clamp(rope_positions[m], 0, S-1) : m
 *   dims j < 48: o_j = bf16(u_j c_j - u_{j+48} s_j), o_{j+48} = bf16(u_{j+48} c_j + u_j s_j)
 *   with c_j = rope_cos_sin[p, j], s_j = rope_cos_sin[p, 48 + j]; dims [96, 128) pass through
 *   v heads: bf16(acc) only
 *   out[h / (56/P), m, h % (56/P), kind, :] = o   (kind 0 = q, 1 = k, 2 = v): the
 *   destination-major pack, destination p taking the contiguous heads [p 56/P, (p+1) 56/P)
 *
 * Arguments:
 *   x              bf16 [M, 5376], contiguous, 16-B aligned
 *   M              rows, 0 <= M <= DIT_MAX_ROWS; 0 is a no-op returning DIT_OK
 *   x_norm_weight  bf16 [5376]
 *   adaln_scale, adaln_shift  tables with equal rows (>= 1)
 *   adaln_index    int64 [M]; any value is allowed (see the guard above)
 *   qkv_weight     bf16 [21504, 5376]
 *   q_norm_weight, k_norm_weight  bf16 [128]
 *   rope_cos_sin   bf16 [S, 96], 1 <= S <= DIT_MAX_ROPE_ROWS
 *   rope_positions int64 [M] or NULL for the identity (then S >= M is required)
 *   ulysses_degree destination count P: 1, 2, 4 or 8 (else DIT_ERR_VALUE)
 *   eps, qk_eps    positive finite RMSNorm epsilons (the Python binding maps qk_eps=None to eps)
 *   workspace      bf16 [M, 5376] scratch, overwritten with a
 *   out            bf16 [P, M, 56/P, 3, 128]; must not overlap any input
 *   stream         hipStream_t
 * Two kernels are enqueued: the row norm/AdaLN kernel and the QKV GEMM with the fused
 * Q/K-norm, RoPE and pack epilogue.
 */
dit_status dit_pre_attn_bf16(const void* x, int64_t M, const void* x_norm_weight,
                             dit_bf16_table adaln_scale, dit_bf16_table adaln_shift,
                             const int64_t* adaln_index, const void* qkv_weight,
                             const void* q_norm_weight, const void* k_norm_weight,
                             const void* rope_cos_sin, int64_t S, const int64_t* rope_positions,
                             int ulysses_degree, float eps, float qk_eps, void* workspace, void* out,
                             void* stream);

/*
 * For callers that cannot allocate: code under HIP graph capture, serving loops and harnesses
 * that forbid hipMalloc.  dit_pre_attn_bf16 without the workspace argument: the workspace
 * [M, 5376] bf16 lives in the library's own static device buffer of DIT_STATIC_WS_MAX_ROWS
 * rows (42 MiB), one per GPU, held from the library's load on that GPU until the process
 * ends.  Same kernels, arguments, checks and results as dit_pre_attn_bf16; the call allocates
 * and frees nothing (the first call on a device looks up the buffer's device address with
 * hipGetSymbolAddress, which allocates nothing either).
 *   M      0 <= M <= DIT_STATIC_WS_MAX_ROWS, else DIT_ERR_SHAPE; 0 is a no-op
 *   out    as in dit_pre_attn_bf16; the caller passes it (it is never allocated here)
 * Every call on one GPU uses that GPU's one buffer, which keeps the last call's contents:
 * calls that overlap in time on one GPU (on different streams, or from several threads) race
 * and must be serialised, for example by issuing them on one stream.  Nothing in the buffer
 * needs to start at zero.
 */
#define DIT_STATIC_WS_MAX_ROWS 4096
dit_status dit_pre_attn_bf16_static_ws(const void* x, int64_t M, const void* x_norm_weight,
                                       dit_bf16_table adaln_scale, dit_bf16_table adaln_shift,
                                       const int64_t* adaln_index, const void* qkv_weight,
                                       const void* q_norm_weight, const void* k_norm_weight,
                                       const void* rope_cos_sin, int64_t S,
                                       const int64_t* rope_positions, int ulysses_degree, float eps,
                                       float qk_eps, void* out, void* stream);

/*
 * The two launches of dit_pre_attn_bf16, callable one at a time (same kernels, same
 * arguments and checks).  dit_norm_adaln_bf16 writes the modulated activation a into
 * workspace [M, 5376] (launch 1: input RMSNorm + indexed AdaLN + guard);
 * dit_qkv_rope_pack_bf16 reads such a workspace and writes out (launch 2: QKV GEMM with the
 * Q/K RMSNorm, RoPE and pack epilogue).  dit_pre_attn_bf16 is exactly the first followed by
 * the second on one stream.  For engines that keep the modulated activation, and for timing
 * each launch.
 */
dit_status dit_norm_adaln_bf16(const void* x, int64_t M, const void* x_norm_weight,
                               dit_bf16_table adaln_scale, dit_bf16_table adaln_shift,
                               const int64_t* adaln_index, float eps, void* workspace, void* stream);

dit_status dit_qkv_rope_pack_bf16(const void* workspace, int64_t M, const void* qkv_weight,
                                  const void* q_norm_weight, const void* k_norm_weight,
                                  const void* rope_cos_sin, int64_t S, const int64_t* rope_positions,
                                  int ulysses_degree, float qk_eps, void* out, void* stream);

/*
 * E4M3 output mode of the pre-attention ("minimax_h3_nvfp4_pre_attention", Parameters:
 * out_mode "e4m3" with per-tensor q_descale / k_descale / v_descale dequantization scales;
 * the page defers their conventions to a page that is missing, and this is the plainest
 * reading).  The same computation as dit_pre_attn_bf16 / dit_qkv_rope_pack_bf16; each bf16
 * result o of the pack is then stored as one byte
 *   out[h / (56/P), m, h % (56/P), kind, d] = e4m3(fl32(o / descale_kind))
 * (float8_e4m3fn, round to nearest even, saturating at +-448; descale_kind = q_descale,
 * k_descale or v_descale), so that code * descale approximates o.
 * Arguments as the bf16 calls, plus:
 *   q_descale, k_descale, v_descale  finite fp32 scales >= FLT_MIN (2^-126), so that each
 *                  reciprocal is finite (else DIT_ERR_VALUE)
 *   out            uint8 e4m3 codes [P, M, 56/P, 3, 128], 16-B aligned; must not overlap any input
 */
dit_status dit_pre_attn_e4m3(const void* x, int64_t M, const void* x_norm_weight,
                             dit_bf16_table adaln_scale, dit_bf16_table adaln_shift,
                             const int64_t* adaln_index, const void* qkv_weight,
                             const void* q_norm_weight, const void* k_norm_weight,
                             const void* rope_cos_sin, int64_t S, const int64_t* rope_positions,
                             int ulysses_degree, float eps, float qk_eps, float q_descale,
                             float k_descale, float v_descale, void* workspace, void* out, void* stream);

dit_status dit_qkv_rope_pack_e4m3(const void* workspace, int64_t M, const void* qkv_weight,
                                  const void* q_norm_weight, const void* k_norm_weight,
                                  const void* rope_cos_sin, int64_t S, const int64_t* rope_positions,
                                  int ulysses_degree, float qk_eps, float q_descale, float k_descale,
                                  float v_descale, void* out, void* stream);

/*
 * BF16 attention output projection with the fused gated residual (the epilogue of
 * "minimax_h3_nvfp4_out_proj", with bf16 operands instead of NVFP4 ones):
 *   o = bf16(attn_out[m] @ o_weight^T)
 *   g = gate[gate_index[m]] if 0 <= gate_index[m] < gate.rows else 0
 *   out[m] = bf16(residual[m] + bf16(g * o))
 * Arguments:
 *   attn_out   bf16 [M, 7168];  0 <= M <= DIT_MAX_ROWS, M = 0 is a no-op
 *   o_weight   bf16 [5376, 7168]
 *   gate       table view [rows, 5376] (the page's gate_msa rows, rows = 9 there)
 *   gate_index int32 [M], any value
 *   residual   bf16 [M, 5376]
 *   out        bf16 [M, 5376]; may be the same pointer as residual (each element is read
 *              before it is written); must not overlap attn_out
 * One kernel is enqueued.
 */
dit_status dit_out_proj_gated_bf16(const void* attn_out, int64_t M, const void* o_weight,
                                   dit_bf16_table gate, const int32_t* gate_index,
                                   const void* residual, void* out, void* stream);

/*
 * FP8 (W8A8) MLP block ("minimax_h3_mlp_fp8_sm120", per-row formula block):
 *   n, a  as in dit_pre_attn_bf16 (a = 0 for rows whose index is outside [0, rows))
 *   s_a = RN(amax|a| / 448)  (fp32),  a_q = e4m3(a / s_a)  (RNE, saturating; amax 0 -> 0)
 *   h = bf16((a_q @ fc1^T) * s_a * fc1_scale)       FP32 accumulation, [M, 28672]
 *   y = bf16(bf16(silu(h[:, :14336])) * h[:, 14336:])
 *   s_y = RN(amax|y| / 448),  y_q = e4m3(y / s_y)
 *   o = bf16((y_q @ fc2^T) * s_y * fc2_scale)
 *   out = bf16(residual + bf16(gate[i] * o)),  gate 0 for guarded rows
 * Arguments:
 *   x            bf16 [M, 5376], 1 <= M <= 149796
 *   x_norm_weight bf16 [5376]
 *   adaln_scale, adaln_shift, gate  tables with equal rows; scale and shift share row_stride
 *   adaln_index  int64 [M]
 *   residual     bf16 [M, 5376]
 *   fc1_q        e4m3 [28672, 5376], rows [0,14336) gate and [14336,28672) up; fc1_scale f32 [28672]
 *   fc2_q        e4m3 [5376, 14336];  fc2_scale f32 [5376]
 *   eps          positive finite
 *   ws_a_q e4m3 [M,5376], ws_a_scale f32 [M], ws_y bf16 [M,14336], ws_y_q e4m3 [M,14336],
 *   ws_y_scale f32 [M]: caller-owned workspaces, all overwritten with the values above
 *   ws_flags     may be NULL; see dit_mlp_fp8_flags_elems
 *   out          bf16 [M, 5376]; may be residual or x, must not overlap any workspace
 * Four kernels are enqueued (norm/AdaLN/quant, FC1+SwiGLU, y quant, FC2+gated residual).
 */
dit_status dit_mlp_fp8(const void* x, int64_t M, const void* x_norm_weight,
                       dit_bf16_table adaln_scale, dit_bf16_table adaln_shift, dit_bf16_table gate,
                       const int64_t* adaln_index, const void* residual, const uint8_t* fc1_q,
                       const float* fc1_scale, const uint8_t* fc2_q, const float* fc2_scale,
                       float eps, uint8_t* ws_a_q, float* ws_a_scale, void* ws_y, uint8_t* ws_y_q,
                       float* ws_y_scale, int32_t* ws_flags, void* out, void* stream);

/*
 * Number of int32 tile-ready flags dit_mlp_fp8 needs for M rows (the counterpart of the
 * page's minimax_h3_mlp_fc2_flags_sm120).  This implementation needs none from the caller: it
 * returns 0 for every M, and ws_flags is ignored.  (Where FC2 quantises y in its own launch, its
 * ready counters live in the library's per-GPU tile-queue pool, zeroed by each launch that uses
 * them.)
 */
int64_t dit_mlp_fp8_flags_elems(int64_t M);

/*
 * MXFP4 (OCP Microscaling Formats v1.0) quantisation, the W4A4 format gfx950's block-scaled
 * MFMA takes natively; it stands where "minimax_h3_nvfp4_out_proj" (description) quantises to
 * NVFP4 (block 16, UE4M3 scales, a global scale):
 *   per block of 32 consecutive values of a row:  E = floor(log2(amax)) - 2 + 127, clamped to
 *   [0, 254] (E = 0 for an all-zero block); scale 2^(E - 127) stored as the E8M0 byte E;
 *   code = E2M1 value nearest v / 2^(E - 127), ties to the even significand, saturating at 6,
 *   sign kept (-0 is code 8).
 * Arguments:
 *   x       bf16 [rows, K], K a positive multiple of 256
 *   codes   uint8 [rows, K / 2]: element 2j of a row in the low nibble of byte j
 *   scales  uint8, dit_mx_scale_bytes(rows, K) bytes, in the MX scale layout: with rows padded
 *           to a multiple of 128, the scale of row r, block b (values 32 b .. 32 b + 31) is the
 *           byte ((r / 128) (K / 256) + b / 8) 1024 + 16 l + 4 ((r % 128) / 32) + (b % 8) / 2,
 *           l = r % 32 + 32 (b % 2) (the order in which the lanes of the 32 x 32 x 64 MFMA take
 *           them).  Padding rows get scale byte 0.
 * rows = 0 is a no-op.  One kernel is enqueued.  Used for the weight once and by
 * dit_out_proj_gated_mxfp4 for the activation on every call.
 */
int64_t dit_mx_scale_bytes(int64_t rows, int64_t K);
dit_status dit_mx_quant_fp4(const void* x, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales,
                            void* stream);

/*
 * MXFP4 W4A4 attention output projection with the fused gated residual ("minimax_h3_nvfp4_out_proj",
 * description, with MXFP4 operands):
 *   (act_codes, act_scales) = dit_mx_quant_fp4(attn_out)
 *   o = bf16(A[m] . W[n]), A and W the values of the activation's and the weight's MXFP4
 *       codes and scales (FP32 accumulation)
 *   out[m] = bf16(residual[m] + bf16(g * o)),  g as in dit_out_proj_gated_bf16
 * Arguments:
 *   attn_out    bf16 [M, 7168]; 0 <= M <= DIT_MAX_ROWS, M = 0 is a no-op
 *   w_codes     uint8 [5376, 3584] and w_scales (dit_mx_scale_bytes(5376, 7168) bytes): the
 *               weight quantised by dit_mx_quant_fp4
 *   gate, gate_index, residual, out   as in dit_out_proj_gated_bf16
 *   act_codes   uint8 [M, 3584] workspace; act_scales dit_mx_scale_bytes(M, 7168) bytes of
 *               workspace (both written, then read by the GEMM)
 *   16-byte alignment for every pointer except gate_index (4)
 * Two kernels are enqueued (quantisation, then the block-scaled GEMM with its epilogue).
 */
/*
 * MXFP4 W4A4 pre-attention ("minimax_h3_nvfp4_pre_attention", description: the normalised and
 * modulated activation is quantised to 4 bits with block scales and the QKV GEMM runs on it and
 * the pre-quantised weight; here in MXFP4, as for dit_out_proj_gated_mxfp4):
 *   a as in dit_pre_attn_bf16 (the bf16 workspace value; a = 0 for guarded rows), written only
 *       as its MXFP4 codes and scales (dit_mx_quant_fp4 of a)
 *   qkv = bf16(A[m] . W[n]) over the MXFP4 values (FP32 accumulation), then the Q/K RMSNorm,
 *       RoPE and pack of dit_pre_attn_bf16
 * Arguments:
 *   x, x_norm_weight, adaln_*, q/k_norm_weight, rope_cos_sin, S, rope_positions,
 *   ulysses_degree, eps, qk_eps, out   as in dit_pre_attn_bf16 (out bf16 [P, M, 56/P, 3, 128])
 *   w_codes    uint8 [21504, 2688] and w_scales (dit_mx_scale_bytes(21504, 5376) bytes): the
 *              qkv weight quantised by dit_mx_quant_fp4
 *   ws_codes   uint8 [M, 2688] workspace; ws_scales dit_mx_scale_bytes(M, 5376) bytes of workspace
 *   16-byte alignment for every pointer except adaln_index and rope_positions (8)
 * Two kernels are enqueued (norm + AdaLN + quantisation, then the block-scaled QKV GEMM).
 */
dit_status dit_pre_attn_mxfp4(const void* x, int64_t M, const void* x_norm_weight,
                              dit_bf16_table adaln_scale, dit_bf16_table adaln_shift,
                              const int64_t* adaln_index, const uint8_t* w_codes,
                              const uint8_t* w_scales, const void* q_norm_weight,
                              const void* k_norm_weight, const void* rope_cos_sin, int64_t S,
                              const int64_t* rope_positions, int ulysses_degree, float eps,
                              float qk_eps, uint8_t* ws_codes, uint8_t* ws_scales, void* out,
                              void* stream);

dit_status dit_out_proj_gated_mxfp4(const void* attn_out, int64_t M, const uint8_t* w_codes,
                                    const uint8_t* w_scales, dit_bf16_table gate,
                                    const int32_t* gate_index, const void* residual,
                                    uint8_t* act_codes, uint8_t* act_scales, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DIT_H */
