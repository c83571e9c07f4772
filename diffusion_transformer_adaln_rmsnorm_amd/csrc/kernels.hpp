// Internal launchers (host side).  Each enqueues its kernel(s) on `stream` and returns the
// launch status; argument validation happens in api.cpp before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

// A zero set of per-XCD tile counters for one persistent GEMM launch on `stream` (the launch's
// last workgroup leaves it zero again), and the persistent grid of the current device.
hipError_t tile_queue(hipStream_t stream, uint32_t** counters, int* grid);

hipError_t launch_norm_adaln_bf16(const uint16_t* x, int64_t M, const uint16_t* xw, const uint16_t* scale,
                                  int64_t ld_scale, const uint16_t* shift, int64_t ld_shift, int64_t rows,
                                  const int64_t* idx, float eps, uint16_t* ws, hipStream_t stream);

hipError_t launch_norm_adaln_fp8q(const uint16_t* x, int64_t M, const uint16_t* xw, const uint16_t* scale,
                                  int64_t ld_scale, const uint16_t* shift, int64_t ld_shift, int64_t rows,
                                  const int64_t* idx, float eps, uint8_t* a_q, float* a_scale,
                                  hipStream_t stream);

// P: Ulysses destination count (1, 2, 4 or 8); out is [P, M, 56 / P, 3, 128]
hipError_t launch_qkv_gemm(const uint16_t* ws, int64_t M, const uint16_t* W, const uint16_t* qw,
                           const uint16_t* kw, const uint16_t* cs, int64_t S, const int64_t* pos, float qk_eps,
                           int P, uint16_t* out, hipStream_t stream);
// M <= 16: one workgroup per head of each kind, K split over its waves (weight streaming)
hipError_t launch_qkv_small(const uint16_t* ws, int64_t M, const uint16_t* W, const uint16_t* qw, const uint16_t* kw,
                            const uint16_t* cs, int64_t S, const int64_t* pos, float qk_eps, int P, uint16_t* out,
                            hipStream_t stream);
// the same with e4m3 output codes: out[...] = e4m3(bf16 result / descale of its kind)
hipError_t launch_qkv_gemm_e4m3(const uint16_t* ws, int64_t M, const uint16_t* W, const uint16_t* qw,
                                const uint16_t* kw, const uint16_t* cs, int64_t S, const int64_t* pos,
                                float qk_eps, int P, float dq, float dk, float dv, uint8_t* out, hipStream_t stream);

hipError_t launch_out_proj_gemm(const uint16_t* attn, int64_t M, const uint16_t* Wo, const uint16_t* gate,
                                int64_t gate_rows, int64_t gate_ld, const int32_t* gate_index,
                                const uint16_t* residual, uint16_t* out, hipStream_t stream);

// MXFP4 pre-attention: the norm/AdaLN rows quantised to MXFP4 codes and scales (M rows, scales
// for M rounded up to 128), then the QKV GEMM on MXFP4 operands with the bf16 epilogue
hipError_t launch_norm_adaln_mxfp4(const uint16_t* x, int64_t M, const uint16_t* xw, const uint16_t* scale,
                                   int64_t ld_scale, const uint16_t* shift, int64_t ld_shift, int64_t rows,
                                   const int64_t* idx, float eps, uint8_t* codes, uint8_t* scales, hipStream_t stream);
hipError_t launch_qkv_gemm_mxfp4(const uint8_t* ws_codes, const uint8_t* ws_scales, int64_t M, const uint8_t* w_codes,
                                 const uint8_t* w_scales, const uint16_t* qw, const uint16_t* kw, const uint16_t* cs,
                                 int64_t S, const int64_t* pos, float qk_eps, int P, uint16_t* out,
                                 hipStream_t stream);

// MXFP4: scale bytes of a [rows, K] matrix in the MX scale layout; quantisation; W4A4 out-proj
int64_t mx_scale_bytes(int64_t rows, int64_t K);
hipError_t launch_mx_quant_fp4(const uint16_t* x, int64_t R, int64_t K, uint8_t* codes, uint8_t* scales,
                               hipStream_t stream);
hipError_t launch_out_proj_mxfp4(const uint8_t* a_codes, const uint8_t* a_scales, int64_t M, const uint8_t* w_codes,
                                 const uint8_t* w_scales, const uint16_t* gate, int64_t gate_rows, int64_t gate_ld,
                                 const int32_t* gate_index, const uint16_t* residual, uint16_t* out,
                                 hipStream_t stream);

hipError_t launch_fc1_swiglu(const uint8_t* a_q, const float* a_scale, int64_t M, const uint8_t* W1,
                             const float* w1s, uint16_t* y, hipStream_t stream);

hipError_t launch_quant_rows(const uint16_t* y, int64_t M, float* y_scale, uint8_t* y_q, hipStream_t stream);

// FC2 with the y quantisation in the same launch (y -> y_q, y_scale, then the gated FC2), for the
// M that fc2_fused_fits accepts (the m tiles split into whole groups per XCD).
bool fc2_fused_fits(int64_t M);
hipError_t launch_fc2_fused(const uint16_t* y, float* y_scale, uint8_t* y_q, int64_t M, const uint8_t* W2,
                            const float* w2s, const uint16_t* gate, int64_t gate_rows, int64_t gate_ld,
                            const int64_t* idx, const uint16_t* residual, uint16_t* out, hipStream_t stream);

hipError_t launch_fc2_gated(const uint8_t* y_q, const float* y_scale, int64_t M, const uint8_t* W2,
                            const float* w2s, const uint16_t* gate, int64_t gate_rows, int64_t gate_ld,
                            const int64_t* idx, const uint16_t* residual, uint16_t* out, hipStream_t stream);

}  // namespace dit
