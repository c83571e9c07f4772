// The bf16 pre-attention with its workspace in a static device buffer, for callers that cannot
// allocate (code under HIP graph capture, serving loops, harnesses that forbid hipMalloc).
//
// The buffer is a file-scope __device__ array: every GPU the library runs on holds its own copy
// from the module's load until the process ends.  Host code never names the array in a kernel
// argument or a copy (in host code that name is a host-side stand-in, not a device address):
// on the first call on a device, with that device current, hipGetSymbolAddress gives the
// device address of that device's copy, which is kept per device and used from then on.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/dit.h"

namespace {

constexpr int kMaxDevices = 64;

// The workspace [DIT_STATIC_WS_MAX_ROWS, 5376] bf16 (42 MiB).  Nothing in it has to start at
// zero: the first launch writes every row the second one reads.
__device__ __align__(256) uint8_t scratch[(size_t)DIT_STATIC_WS_MAX_ROWS * DIT_HIDDEN * 2];

std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` on each device, once looked up

// The current device's copy of `scratch`, looked up on the first call on that device.
hipError_t scratch_on_current_device(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" dit_status dit_pre_attn_bf16_static_ws(const void* x, int64_t M, const void* x_norm_weight,
                                                   dit_bf16_table adaln_scale, dit_bf16_table adaln_shift,
                                                   const int64_t* adaln_index, const void* qkv_weight,
                                                   const void* q_norm_weight, const void* k_norm_weight,
                                                   const void* rope_cos_sin, int64_t S,
                                                   const int64_t* rope_positions, int ulysses_degree, float eps,
                                                   float qk_eps, void* out, void* stream) {
    if (M < 0 || M > DIT_STATIC_WS_MAX_ROWS) return DIT_ERR_SHAPE;
    // Every other check first, before the device is touched: the M = 0 form of the call checks
    // all arguments and launches nothing (`out` stands in for the workspace, which it never
    // reads); only the identity-position rule S >= M depends on M.
    dit_status st = dit_pre_attn_bf16(x, 0, x_norm_weight, adaln_scale, adaln_shift, adaln_index, qkv_weight,
                                      q_norm_weight, k_norm_weight, rope_cos_sin, S, rope_positions, ulysses_degree,
                                      eps, qk_eps, out, out, stream);
    if (st != DIT_OK) return st;
    if (!rope_positions && S < M) return DIT_ERR_SHAPE;
    if (M == 0) return DIT_OK;
    void* ws = nullptr;
    if (scratch_on_current_device(&ws) != hipSuccess) return DIT_ERR_LAUNCH;
    return dit_pre_attn_bf16(x, M, x_norm_weight, adaln_scale, adaln_shift, adaln_index, qkv_weight, q_norm_weight,
                             k_norm_weight, rope_cos_sin, S, rope_positions, ulysses_degree, eps, qk_eps, ws, out,
                             stream);
}
