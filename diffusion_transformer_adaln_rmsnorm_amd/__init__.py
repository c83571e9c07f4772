"""MI355X (gfx950) MiniMax-H3 AdaLN-modulated projection stages.

Thin Python binding over the C ABI in include/dit.h (libdit.so, built in-tree by
``_build.build()``).  The three functions take torch tensors, check the things a raw
pointer cannot carry (device, dtype, shape, unit column stride), allocate optional outputs
and workspaces with torch when they are omitted (as the FlashInfer pages do), and pass raw
device pointers and the current stream to the library.  Every step of the computation runs
in the library's HIP kernels; there is no fallback: if the library is missing or the device
is not a GPU, the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["dit_pre_attn_bf16", "dit_pre_attn_bf16_static_ws", "dit_pre_attn_e4m3", "dit_norm_adaln_bf16", "dit_qkv_rope_pack_bf16",
           "dit_qkv_rope_pack_e4m3", "dit_out_proj_gated_bf16", "dit_mlp_fp8", "dit_mlp_fp8_flags_elems",
           "dit_mx_scale_bytes", "dit_mx_quant_fp4", "dit_out_proj_gated_mxfp4", "dit_pre_attn_mxfp4",
           "DitError", "load_library", "LIB_PATH", "HIDDEN", "HEADS", "HEAD_DIM", "QKV_ROWS", "ATTN_WIDTH",
           "INTER", "FC1_ROWS", "MLP_MAX_M", "STATIC_WS_MAX_ROWS"]

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdit.so")

HIDDEN, HEADS, HEAD_DIM = 5376, 56, 128
QKV_ROWS, ATTN_WIDTH, INTER, FC1_ROWS = 21504, 7168, 14336, 28672
MLP_MAX_M = 149796
STATIC_WS_MAX_ROWS = 4096      # rows of dit_pre_attn_bf16_static_ws's static workspace

STATUS = {0: "DIT_OK", 1: "DIT_ERR_NULL", 2: "DIT_ERR_SHAPE", 3: "DIT_ERR_ALIGN", 4: "DIT_ERR_STRIDE",
          5: "DIT_ERR_UNSUPPORTED", 6: "DIT_ERR_LAUNCH", 7: "DIT_ERR_VALUE"}


class DitError(ValueError):
    """A dit_* call returned a non-OK status."""

    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, status)}")


class Table(ctypes.Structure):
    """dit_bf16_table: {ptr, rows, row_stride (elements)}."""
    _fields_ = [("ptr", ctypes.c_void_p), ("rows", ctypes.c_int64), ("row_stride", ctypes.c_int64)]


_p, _i64, _i32, _f = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
_LIB = None


def load_library(path: str = LIB_PATH):
    """Load libdit.so (after torch, so both use the one HIP runtime torch loaded)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(f"libdit.so not built at {path}; run __graft_entry__.build() "
                           "(or python -m diffusion_transformer_adaln_rmsnorm_amd._build)")
    L = ctypes.CDLL(path)
    L.dit_status_string.restype = ctypes.c_char_p
    L.dit_status_string.argtypes = [_i32]
    L.dit_abi_version.restype = _i32
    L.dit_abi_version.argtypes = []
    L.dit_mlp_fp8_flags_elems.restype = _i64
    L.dit_mlp_fp8_flags_elems.argtypes = [_i64]
    L.dit_pre_attn_bf16.restype = _i32
    L.dit_pre_attn_bf16.argtypes = [_p, _i64, _p, Table, Table, _p, _p, _p, _p, _p, _i64, _p, _i32, _f, _f, _p, _p,
                                    _p]
    L.dit_pre_attn_bf16_static_ws.restype = _i32
    L.dit_pre_attn_bf16_static_ws.argtypes = [_p, _i64, _p, Table, Table, _p, _p, _p, _p, _p, _i64, _p, _i32, _f, _f,
                                              _p, _p]
    L.dit_norm_adaln_bf16.restype = _i32
    L.dit_norm_adaln_bf16.argtypes = [_p, _i64, _p, Table, Table, _p, _f, _p, _p]
    L.dit_qkv_rope_pack_bf16.restype = _i32
    L.dit_qkv_rope_pack_bf16.argtypes = [_p, _i64, _p, _p, _p, _p, _i64, _p, _i32, _f, _p, _p]
    L.dit_pre_attn_e4m3.restype = _i32
    L.dit_pre_attn_e4m3.argtypes = [_p, _i64, _p, Table, Table, _p, _p, _p, _p, _p, _i64, _p, _i32, _f, _f, _f, _f, _f,
                                    _p, _p, _p]
    L.dit_qkv_rope_pack_e4m3.restype = _i32
    L.dit_qkv_rope_pack_e4m3.argtypes = [_p, _i64, _p, _p, _p, _p, _i64, _p, _i32, _f, _f, _f, _f, _p, _p]
    L.dit_out_proj_gated_bf16.restype = _i32
    L.dit_out_proj_gated_bf16.argtypes = [_p, _i64, _p, Table, _p, _p, _p, _p]
    L.dit_mx_scale_bytes.restype = _i64
    L.dit_mx_scale_bytes.argtypes = [_i64, _i64]
    L.dit_mx_quant_fp4.restype = _i32
    L.dit_mx_quant_fp4.argtypes = [_p, _i64, _i64, _p, _p, _p]
    L.dit_pre_attn_mxfp4.restype = _i32
    L.dit_pre_attn_mxfp4.argtypes = [_p, _i64, _p, Table, Table, _p, _p, _p, _p, _p, _p, _i64, _p, _i32, _f, _f, _p,
                                     _p, _p, _p]
    L.dit_out_proj_gated_mxfp4.restype = _i32
    L.dit_out_proj_gated_mxfp4.argtypes = [_p, _i64, _p, _p, Table, _p, _p, _p, _p, _p, _p]
    L.dit_mlp_fp8.restype = _i32
    L.dit_mlp_fp8.argtypes = [_p, _i64, _p, Table, Table, Table, _p, _p, _p, _p, _p, _p, _f, _p, _p, _p, _p, _p, _p,
                              _p, _p]
    _LIB = L
    return L


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, shape=None, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _table(t: torch.Tensor, name: str) -> Table:
    _need(t, name, torch.bfloat16, contiguous=False)
    if t.dim() != 2 or t.shape[1] != HIDDEN:
        raise ValueError(f"{name} must be [rows, {HIDDEN}] (got {tuple(t.shape)})")
    if t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    return Table(t.data_ptr(), t.shape[0], t.stride(0))


_EMPTY = {}   # device -> a small buffer whose address stands in for zero-size tensors


def _ptr(t):
    """The data pointer of t.  torch gives a zero-size tensor a null pointer, which the C ABI
    refuses even where the size makes the call a no-op (M = 0), so such a tensor passes the
    address of a small, never-touched buffer on its device instead (256-byte aligned)."""
    if t is None:
        return None
    if t.numel() == 0:
        if t.device not in _EMPTY:
            _EMPTY[t.device] = torch.empty(256, dtype=torch.uint8, device=t.device)
        return ctypes.c_void_p(_EMPTY[t.device].data_ptr())
    return ctypes.c_void_p(t.data_ptr())


def _check(fn, st):
    if st != 0:
        raise DitError(fn, st)


_E4M3_DTYPES = (torch.uint8, torch.float8_e4m3fn)


def _need_out(out, e4m3: bool, P: int, M: int):
    """out [P, M, 56 // P, 3, 128]: bf16, or one byte per element (uint8 or float8_e4m3fn codes)."""
    if P not in (1, 2, 4, 8):
        return                       # the library rejects the degree (DIT_ERR_VALUE)
    shape = (P, M, HEADS // P, 3, HEAD_DIM)
    if not e4m3:
        _need(out, "out", torch.bfloat16, shape)
    elif out.dtype not in _E4M3_DTYPES:
        raise ValueError(f"out must be uint8 or float8_e4m3fn, got {out.dtype}")
    else:
        _need(out, "out", out.dtype, shape)


def dit_pre_attn_bf16(x, x_norm_weight, adaln_scale, adaln_shift, adaln_index, qkv_weight, q_norm_weight,
                      k_norm_weight, rope_cos_sin, *, ulysses_degree: int, out, eps: float = 1e-5,
                      qk_eps: float | None = None, rope_positions=None, workspace=None):
    """BF16 pre-attention stage; writes `out` [P, M, 56 // P, 3, 128] and returns it."""
    return _pre_attn(x, x_norm_weight, adaln_scale, adaln_shift, adaln_index, qkv_weight, q_norm_weight,
                     k_norm_weight, rope_cos_sin, ulysses_degree, out, eps, qk_eps, rope_positions, workspace, None)


def dit_pre_attn_bf16_static_ws(x, x_norm_weight, adaln_scale, adaln_shift, adaln_index, qkv_weight,
                                q_norm_weight, k_norm_weight, rope_cos_sin, *, ulysses_degree: int, out,
                                eps: float = 1e-5, qk_eps: float | None = None, rope_positions=None):
    """dit_pre_attn_bf16 with the workspace in the library's static per-GPU buffer (M <=
    STATIC_WS_MAX_ROWS), for callers that cannot allocate; `out` must be given, and nothing is
    allocated.  Calls that overlap in time on one GPU race on that buffer."""
    if out is None:
        raise ValueError("dit_pre_attn_bf16_static_ws allocates nothing: pass out")
    return _pre_attn(x, x_norm_weight, adaln_scale, adaln_shift, adaln_index, qkv_weight, q_norm_weight,
                     k_norm_weight, rope_cos_sin, ulysses_degree, out, eps, qk_eps, rope_positions, _STATIC, None)


def dit_pre_attn_e4m3(x, x_norm_weight, adaln_scale, adaln_shift, adaln_index, qkv_weight, q_norm_weight,
                      k_norm_weight, rope_cos_sin, *, ulysses_degree: int, out, q_descale: float, k_descale: float,
                      v_descale: float, eps: float = 1e-5, qk_eps: float | None = None, rope_positions=None,
                      workspace=None):
    """Pre-attention stage with e4m3 output codes: out [P, M, 56 // P, 3, 128] (uint8 or
    float8_e4m3fn) = e4m3(bf16 result / descale of its kind); returns out."""
    return _pre_attn(x, x_norm_weight, adaln_scale, adaln_shift, adaln_index, qkv_weight, q_norm_weight,
                     k_norm_weight, rope_cos_sin, ulysses_degree, out, eps, qk_eps, rope_positions, workspace,
                     (q_descale, k_descale, v_descale))


_STATIC = object()     # workspace marker: the library's static buffer


def _pre_attn(x, x_norm_weight, adaln_scale, adaln_shift, adaln_index, qkv_weight, q_norm_weight, k_norm_weight,
              rope_cos_sin, ulysses_degree, out, eps, qk_eps, rope_positions, workspace, descale):
    L = load_library()
    M = x.shape[0] if x.dim() == 2 else -1
    _need(x, "x", torch.bfloat16, (M, HIDDEN))
    _need(x_norm_weight, "x_norm_weight", torch.bfloat16, (HIDDEN,))
    ts, th = _table(adaln_scale, "adaln_scale"), _table(adaln_shift, "adaln_shift")
    _need(adaln_index, "adaln_index", torch.int64, (M,))
    _need(qkv_weight, "qkv_weight", torch.bfloat16, (QKV_ROWS, HIDDEN))
    _need(q_norm_weight, "q_norm_weight", torch.bfloat16, (HEAD_DIM,))
    _need(k_norm_weight, "k_norm_weight", torch.bfloat16, (HEAD_DIM,))
    if rope_cos_sin.dim() != 2:
        raise ValueError("rope_cos_sin must be [S, 96]")
    S = rope_cos_sin.shape[0]
    _need(rope_cos_sin, "rope_cos_sin", torch.bfloat16, (S, 96))
    if rope_positions is not None:
        _need(rope_positions, "rope_positions", torch.int64, (M,))
    P = int(ulysses_degree)
    _need_out(out, descale is not None, P, M)
    qk = eps if qk_eps is None else qk_eps
    args = (_ptr(x), M, _ptr(x_norm_weight), ts, th, _ptr(adaln_index), _ptr(qkv_weight), _ptr(q_norm_weight),
            _ptr(k_norm_weight), _ptr(rope_cos_sin), S, _ptr(rope_positions), P, float(eps), float(qk))
    if workspace is _STATIC:
        _check("dit_pre_attn_bf16_static_ws", L.dit_pre_attn_bf16_static_ws(*args, _ptr(out), _stream()))
        return out
    if workspace is None:
        workspace = torch.empty((M, HIDDEN), dtype=torch.bfloat16, device=x.device)
    _need(workspace, "workspace", torch.bfloat16, (M, HIDDEN))
    if descale is None:
        st = L.dit_pre_attn_bf16(*args, _ptr(workspace), _ptr(out), _stream())
        _check("dit_pre_attn_bf16", st)
    else:
        st = L.dit_pre_attn_e4m3(*args, *(float(d) for d in descale), _ptr(workspace), _ptr(out), _stream())
        _check("dit_pre_attn_e4m3", st)
    return out


def dit_pre_attn_mxfp4(x, x_norm_weight, adaln_scale, adaln_shift, adaln_index, w_codes, w_scales, q_norm_weight,
                       k_norm_weight, rope_cos_sin, *, ulysses_degree: int, out, eps: float = 1e-5,
                       qk_eps: float | None = None, rope_positions=None, ws_codes=None, ws_scales=None):
    """MXFP4 W4A4 pre-attention; w_codes / w_scales come from dit_mx_quant_fp4 of the bf16 qkv weight
    [21504, 5376].  Writes out [P, M, 56 // P, 3, 128] bf16 and returns it; the workspace codes and
    scales (allocated when omitted) receive the quantised activation."""
    L = load_library()
    M = x.shape[0] if x.dim() == 2 else -1
    dev = x.device
    _need(x, "x", torch.bfloat16, (M, HIDDEN))
    _need(x_norm_weight, "x_norm_weight", torch.bfloat16, (HIDDEN,))
    ts, th = _table(adaln_scale, "adaln_scale"), _table(adaln_shift, "adaln_shift")
    _need(adaln_index, "adaln_index", torch.int64, (M,))
    _need(w_codes, "w_codes", torch.uint8, (QKV_ROWS, HIDDEN // 2))
    _need(w_scales, "w_scales", torch.uint8, (dit_mx_scale_bytes(QKV_ROWS, HIDDEN),))
    _need(q_norm_weight, "q_norm_weight", torch.bfloat16, (HEAD_DIM,))
    _need(k_norm_weight, "k_norm_weight", torch.bfloat16, (HEAD_DIM,))
    if rope_cos_sin.dim() != 2:
        raise ValueError("rope_cos_sin must be [S, 96]")
    S = rope_cos_sin.shape[0]
    _need(rope_cos_sin, "rope_cos_sin", torch.bfloat16, (S, 96))
    if rope_positions is not None:
        _need(rope_positions, "rope_positions", torch.int64, (M,))
    P = int(ulysses_degree)
    _need_out(out, False, P, M)
    if ws_codes is None:
        ws_codes = torch.empty((M, HIDDEN // 2), dtype=torch.uint8, device=dev)
    if ws_scales is None:
        ws_scales = torch.empty((dit_mx_scale_bytes(M, HIDDEN),), dtype=torch.uint8, device=dev)
    _need(ws_codes, "ws_codes", torch.uint8, (M, HIDDEN // 2))
    _need(ws_scales, "ws_scales", torch.uint8, (dit_mx_scale_bytes(M, HIDDEN),))
    qk = eps if qk_eps is None else qk_eps
    st = L.dit_pre_attn_mxfp4(_ptr(x), M, _ptr(x_norm_weight), ts, th, _ptr(adaln_index), _ptr(w_codes),
                              _ptr(w_scales), _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(rope_cos_sin), S,
                              _ptr(rope_positions), P, float(eps), float(qk), _ptr(ws_codes), _ptr(ws_scales),
                              _ptr(out), _stream())
    _check("dit_pre_attn_mxfp4", st)
    return out


def dit_norm_adaln_bf16(x, x_norm_weight, adaln_scale, adaln_shift, adaln_index, *, workspace, eps: float = 1e-5):
    """Launch 1 of the pre-attention stage: writes the modulated activation into workspace."""
    L = load_library()
    M = x.shape[0] if x.dim() == 2 else -1
    _need(x, "x", torch.bfloat16, (M, HIDDEN))
    _need(x_norm_weight, "x_norm_weight", torch.bfloat16, (HIDDEN,))
    ts, th = _table(adaln_scale, "adaln_scale"), _table(adaln_shift, "adaln_shift")
    _need(adaln_index, "adaln_index", torch.int64, (M,))
    _need(workspace, "workspace", torch.bfloat16, (M, HIDDEN))
    st = L.dit_norm_adaln_bf16(_ptr(x), M, _ptr(x_norm_weight), ts, th, _ptr(adaln_index), float(eps),
                               _ptr(workspace), _stream())
    _check("dit_norm_adaln_bf16", st)
    return workspace


def dit_qkv_rope_pack_bf16(workspace, qkv_weight, q_norm_weight, k_norm_weight, rope_cos_sin, *,
                           ulysses_degree: int, out, qk_eps: float = 1e-5, rope_positions=None):
    """Launch 2 of the pre-attention stage: QKV GEMM + Q/K RMSNorm + RoPE + pack into out."""
    return _qkv_rope_pack(workspace, qkv_weight, q_norm_weight, k_norm_weight, rope_cos_sin, ulysses_degree, out,
                          qk_eps, rope_positions, None)


def dit_qkv_rope_pack_e4m3(workspace, qkv_weight, q_norm_weight, k_norm_weight, rope_cos_sin, *,
                           ulysses_degree: int, out, q_descale: float, k_descale: float, v_descale: float,
                           qk_eps: float = 1e-5, rope_positions=None):
    """Launch 2 with e4m3 output codes (see dit_pre_attn_e4m3)."""
    return _qkv_rope_pack(workspace, qkv_weight, q_norm_weight, k_norm_weight, rope_cos_sin, ulysses_degree, out,
                          qk_eps, rope_positions, (q_descale, k_descale, v_descale))


def _qkv_rope_pack(workspace, qkv_weight, q_norm_weight, k_norm_weight, rope_cos_sin, ulysses_degree, out, qk_eps,
                   rope_positions, descale):
    L = load_library()
    M = workspace.shape[0] if workspace.dim() == 2 else -1
    _need(workspace, "workspace", torch.bfloat16, (M, HIDDEN))
    _need(qkv_weight, "qkv_weight", torch.bfloat16, (QKV_ROWS, HIDDEN))
    _need(q_norm_weight, "q_norm_weight", torch.bfloat16, (HEAD_DIM,))
    _need(k_norm_weight, "k_norm_weight", torch.bfloat16, (HEAD_DIM,))
    if rope_cos_sin.dim() != 2:
        raise ValueError("rope_cos_sin must be [S, 96]")
    S = rope_cos_sin.shape[0]
    _need(rope_cos_sin, "rope_cos_sin", torch.bfloat16, (S, 96))
    if rope_positions is not None:
        _need(rope_positions, "rope_positions", torch.int64, (M,))
    P = int(ulysses_degree)
    _need_out(out, descale is not None, P, M)
    args = (_ptr(workspace), M, _ptr(qkv_weight), _ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(rope_cos_sin), S,
            _ptr(rope_positions), P, float(qk_eps))
    if descale is None:
        st = L.dit_qkv_rope_pack_bf16(*args, _ptr(out), _stream())
        _check("dit_qkv_rope_pack_bf16", st)
    else:
        st = L.dit_qkv_rope_pack_e4m3(*args, *(float(d) for d in descale), _ptr(out), _stream())
        _check("dit_qkv_rope_pack_e4m3", st)
    return out


def dit_out_proj_gated_bf16(attn_out, o_weight, gate, gate_index, residual, *, out=None):
    """BF16 out-projection with the gated residual; returns out [M, 5376]."""
    L = load_library()
    M = attn_out.shape[0] if attn_out.dim() == 2 else -1
    _need(attn_out, "attn_out", torch.bfloat16, (M, ATTN_WIDTH))
    _need(o_weight, "o_weight", torch.bfloat16, (HIDDEN, ATTN_WIDTH))
    tg = _table(gate, "gate")
    _need(gate_index, "gate_index", torch.int32, (M,))
    _need(residual, "residual", torch.bfloat16, (M, HIDDEN))
    if out is None:
        out = torch.empty((M, HIDDEN), dtype=torch.bfloat16, device=attn_out.device)
    _need(out, "out", torch.bfloat16, (M, HIDDEN))
    st = L.dit_out_proj_gated_bf16(_ptr(attn_out), M, _ptr(o_weight), tg, _ptr(gate_index), _ptr(residual),
                                   _ptr(out), _stream())
    _check("dit_out_proj_gated_bf16", st)
    return out


def dit_mx_scale_bytes(rows: int, K: int) -> int:
    return int(load_library().dit_mx_scale_bytes(int(rows), int(K)))


def dit_mx_quant_fp4(x, *, codes=None, scales=None):
    """MXFP4 of bf16 rows x [R, K] (K % 256 == 0): returns (codes uint8 [R, K/2], scales uint8
    [dit_mx_scale_bytes(R, K)] in the MX scale layout)."""
    L = load_library()
    R, K = (x.shape[0], x.shape[1]) if x.dim() == 2 else (-1, -1)
    _need(x, "x", torch.bfloat16, (R, K))
    if codes is None:
        codes = torch.empty((R, K // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((dit_mx_scale_bytes(R, K),), dtype=torch.uint8, device=x.device)
    _need(codes, "codes", torch.uint8, (R, K // 2))
    _need(scales, "scales", torch.uint8, (dit_mx_scale_bytes(R, K),))
    st = L.dit_mx_quant_fp4(_ptr(x), R, K, _ptr(codes), _ptr(scales), _stream())
    _check("dit_mx_quant_fp4", st)
    return codes, scales


def dit_out_proj_gated_mxfp4(attn_out, w_codes, w_scales, gate, gate_index, residual, *, out=None, act_codes=None,
                             act_scales=None):
    """MXFP4 W4A4 out-projection with the gated residual; returns out [M, 5376].  w_codes /
    w_scales come from dit_mx_quant_fp4 of the bf16 weight [5376, 7168]."""
    L = load_library()
    M = attn_out.shape[0] if attn_out.dim() == 2 else -1
    dev = attn_out.device
    _need(attn_out, "attn_out", torch.bfloat16, (M, ATTN_WIDTH))
    _need(w_codes, "w_codes", torch.uint8, (HIDDEN, ATTN_WIDTH // 2))
    _need(w_scales, "w_scales", torch.uint8, (dit_mx_scale_bytes(HIDDEN, ATTN_WIDTH),))
    tg = _table(gate, "gate")
    _need(gate_index, "gate_index", torch.int32, (M,))
    _need(residual, "residual", torch.bfloat16, (M, HIDDEN))
    if out is None:
        out = torch.empty((M, HIDDEN), dtype=torch.bfloat16, device=dev)
    if act_codes is None:
        act_codes = torch.empty((M, ATTN_WIDTH // 2), dtype=torch.uint8, device=dev)
    if act_scales is None:
        act_scales = torch.empty((dit_mx_scale_bytes(M, ATTN_WIDTH),), dtype=torch.uint8, device=dev)
    _need(out, "out", torch.bfloat16, (M, HIDDEN))
    _need(act_codes, "act_codes", torch.uint8, (M, ATTN_WIDTH // 2))
    _need(act_scales, "act_scales", torch.uint8, (dit_mx_scale_bytes(M, ATTN_WIDTH),))
    st = L.dit_out_proj_gated_mxfp4(_ptr(attn_out), M, _ptr(w_codes), _ptr(w_scales), tg, _ptr(gate_index),
                                    _ptr(residual), _ptr(act_codes), _ptr(act_scales), _ptr(out), _stream())
    _check("dit_out_proj_gated_mxfp4", st)
    return out


def dit_mlp_fp8_flags_elems(M: int) -> int:
    return int(load_library().dit_mlp_fp8_flags_elems(int(M)))


def dit_mlp_fp8(x, x_norm_weight, adaln_scale, adaln_shift, adaln_index, gate, residual, fc1_weight_q,
                fc1_weight_scale, fc2_weight_q, fc2_weight_scale, *, out=None, workspace_a_q=None,
                workspace_a_scale=None, workspace_y=None, workspace_y_q=None, workspace_y_scale=None,
                workspace_flags=None, eps: float = 1e-5):
    """FP8 W8A8 MLP block; returns out [M, 5376] (workspaces are filled as a side effect)."""
    L = load_library()
    M = x.shape[0] if x.dim() == 2 else -1
    dev = x.device
    _need(x, "x", torch.bfloat16, (M, HIDDEN))
    _need(x_norm_weight, "x_norm_weight", torch.bfloat16, (HIDDEN,))
    ts, th, tg = _table(adaln_scale, "adaln_scale"), _table(adaln_shift, "adaln_shift"), _table(gate, "gate")
    _need(adaln_index, "adaln_index", torch.int64, (M,))
    _need(residual, "residual", torch.bfloat16, (M, HIDDEN))
    _need(fc1_weight_q, "fc1_weight_q", torch.float8_e4m3fn, (FC1_ROWS, HIDDEN))
    _need(fc1_weight_scale, "fc1_weight_scale", torch.float32, (FC1_ROWS,))
    _need(fc2_weight_q, "fc2_weight_q", torch.float8_e4m3fn, (HIDDEN, INTER))
    _need(fc2_weight_scale, "fc2_weight_scale", torch.float32, (HIDDEN,))
    e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)  # noqa: E731
    out = e((M, HIDDEN), torch.bfloat16) if out is None else out
    a_q = e((M, HIDDEN), torch.float8_e4m3fn) if workspace_a_q is None else workspace_a_q
    a_s = e((M,), torch.float32) if workspace_a_scale is None else workspace_a_scale
    y = e((M, INTER), torch.bfloat16) if workspace_y is None else workspace_y
    y_q = e((M, INTER), torch.float8_e4m3fn) if workspace_y_q is None else workspace_y_q
    y_s = e((M,), torch.float32) if workspace_y_scale is None else workspace_y_scale
    _need(out, "out", torch.bfloat16, (M, HIDDEN))
    _need(a_q, "workspace_a_q", torch.float8_e4m3fn, (M, HIDDEN))
    _need(a_s, "workspace_a_scale", torch.float32, (M,))
    _need(y, "workspace_y", torch.bfloat16, (M, INTER))
    _need(y_q, "workspace_y_q", torch.float8_e4m3fn, (M, INTER))
    _need(y_s, "workspace_y_scale", torch.float32, (M,))
    if workspace_flags is not None:
        _need(workspace_flags, "workspace_flags", torch.int32, contiguous=True)
    st = L.dit_mlp_fp8(_ptr(x), M, _ptr(x_norm_weight), ts, th, tg, _ptr(adaln_index), _ptr(residual),
                       _ptr(fc1_weight_q), _ptr(fc1_weight_scale), _ptr(fc2_weight_q), _ptr(fc2_weight_scale),
                       float(eps), _ptr(a_q), _ptr(a_s), _ptr(y), _ptr(y_q), _ptr(y_s), _ptr(workspace_flags),
                       _ptr(out), _stream())
    _check("dit_mlp_fp8", st)
    return out
