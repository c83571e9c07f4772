"""CPU oracle for the MiniMax-H3 AdaLN-modulated projection stages.

TEST INFRASTRUCTURE ONLY: tests, the package smoke check and the benchmark's CPU baseline
are the only callers.  The HIP path never imports this package and this package never
imports the HIP path.

The arithmetic lives in dit_oracle.c (plain loops, fp64 between the rounding points that
the FlashInfer MiniMax-H3 pages print).  This wrapper only marshals numpy arrays, resolves
identity RoPE positions (None -> the row's own number, as the bf16 pre-attention page's
rope_positions entry states) and fans rows out over threads (rows are independent and
ctypes releases the GIL during each call).

brute.py is a second, independent NumPy transcription used to cross-check this one on
one- and two-row inputs.
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

HIDDEN, HEADS, HEAD_DIM = 5376, 56, 128
QKV_ROWS, ATTN_WIDTH, INTER = 21504, 7168, 14336

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_d = ctypes.c_double


def lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(HERE, "liboracle.so")
        if not os.path.exists(path):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(path)
        L.oracle_round_bf16.restype = ctypes.c_uint16
        L.oracle_round_bf16.argtypes = [_d]
        L.oracle_bf16_value.restype = _d
        L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.oracle_round_e4m3.restype = ctypes.c_uint8
        L.oracle_round_e4m3.argtypes = [_d]
        L.oracle_e4m3_value.restype = _d
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_quant_out_e4m3.restype = None
        L.oracle_quant_out_e4m3.argtypes = [_p, _i64, _d, _d, _d, _p]
        L.oracle_pre_attn.restype = None
        L.oracle_pre_attn.argtypes = [_i64, _i64, _p, _p, _p, _p, _i64, _i64, _p, _p, _p, _p, _p, _i64, _p,
                                      _d, _d, _p, _p]
        L.oracle_out_proj.restype = None
        L.oracle_out_proj.argtypes = [_i64, _i64, _p, _p, _p, _i64, _i64, _p, _p, _p]
        L.oracle_e2m1_value.restype = _d
        L.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
        L.oracle_round_e2m1.restype = ctypes.c_uint8
        L.oracle_round_e2m1.argtypes = [_d]
        L.oracle_mx_scale_exp.restype = ctypes.c_int
        L.oracle_mx_scale_exp.argtypes = [_d]
        L.oracle_mx_quant_fp4.restype = None
        L.oracle_mx_quant_fp4.argtypes = [_p, _i64, _i64, _p, _p]
        L.oracle_out_proj_mxfp4.restype = None
        L.oracle_out_proj_mxfp4.argtypes = [_i64, _i64, _p, _p, _p, _p, _p, _i64, _i64, _p, _p, _p]
        L.oracle_norm_adaln.restype = None
        L.oracle_norm_adaln.argtypes = [_i64, _i64, _p, _p, _p, _p, _i64, _i64, _p, _d, _p]
        L.oracle_qkv_mxfp4.restype = None
        L.oracle_qkv_mxfp4.argtypes = [_i64, _i64, _p, _p, _p, _p, _p, _p, _p, _i64, _p, _d, _p]
        L.oracle_mlp_fc2.restype = None
        L.oracle_mlp_fc2.argtypes = [_i64, _i64, _p, _p, _p, _i64, _i64, _p, _p, _p, _p, _p]
        L.oracle_mlp.restype = None
        L.oracle_mlp.argtypes = [_i64, _i64, _p, _p, _p, _p, _p, _i64, _i64, _p, _p, _p, _p, _p, _p, _d,
                                 _p, _p, _p, _p, _p, _p]
        _LIB = L
    return _LIB


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def round_bf16(v: float) -> int:
    return int(lib().oracle_round_bf16(float(v)))


def bf16_value(b: int) -> float:
    return float(lib().oracle_bf16_value(int(b)))


def round_e4m3(v: float) -> int:
    return int(lib().oracle_round_e4m3(float(v)))


def e4m3_value(c: int) -> float:
    return float(lib().oracle_e4m3_value(int(c)))


def _default_threads():
    return max(1, min(16, os.cpu_count() or 1))


def _fan_out(fn, nrows, threads, min_rows=1):
    threads = max(1, min(threads or _default_threads(), nrows))
    if threads == 1 or nrows <= min_rows:
        fn(0, nrows)
        return 1
    bounds = np.linspace(0, nrows, threads + 1).astype(np.int64)
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda t: fn(int(bounds[t]), int(bounds[t + 1])), range(threads)))
    return threads


def _table(t):
    """(base array, element offset, rows, row stride) of a synth.Table-like object."""
    return t.base, int(t.offset), int(t.rows), int(t.row_stride)


def _table_ptr(base, offset):
    return ctypes.c_void_p(base.ctypes.data + 2 * offset)


def pre_attn(d, rows_sel=None, threads=None):
    """Oracle of the bf16 pre-attention stage on the rows rows_sel (default all).

    Returns (workspace [R,5376] uint16, out [R,56,3,128] uint16) for the selected rows.
    """
    M = d["M"]
    sel = np.arange(M, dtype=np.int64) if rows_sel is None else np.asarray(rows_sel, np.int64)
    R = sel.size
    x = _c(d["x"].reshape(M, HIDDEN)[sel], np.uint16)
    idx = _c(d["adaln_index"][sel], np.int64)
    pos = sel.copy() if d.get("rope_positions") is None else _c(d["rope_positions"][sel], np.int64)
    sc_b, sc_o, rows, ld = _table(d["adaln_scale"])
    sh_b, sh_o, rows2, ld2 = _table(d["adaln_shift"])
    assert rows == rows2 and ld == ld2
    W = _c(d["qkv_weight"], np.uint16)
    xw = _c(d["x_norm_weight"], np.uint16)
    qw = _c(d["q_norm_weight"], np.uint16)
    kw = _c(d["k_norm_weight"], np.uint16)
    cs = _c(d["rope_cos_sin"], np.uint16)
    S = int(d["S"])
    ws = np.zeros((R, HIDDEN), np.uint16)
    out = np.zeros((R, HEADS, 3, HEAD_DIM), np.uint16)
    L = lib()
    qk_eps = d["qk_eps"] if d.get("qk_eps") is not None else d["eps"]
    eps32 = float(np.float32(d["eps"]))
    qk32 = float(np.float32(qk_eps))

    def run(r0, r1):
        L.oracle_pre_attn(r0, r1, _ptr(x), _ptr(xw), _table_ptr(sc_b, sc_o), _table_ptr(sh_b, sh_o), rows, ld,
                          _ptr(idx), _ptr(W), _ptr(qw), _ptr(kw), _ptr(cs), S, _ptr(pos), eps32, qk32,
                          _ptr(ws), _ptr(out))

    _fan_out(run, R, threads)
    return ws, out


def ulysses_pack(out_rows, P):
    """Destination-major pack of pre-attention outputs for P Ulysses destinations.

    out_rows is [M, 56, 3, 128] (one row per token, heads in q/k/v weight order, as pre_attn
    returns it).  The bf16 pre-attention page gives out the shape [P, M, 56 // P, 3, 128] with
    P in {1, 2, 4, 8}; destination p takes the contiguous head block [p * 56 // P, (p + 1) *
    56 // P) of every token (reading: the all-to-all that consumes out sends block p to rank p).
    Returns that [P, M, 56 // P, 3, 128] array.
    """
    if P not in (1, 2, 4, 8):
        raise ValueError(f"ulysses degree {P} is not one of 1, 2, 4, 8")
    a = np.asarray(out_rows)
    M = a.shape[0]
    hl = HEADS // P
    packed = np.empty((P, M, hl, 3, HEAD_DIM), a.dtype)
    for p in range(P):
        packed[p] = a[:, p * hl:(p + 1) * hl]
    return packed


def quant_out_e4m3(out_bits, q_descale, k_descale, v_descale):
    """e4m3 output mode: codes of the packed bf16 pre-attention output (uint16 bit patterns,
    trailing axes [3, 128]), code = e4m3(fl32(v / descale)) with the descale of the element's
    kind, saturating at 448 ("minimax_h3_nvfp4_pre_attention", Parameters: out_mode and
    q/k/v_descale).  The descales are fp32 values."""
    a = np.ascontiguousarray(out_bits, dtype=np.uint16)
    assert a.shape[-2:] == (3, HEAD_DIM), a.shape
    code = np.empty(a.shape, dtype=np.uint8)
    lib().oracle_quant_out_e4m3(_ptr(a), a.size, float(np.float32(q_descale)), float(np.float32(k_descale)),
                                float(np.float32(v_descale)), _ptr(code))
    return code


def out_proj(d, rows_sel=None, threads=None):
    """Oracle of the bf16 out-projection with gated residual; returns out [R,5376] uint16."""
    M = d["M"]
    sel = np.arange(M, dtype=np.int64) if rows_sel is None else np.asarray(rows_sel, np.int64)
    R = sel.size
    attn = _c(d["attn_out"].reshape(M, ATTN_WIDTH)[sel], np.uint16)
    gi = _c(d["gate_index"][sel], np.int32)
    res = _c(d["residual"].reshape(M, HIDDEN)[sel], np.uint16)
    g_b, g_o, rows, ld = _table(d["gate"])
    Wo = _c(d["o_weight"], np.uint16)
    out = np.zeros((R, HIDDEN), np.uint16)
    L = lib()

    def run(r0, r1):
        L.oracle_out_proj(r0, r1, _ptr(attn), _ptr(Wo), _table_ptr(g_b, g_o), rows, ld, _ptr(gi), _ptr(res),
                          _ptr(out))

    _fan_out(run, R, threads)
    return out


def e2m1_value(c: int) -> float:
    return lib().oracle_e2m1_value(c)


def round_e2m1(v: float) -> int:
    return lib().oracle_round_e2m1(v)


def mx_scale_exp(amax: float) -> int:
    return lib().oracle_mx_scale_exp(amax)


def mx_quant_fp4(x_bits, threads=None):
    """MXFP4 of bf16 rows x [R, K] (uint16 bits, K % 32 == 0): (codes [R, K/2] uint8 with element
    2j in the low nibble of byte j, scales [R, K/32] uint8 E8M0, row-major)."""
    x = _c(x_bits, np.uint16)
    R, K = x.shape
    codes = np.zeros((R, K // 2), np.uint8)
    scales = np.zeros((R, K // 32), np.uint8)
    L = lib()

    def run(r0, r1):
        L.oracle_mx_quant_fp4(ctypes.c_void_p(x.ctypes.data + 2 * r0 * K), r1 - r0, K,
                              ctypes.c_void_p(codes.ctypes.data + r0 * (K // 2)),
                              ctypes.c_void_p(scales.ctypes.data + r0 * (K // 32)))

    _fan_out(run, R, threads)
    return codes, scales


def mx_values(codes, scales):
    """The values of MXFP4 rows (codes [R, K/2], row-major scales [R, K/32]) as float64, through
    the oracle's own E2M1 decoder."""
    codes = np.asarray(codes, np.uint8)
    tab = np.array([e2m1_value(c) for c in range(16)])
    R, H = codes.shape
    v = np.empty((R, 2 * H))
    v[:, 0::2] = tab[codes & 15]
    v[:, 1::2] = tab[codes >> 4]
    return v * np.exp2(np.repeat(np.asarray(scales, np.float64) - 127.0, 32, axis=1))


def out_proj_mxfp4(a_codes, a_scales, w_codes, w_scales, d, rows_sel=None, threads=4):
    """Oracle of the MXFP4 W4A4 out-projection with gated residual on the rows rows_sel of the
    activation codes/scales [M, 3584] / [M, 224] (row-major) and weight codes/scales [5376, 3584] /
    [5376, 224]; gate, gate_index and residual come from d.  Returns out [R, 5376] uint16.  Each
    call holds W's values in 308 MB of doubles, so few threads."""
    M = d["M"]
    sel = np.arange(M, dtype=np.int64) if rows_sel is None else np.asarray(rows_sel, np.int64)
    R = sel.size
    ac = _c(np.asarray(a_codes)[sel], np.uint8)
    asc = _c(np.asarray(a_scales)[sel], np.uint8)
    wc = _c(w_codes, np.uint8)
    wsc = _c(w_scales, np.uint8)
    gi = _c(d["gate_index"][sel], np.int32)
    res = _c(d["residual"].reshape(M, HIDDEN)[sel], np.uint16)
    g_b, g_o, rows, ld = _table(d["gate"])
    out = np.zeros((R, HIDDEN), np.uint16)
    L = lib()

    def run(r0, r1):
        L.oracle_out_proj_mxfp4(r0, r1, _ptr(ac), _ptr(asc), _ptr(wc), _ptr(wsc), _table_ptr(g_b, g_o), rows, ld,
                                _ptr(gi), _ptr(res), _ptr(out))

    _fan_out(run, R, threads)
    return out


def norm_adaln(d, rows_sel=None, threads=None):
    """The pre-attention workspace a [R, 5376] (uint16 bits) of the rows rows_sel."""
    M = d["M"]
    sel = np.arange(M, dtype=np.int64) if rows_sel is None else np.asarray(rows_sel, np.int64)
    R = sel.size
    x = _c(d["x"].reshape(M, HIDDEN)[sel], np.uint16)
    idx = _c(d["adaln_index"][sel], np.int64)
    sc_b, sc_o, rows, ld = _table(d["adaln_scale"])
    sh_b, sh_o, _, _ = _table(d["adaln_shift"])
    xw = _c(d["x_norm_weight"], np.uint16)
    ws = np.zeros((R, HIDDEN), np.uint16)
    L = lib()

    def run(r0, r1):
        L.oracle_norm_adaln(r0, r1, _ptr(x), _ptr(xw), _table_ptr(sc_b, sc_o), _table_ptr(sh_b, sh_o), rows, ld,
                            _ptr(idx), float(np.float32(d["eps"])), _ptr(ws))

    _fan_out(run, R, threads)
    return ws


def qkv_mxfp4(ws_codes, ws_scales, w_codes, w_scales, d, rows_sel=None, threads=None):
    """The MXFP4 QKV GEMM and the pre-attention epilogue on the workspace codes/scales of rows
    rows_sel ([R, 2688] / [R, 168] row-major, already selected) and the weight's ([21504, 2688] /
    [21504, 168]); positions, cos/sin and norm weights from d.  Returns out [R, 56, 3, 128]."""
    M = d["M"]
    sel = np.arange(M, dtype=np.int64) if rows_sel is None else np.asarray(rows_sel, np.int64)
    R = sel.size
    pos = sel.copy() if d.get("rope_positions") is None else _c(d["rope_positions"][sel], np.int64)
    qk_eps = d["qk_eps"] if d.get("qk_eps") is not None else d["eps"]
    ac, asc = _c(ws_codes, np.uint8), _c(ws_scales, np.uint8)
    wc, wsc = _c(w_codes, np.uint8), _c(w_scales, np.uint8)
    qw, kw = _c(d["q_norm_weight"], np.uint16), _c(d["k_norm_weight"], np.uint16)
    cs = _c(d["rope_cos_sin"], np.uint16)
    out = np.zeros((R, HEADS, 3, HEAD_DIM), np.uint16)
    L = lib()

    def run(r0, r1):
        L.oracle_qkv_mxfp4(r0, r1, _ptr(ac), _ptr(asc), _ptr(wc), _ptr(wsc), _ptr(qw), _ptr(kw), _ptr(cs),
                           int(d["S"]), _ptr(pos), float(np.float32(qk_eps)), _ptr(out))

    _fan_out(run, R, threads)
    return out


def pre_attn_mxfp4(d, w_codes, w_scales, rows_sel=None, threads=None):
    """The MXFP4 W4A4 pre-attention of the rows rows_sel: the workspace a, its MXFP4 codes and
    scales (row-major), and out [R, 56, 3, 128]."""
    ws = norm_adaln(d, rows_sel, threads)
    c, s = mx_quant_fp4(ws, threads)
    return ws, c, s, qkv_mxfp4(c, s, w_codes, w_scales, d, rows_sel, threads)


def mlp_fc2(y_q, y_scale, d, rows_sel=None, threads=None):
    """The MLP's FC2 + gated residual stage alone, on given codes y_q [R, 14336] u8 and scales
    y_scale [R] f32 of the rows rows_sel (already selected), with those rows' index and residual
    from d: out [R, 5376] u16.  The reference for that stage on another path's own y_q."""
    M = d["M"]
    sel = np.arange(M, dtype=np.int64) if rows_sel is None else np.asarray(rows_sel, np.int64)
    R = sel.size
    yq = _c(y_q, np.uint8)
    ys = _c(y_scale, np.float32)
    assert yq.shape == (R, INTER) and ys.shape == (R,)
    idx = _c(d["adaln_index"][sel], np.int64)
    res = _c(d["residual"].reshape(M, HIDDEN)[sel], np.uint16)
    g_b, g_o, rows, ld = _table(d["gate"])
    W2 = _c(d["fc2_q"], np.uint8)
    s2 = _c(d["fc2_scale"], np.float32)
    out = np.zeros((R, HIDDEN), np.uint16)
    L = lib()

    def run(r0, r1):
        L.oracle_mlp_fc2(r0, r1, _ptr(yq), _ptr(ys), _table_ptr(g_b, g_o), rows, ld, _ptr(idx), _ptr(res), _ptr(W2),
                         _ptr(s2), _ptr(out))

    _fan_out(run, R, threads)
    return out


def mlp(d, rows_sel=None, threads=None):
    """Oracle of the FP8 W8A8 MLP block on the selected rows.

    Returns a dict with a_q [R,5376] u8, a_scale [R] f32, y [R,14336] u16, y_q [R,14336] u8,
    y_scale [R] f32, out [R,5376] u16.
    """
    M = d["M"]
    sel = np.arange(M, dtype=np.int64) if rows_sel is None else np.asarray(rows_sel, np.int64)
    R = sel.size
    x = _c(d["x"].reshape(M, HIDDEN)[sel], np.uint16)
    idx = _c(d["adaln_index"][sel], np.int64)
    res = _c(d["residual"].reshape(M, HIDDEN)[sel], np.uint16)
    sc_b, sc_o, rows, ld = _table(d["adaln_scale"])
    sh_b, sh_o, rows2, ld2 = _table(d["adaln_shift"])
    g_b, g_o, rows3, ld3 = _table(d["gate"])
    assert rows == rows2 == rows3 and ld == ld2 == ld3
    xw = _c(d["x_norm_weight"], np.uint16)
    W1 = _c(d["fc1_q"], np.uint8)
    s1 = _c(d["fc1_scale"], np.float32)
    W2 = _c(d["fc2_q"], np.uint8)
    s2 = _c(d["fc2_scale"], np.float32)
    o = {
        "a_q": np.zeros((R, HIDDEN), np.uint8), "a_scale": np.zeros(R, np.float32),
        "y": np.zeros((R, INTER), np.uint16), "y_q": np.zeros((R, INTER), np.uint8),
        "y_scale": np.zeros(R, np.float32), "out": np.zeros((R, HIDDEN), np.uint16),
    }
    L = lib()
    eps32 = float(np.float32(d["eps"]))

    def run(r0, r1):
        L.oracle_mlp(r0, r1, _ptr(x), _ptr(xw), _table_ptr(sc_b, sc_o), _table_ptr(sh_b, sh_o),
                     _table_ptr(g_b, g_o), rows, ld, _ptr(idx), _ptr(res), _ptr(W1), _ptr(s1), _ptr(W2), _ptr(s2),
                     eps32, _ptr(o["a_q"]), _ptr(o["a_scale"]), _ptr(o["y"]), _ptr(o["y_q"]), _ptr(o["y_scale"]),
                     _ptr(o["out"]))

    _fan_out(run, R, threads)
    return o
