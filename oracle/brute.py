"""Brute-force NumPy transcription of the MiniMax-H3 stage formulas, for one or two rows.

TEST INFRASTRUCTURE ONLY.  A second, independently written reading of the same pages as
dit_oracle.c (vectorised float64 NumPy instead of C loops, its own rounding helpers), used
only to cross-check that oracle on tiny inputs.  Sources: the per-row formula block of the
fp8 MLP page, the bf16 pre-attention page's description and parameter list, and the nvfp4
out-proj page's gated-residual description.
"""
from __future__ import annotations

import numpy as np

HIDDEN, HEADS, HEAD_DIM = 5376, 56, 128


def bf16_of_bits(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rne_bf16(v):
    """Round float64 values to the nearest bf16 value (returned as float64), ties to even."""
    v = np.asarray(v, np.float64)
    m, e = np.frexp(np.abs(v))                      # |v| = m * 2^e, m in [0.5, 1)
    step_exp = np.where(e - 1 >= -126, e - 8, -133)
    r = np.rint(np.ldexp(np.abs(v), -step_exp))     # np.rint rounds half to even
    return np.copysign(np.ldexp(r, step_exp), v)


def bits_of_bf16(v):
    return (np.asarray(v, np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def rne_e4m3_value(v):
    """Round to the nearest float8_e4m3fn value, ties to even, saturating at +-448."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    m, e = np.frexp(a)
    step_exp = np.where(e - 1 >= -6, e - 4, -9)
    r = np.ldexp(np.rint(np.ldexp(a, -step_exp)), step_exp)
    r = np.minimum(r, 448.0)
    return np.copysign(r, v)


def e4m3_code_of_value(v):
    """Code byte of an exactly representable e4m3fn value."""
    v = np.asarray(v, np.float64)
    sign = np.signbit(v).astype(np.uint8) << 7
    a = np.abs(v)
    code = np.zeros(v.shape, np.uint8)
    nz = a > 0
    m, e = np.frexp(np.where(nz, a, 1.0))
    E = e - 1
    normal = nz & (E >= -6)
    mant = np.round((np.ldexp(np.where(nz, a, 1.0), -E) - 1.0) * 8).astype(np.int64)
    code = np.where(normal, ((E + 7) << 3) | mant, code)
    sub = nz & ~normal
    code = np.where(sub, np.round(np.ldexp(np.where(nz, a, 0.0), 9)).astype(np.int64), code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e4m3_of_code(c):
    c = np.asarray(c, np.uint8).astype(np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    ex = (c >> 3) & 15
    mt = c & 7
    v = np.where(ex == 0, np.ldexp(mt.astype(np.float64), -9), np.ldexp(1.0 + mt / 8.0, ex - 7))
    return s * v


def _tab_rows(t):
    out = np.empty((t.rows, t.cols), np.uint16)
    for r in range(t.rows):
        s = t.offset + r * t.row_stride
        out[r] = t.base[s:s + t.cols]
    return out


def norm_adaln(x_bits, xw_bits, scale_t, shift_t, idx, eps):
    """a for each row (float64 values on the bf16 grid) and the per-row valid flag."""
    x = bf16_of_bits(x_bits)
    w = bf16_of_bits(xw_bits)
    sc = bf16_of_bits(_tab_rows(scale_t))
    sh = bf16_of_bits(_tab_rows(shift_t))
    rows = scale_t.rows
    R = x.shape[0]
    a = np.zeros_like(x)
    valid = np.zeros(R, bool)
    for m in range(R):
        i = int(idx[m])
        if not (0 <= i < rows):
            continue
        valid[m] = True
        rinv = 1.0 / np.sqrt(np.mean(x[m] ** 2) + eps)
        n = rne_bf16(x[m] * rinv * w)
        a[m] = rne_bf16(sh[i] + n * rne_bf16(1.0 + sc[i]))
    return a, valid


def pre_attn(d, rows_sel):
    M = d["M"]
    sel = np.asarray(rows_sel, np.int64)
    eps = float(np.float32(d["eps"]))
    a, _ = norm_adaln(d["x"].reshape(M, HIDDEN)[sel], d["x_norm_weight"], d["adaln_scale"], d["adaln_shift"],
                      d["adaln_index"][sel], eps)
    W = bf16_of_bits(d["qkv_weight"]).reshape(3, HEADS, HEAD_DIM, HIDDEN)
    qkv = rne_bf16(np.einsum("rk,thdk->rthd", a, W))           # [R, kind, head, dim]
    return bits_of_bf16(a), _qkv_epilogue(d, sel, qkv)


def _qkv_epilogue(d, sel, qkv):
    """qkv [R, kind, head, dim] (bf16 values) -> packed out bits [R, head, kind, dim]."""
    qk_eps = float(np.float32(d["qk_eps"] if d.get("qk_eps") is not None else d["eps"]))
    S = d["S"]
    cs = bf16_of_bits(d["rope_cos_sin"]).reshape(S, 96)
    pos = sel if d.get("rope_positions") is None else d["rope_positions"][sel]
    pos = np.clip(pos, 0, S - 1)
    out = np.empty_like(qkv)
    out[:, 2] = qkv[:, 2]
    for kind, wbits in ((0, d["q_norm_weight"]), (1, d["k_norm_weight"])):
        v = qkv[:, kind]                                         # [R, H, 128]
        w = bf16_of_bits(wbits)
        r2 = 1.0 / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + qk_eps)
        u = rne_bf16(v * r2 * w)
        c = cs[pos, None, :48]
        s = cs[pos, None, 48:]
        x1, x2 = u[..., :48], u[..., 48:96]
        # NeoX rotate-half: [x1, x2] * cos + [-x2, x1] * sin
        out[:, kind, :, :48] = rne_bf16(x1 * c - x2 * s)
        out[:, kind, :, 48:96] = rne_bf16(x2 * c + x1 * s)
        out[:, kind, :, 96:] = u[..., 96:]
    packed = np.transpose(out, (0, 2, 1, 3))                    # [R, head, kind, dim]
    return bits_of_bf16(packed)


# ---- MXFP4 (OCP Microscaling): its own NumPy reading of the format, for the cross-check

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def mx_quant(x_bits):
    """bf16 rows [R, K] -> (codes [R, K/2], scales [R, K/32]): per 32-block, X = 2^(floor(log2
    amax) - 2) (byte clamped to [0, 254], 0 for a zero block); each element the nearest E2M1
    magnitude of |v| / X (the two grid neighbours compared, a tie going to the even index),
    6 beyond the grid, sign bit from v."""
    v = bf16_of_bits(x_bits)
    R, K = v.shape
    v = v.reshape(R, K // 32, 32)
    amax = np.abs(v).max(axis=2)
    _, e = np.frexp(amax)
    E = np.where(amax > 0, np.clip(e - 3 + 127, 0, 254), 0)
    y = np.abs(v) / np.exp2(E - 127.0)[..., None]
    lo = np.clip(np.searchsorted(E2M1, y, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    d_lo, d_hi = y - E2M1[lo], E2M1[hi] - y
    up = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(y >= 6.0, 7, np.where(up, hi, lo))
    code = (idx | (np.signbit(v).astype(np.int64) << 3)).reshape(R, K).astype(np.uint8)
    return (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8), E.astype(np.uint8)


def mx_values(codes, scales):
    c = np.asarray(codes, np.uint8)
    R, H = c.shape
    nib = np.empty((R, 2 * H), np.int64)
    nib[:, 0::2], nib[:, 1::2] = c & 15, c >> 4
    mag = E2M1[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    return mag * np.exp2(np.repeat(np.asarray(scales, np.float64) - 127.0, 32, axis=1))


def qkv_mxfp4(d, rows_sel, ws_codes, ws_scales, w_codes, w_scales):
    """The MXFP4 QKV product of the given workspace codes (rows rows_sel) and weight codes, then
    the pre-attention epilogue."""
    sel = np.asarray(rows_sel, np.int64)
    A = mx_values(ws_codes, ws_scales)
    acc = np.empty((A.shape[0], 3 * HEADS * HEAD_DIM))
    for n0 in range(0, acc.shape[1], 2048):                     # W's values a slab at a time
        acc[:, n0:n0 + 2048] = A @ mx_values(w_codes[n0:n0 + 2048], w_scales[n0:n0 + 2048]).T
    qkv = rne_bf16(acc).reshape(-1, 3, HEADS, HEAD_DIM)
    return _qkv_epilogue(d, sel, qkv)


def out_proj(d, rows_sel):
    M = d["M"]
    sel = np.asarray(rows_sel, np.int64)
    attn = bf16_of_bits(d["attn_out"].reshape(M, -1)[sel])
    Wo = bf16_of_bits(d["o_weight"]).reshape(HIDDEN, -1)
    o = rne_bf16(attn @ Wo.T)
    gt = bf16_of_bits(_tab_rows(d["gate"]))
    gi = d["gate_index"][sel].astype(np.int64)
    ok = (gi >= 0) & (gi < d["gate"].rows)
    g = np.where(ok[:, None], gt[np.where(ok, gi, 0)], 0.0)
    res = bf16_of_bits(d["residual"].reshape(M, HIDDEN)[sel])
    return bits_of_bf16(rne_bf16(res + rne_bf16(g * o)))


def _quant(v):
    amax = np.max(np.abs(v), axis=-1)
    s = (amax / 448.0).astype(np.float32).astype(np.float64)
    q = np.zeros_like(v)
    nz = s > 0
    q[nz] = rne_e4m3_value((v[nz] / s[nz, None]).astype(np.float32).astype(np.float64))
    return q, s


def mlp(d, rows_sel):
    M = d["M"]
    sel = np.asarray(rows_sel, np.int64)
    eps = float(np.float32(d["eps"]))
    idx = d["adaln_index"][sel]
    a, valid = norm_adaln(d["x"].reshape(M, HIDDEN)[sel], d["x_norm_weight"], d["adaln_scale"], d["adaln_shift"],
                          idx, eps)
    aq, sa = _quant(a)
    W1 = e4m3_of_code(d["fc1_q"])
    h = rne_bf16((aq @ W1.T) * sa[:, None] * d["fc1_scale"].astype(np.float64)[None, :])
    hg, hu = h[:, :14336], h[:, 14336:]
    silu = rne_bf16(hg / (1.0 + np.exp(-hg)))
    y = rne_bf16(silu * hu)
    yq, sy = _quant(y)
    W2 = e4m3_of_code(d["fc2_q"])
    o = rne_bf16((yq @ W2.T) * sy[:, None] * d["fc2_scale"].astype(np.float64)[None, :])
    gt = bf16_of_bits(_tab_rows(d["gate"]))
    g = np.where(valid[:, None], gt[np.where(valid, idx, 0)], 0.0)
    res = bf16_of_bits(d["residual"].reshape(M, HIDDEN)[sel])
    out = rne_bf16(res + rne_bf16(g * o))
    return {"a_q": e4m3_code_of_value(aq), "a_scale": sa.astype(np.float32), "y": bits_of_bf16(y),
            "y_q": e4m3_code_of_value(yq), "y_scale": sy.astype(np.float32), "out": bits_of_bf16(out)}
