"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: textbook encodings, torch
library routines (dtype conversions, rms_norm, silu, float64 matmul), closed forms of special
cases (one-hot weights, exact rotation angles, unit or zero tables) and invariants.  The last
group cross-checks it with the independent NumPy transcription on one and two rows.
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import brute
from tests.helpers import (bf16_val, e4m3_val, is_nearest_bf16, ordered_e4m3, torch_e4m3, ulp_diff_bf16)

GOLD = os.path.join(os.path.dirname(__file__), "golden")
H, NH, HD = synth.HIDDEN, synth.HEADS, synth.HEAD_DIM
INT64_MIN, INT64_MAX = -(1 << 63), (1 << 63) - 1


def _golden(name):
    rows = []
    for line in open(os.path.join(GOLD, name)):
        line = line.split("#")[0].strip()
        if line:
            v, c = line.split()
            rows.append((float(v), int(c, 16)))
    return rows


# ---------------------------------------------------------------- number formats

def test_golden_e4m3_encodings():
    for v, c in _golden("e4m3fn_codes.txt"):
        assert oracle.round_e4m3(v) == c, (v, hex(c))
        assert oracle.e4m3_value(c) == v


def test_golden_bf16_encodings():
    for v, c in _golden("bf16_codes.txt"):
        assert oracle.round_bf16(v) == c, (v, hex(c))


def test_round_bf16_matches_torch_on_fp32_values():
    g = np.random.Generator(np.random.PCG64(1))
    bits = g.integers(0, 1 << 32, size=20000, dtype=np.uint64).astype(np.uint32)
    bits[:4000] = (bits[:4000] & 0xFFFF0000) | 0x8000          # exact ties
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) < 3.3e38)]
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.round_bf16(float(t)) for t in v], np.uint16)
    assert np.array_equal(got, ref)


def test_round_bf16_is_single_rounding_from_double():
    # 1 + 2^-8 + 2^-30 lies just above a bf16 tie; rounding through fp32 first would land on
    # the tie and go to even (1.0).  The nearest bf16 is 1 + 2^-7.
    assert oracle.round_bf16(1 + 2**-8 + 2**-30) == 0x3F81
    assert oracle.round_bf16(-(1 + 2**-8 + 2**-30)) == 0xBF81


def test_round_e4m3_matches_torch_in_range():
    g = np.random.Generator(np.random.PCG64(2))
    v = (g.standard_normal(20000) * np.exp2(g.integers(-12, 9, 20000))).astype(np.float32)
    v = np.clip(v, -448, 448).astype(np.float32)
    # exact ties between neighbouring codes, normal and subnormal
    ties = []
    for c in range(0, 0x7E):
        a, b = oracle.e4m3_value(c), oracle.e4m3_value(c + 1)
        ties += [(a + b) / 2, -(a + b) / 2]
    v = np.concatenate([v, np.array(ties, np.float32)])
    ref = torch_e4m3(v)
    got = np.array([oracle.round_e4m3(float(t)) for t in v], np.uint8)
    assert np.array_equal(got, ref)


def test_round_e4m3_saturates():
    for v in (448.0, 449.0, 463.9, 464.0, 480.0, 1e6, 3.0e38):
        assert oracle.round_e4m3(v) == 0x7E
        assert oracle.round_e4m3(-v) == 0xFE


# ---------------------------------------------------------------- pre-attention inputs

_W_RANDOM = {}


def _random_qkv_weight():
    if "w" not in _W_RANDOM:
        _W_RANDOM["w"] = synth.to_bf16_bits(synth.normal(7, "qkv_weight", (synth.QKV_ROWS, H), 1 / math.sqrt(H)))
    return _W_RANDOM["w"]


def _one_hot_k(n):
    return (n * 5 + 3) % H


def _one_hot_qkv_weight():
    W = np.zeros((synth.QKV_ROWS, H), np.uint16)
    n = np.arange(synth.QKV_ROWS)
    W[n, _one_hot_k(n)] = 0x3F80
    return W


def _pre(M, weight, seed=11, **kw):
    return synth.pre_attn_inputs(M, seed=seed, weight=weight, **kw)


def _set_tables(d, scale_rows, shift_rows):
    rows = scale_rows.shape[0]
    d["adaln_scale"] = synth.Table(synth.to_bf16_bits(scale_rows).reshape(-1), 0, rows, H)
    d["adaln_shift"] = synth.Table(synth.to_bf16_bits(shift_rows).reshape(-1), 0, rows, H)
    d["rows"] = rows


def _set_cache(d, cos, sin):
    """Cache with the given [S,48] cos/sin columns."""
    d["rope_cos_sin"] = synth.to_bf16_bits(np.concatenate([cos, sin], axis=1).astype(np.float32))
    d["S"] = cos.shape[0]


def _unit_qk(d):
    d["q_norm_weight"] = np.full(HD, 0x3F80, np.uint16)
    d["k_norm_weight"] = np.full(HD, 0x3F80, np.uint16)


def _rmsnorm_lib(x64, w64, eps):
    return torch.nn.functional.rms_norm(torch.from_numpy(x64), (x64.shape[-1],), torch.from_numpy(w64),
                                        eps).numpy()


# ---------------------------------------------------------------- norm + AdaLN

def test_guard_zeroes_rows_for_any_out_of_range_int64():
    M = 8
    d = _pre(M, _one_hot_qkv_weight(), rows=3, wide_tables=False, bad_index_frac=0.0)
    bad = [-1, 3, 1 << 32, -(1 << 32), INT64_MIN, INT64_MAX]
    d["adaln_index"][:6] = bad
    d["adaln_index"][6:] = [0, 2]
    ws, out = oracle.pre_attn(d)
    assert np.all(ws[:6] == 0)                       # +0 bit patterns
    assert np.all(bf16_val(out[:6]) == 0.0)          # value zero (sign of zero not fixed)
    assert np.all(ws[6:] != 0)


def test_identity_modulation_is_rmsnorm():
    # one table row, scale = 0, shift = 0: a = bf16(rmsnorm(x) * w) (library rms_norm in float64)
    M = 3
    d = _pre(M, _one_hot_qkv_weight(), rows=1, wide_tables=False, bad_index_frac=0.0)
    _set_tables(d, np.zeros((1, H), np.float32), np.zeros((1, H), np.float32))
    d["adaln_index"][:] = 0
    ws, _ = oracle.pre_attn(d)
    x = bf16_val(d["x"]).reshape(M, H)
    w = bf16_val(d["x_norm_weight"])
    ref = _rmsnorm_lib(x, w, float(np.float32(d["eps"])))
    assert is_nearest_bf16(ws, ref).all()


def test_constant_row_closed_form():
    # x = c on every column with unit weight: n = bf16(c / sqrt(c^2 + eps)).  The small c makes
    # eps visible (2^-9: c^2 = 3.8e-6 against eps = 1e-5).
    c = [0.375, -3.0, 2.0 ** -9]
    M = len(c)
    d = _pre(M, _one_hot_qkv_weight(), rows=1, wide_tables=False, bad_index_frac=0.0)
    _set_tables(d, np.zeros((1, H), np.float32), np.zeros((1, H), np.float32))
    d["adaln_index"][:] = 0
    d["x"] = synth.to_bf16_bits(np.array([[v] * H for v in c], np.float32))
    d["x_norm_weight"] = np.full(H, 0x3F80, np.uint16)
    ws, _ = oracle.pre_attn(d)
    eps = float(np.float32(1e-5))
    for m in range(M):
        exact = c[m] / math.sqrt(c[m] ** 2 + eps)
        assert np.all(ws[m] == oracle.round_bf16(exact))
        assert is_nearest_bf16(ws[m][:1], [exact]).all()


def test_modulation_special_rows():
    # row 0: scale = -1 (bf16(1+scale) = 0) so a = shift exactly; row 1: scale = 1, shift = 0
    # so a = 2n exactly.  Pins the table row chosen, the shift/scale roles and the 1+scale.
    M = 4
    d = _pre(M, _one_hot_qkv_weight(), rows=2, wide_tables=True, bad_index_frac=0.0)
    g = np.random.Generator(np.random.PCG64(3))
    shift0 = g.standard_normal(H).astype(np.float32) * 0.3
    sc = np.stack([np.full(H, -1.0), np.full(H, 1.0)]).astype(np.float32)
    sh = np.stack([shift0, np.zeros(H)]).astype(np.float32)
    # keep the wide layout: rebuild a [2, 6*5376] matrix with shift = chunk 0, scale = chunk 1
    wide = np.zeros((2, 6 * H), np.float32)
    wide[:, 0:H] = sh
    wide[:, H:2 * H] = sc
    wide[:, 2 * H:] = 7.0                       # unrelated chunks must not be read
    base = synth.to_bf16_bits(wide).reshape(-1)
    d["adaln_shift"] = synth.Table(base, 0, 2, 6 * H)
    d["adaln_scale"] = synth.Table(base, H, 2, 6 * H)
    d["adaln_index"][:] = [0, 1, 1, 0]
    ws, _ = oracle.pre_attn(d)
    # n from the identity modulation
    d2 = dict(d)
    _set_tables(d2, np.zeros((1, H), np.float32), np.zeros((1, H), np.float32))
    d2["adaln_index"] = np.zeros(M, np.int64)
    n_bits, _ = oracle.pre_attn(d2)
    sh_bits = synth.to_bf16_bits(shift0)
    for m in (0, 3):
        assert np.array_equal(ws[m], sh_bits)
    for m in (1, 2):
        assert np.array_equal(bf16_val(ws[m]), 2.0 * bf16_val(n_bits[m]))


# ---------------------------------------------------------------- GEMM, pack, Q/K norm, RoPE

def _pack_case(M=3, cos=None, sin=None, seed=12):
    d = _pre(M, _one_hot_qkv_weight(), seed=seed, rows=2, wide_tables=True, bad_index_frac=0.0, S=M,
             positions="identity")
    _unit_qk(d)
    if cos is None:
        cos = np.ones((M, 48), np.float32)
        sin = np.zeros((M, 48), np.float32)
    _set_cache(d, cos, sin)
    return d


def test_pack_one_hot_v_heads_bit_exact():
    d = _pack_case()
    ws, out = oracle.pre_attn(d)
    M = d["M"]
    for m in range(M):
        for h in range(NH):
            n = 2 * NH * HD + h * HD + np.arange(HD)
            assert np.array_equal(out[m, h, 2], ws[m, _one_hot_k(n)])


def test_qk_norm_one_hot_matches_library_rmsnorm():
    d = _pack_case()
    ws, out = oracle.pre_attn(d)
    qk_eps = float(np.float32(d["qk_eps"]))
    for kind in (0, 1):
        n = kind * NH * HD + np.arange(NH * HD)
        v = bf16_val(ws[:, _one_hot_k(n)]).reshape(-1, NH, HD)      # qkv = a[k(n)] exactly
        ref = _rmsnorm_lib(v, np.ones(HD), qk_eps)
        assert is_nearest_bf16(out[:, :, kind], ref).all()


def test_qk_norm_unit_rms():
    d = _pack_case(M=2)
    _, out = oracle.pre_attn(d)
    for kind in (0, 1):
        u = bf16_val(out[:, :, kind])
        ms = np.mean(u * u, axis=-1)
        assert np.all(np.abs(ms - 1.0) < 2.0 ** -6), ms


def test_rope_exact_angles_permute_and_negate():
    M = 3
    base = _pack_case(M=M)
    _, out_u = oracle.pre_attn(base)                       # cos = 1, sin = 0: out = u
    cs_pairs = [(1.0, 0.0), (0.0, 1.0), (-1.0, 0.0), (0.0, -1.0)]
    j = np.arange(48)
    c = np.array([cs_pairs[(t + m) % 4][0] for m in range(M) for t in j], np.float32).reshape(M, 48)
    s = np.array([cs_pairs[(t + m) % 4][1] for m in range(M) for t in j], np.float32).reshape(M, 48)
    d = _pack_case(M=M, cos=c, sin=s)
    _, out = oracle.pre_attn(d)
    for m in range(M):
        for kind in (0, 1):
            u = bf16_val(out_u[m, :, kind])
            o = bf16_val(out[m, :, kind])
            for t in range(48):
                cc, ss = cs_pairs[(t + m) % 4]
                exp_lo = u[:, t] * cc - u[:, t + 48] * ss
                exp_hi = u[:, t + 48] * cc + u[:, t] * ss
                assert np.array_equal(o[:, t], exp_lo), (m, kind, t)
                assert np.array_equal(o[:, t + 48], exp_hi), (m, kind, t)
            assert np.array_equal(out[m, :, kind, 96:], out_u[m, :, kind, 96:])   # pass-through
        assert np.array_equal(out[m, :, 2], out_u[m, :, 2])                     # V untouched


def test_rope_random_angles_is_complex_rotation():
    M = 4
    base = _pack_case(M=M)
    _, out_u = oracle.pre_attn(base)
    g = np.random.Generator(np.random.PCG64(5))
    th = g.uniform(0, 2 * np.pi, (M, 48))
    cb = synth.to_bf16_bits(np.cos(th).astype(np.float32))
    sb = synth.to_bf16_bits(np.sin(th).astype(np.float32))
    d = _pack_case(M=M, cos=bf16_val(cb).astype(np.float32), sin=bf16_val(sb).astype(np.float32))
    _, out = oracle.pre_attn(d)
    for kind in (0, 1):
        u = bf16_val(out_u[:, :, kind])
        z = (u[..., :48] + 1j * u[..., 48:96]) * (bf16_val(cb) + 1j * bf16_val(sb))[:, None, :]
        assert is_nearest_bf16(out[:, :, kind, :48], z.real).all()
        assert is_nearest_bf16(out[:, :, kind, 48:96], z.imag).all()
        o = bf16_val(out[:, :, kind])
        n_in = u[..., :48] ** 2 + u[..., 48:96] ** 2
        n_out = o[..., :48] ** 2 + o[..., 48:96] ** 2
        cs2 = (bf16_val(cb) ** 2 + bf16_val(sb) ** 2)[:, None, :]
        assert np.allclose(n_out, n_in * cs2, rtol=2 ** -6, atol=1e-6)
        assert np.array_equal(out[:, :, kind, 96:], out_u[:, :, kind, 96:])


def test_positions_clamp_and_identity():
    M = 4
    d = _pre(M, _one_hot_qkv_weight(), rows=2, wide_tables=True, bad_index_frac=0.0, S=6, positions="identity")
    _, out_id = oracle.pre_attn(d)
    d["rope_positions"] = np.arange(M, dtype=np.int64)
    _, out_ar = oracle.pre_attn(d)
    assert np.array_equal(out_id, out_ar)
    d["rope_positions"] = np.array([-5, 6, INT64_MIN, INT64_MAX], np.int64)
    _, out_bad = oracle.pre_attn(d)
    d["rope_positions"] = np.array([0, 5, 0, 5], np.int64)
    _, out_ok = oracle.pre_attn(d)
    assert np.array_equal(out_bad, out_ok)


def test_qkv_projection_matches_float64_matmul():
    M = 3
    d = _pre(M, _random_qkv_weight(), rows=2, wide_tables=True, bad_index_frac=0.0)
    ws, out = oracle.pre_attn(d)
    Wv = bf16_val(d["qkv_weight"][2 * NH * HD:]).reshape(NH * HD, H)
    ref = bf16_val(ws) @ Wv.T                              # library float64 matmul
    assert is_nearest_bf16(out[:, :, 2].reshape(M, -1), ref, rtol=1e-10).all()


def test_row_permutation():
    M = 4
    d = _pre(M, _random_qkv_weight(), rows=2, wide_tables=True, bad_index_frac=0.0, S=8, positions="random",
             n_bad_positions=1)
    ws, out = oracle.pre_attn(d)
    perm = np.array([2, 0, 3, 1])
    dp = dict(d)
    dp["x"] = d["x"].reshape(M, H)[perm].copy()
    dp["adaln_index"] = d["adaln_index"][perm].copy()
    dp["rope_positions"] = d["rope_positions"][perm].copy()
    wsp, outp = oracle.pre_attn(dp)
    assert np.array_equal(wsp, ws[perm]) and np.array_equal(outp, out[perm])


# ---------------------------------------------------------------- out-projection

def _one_hot_o_weight():
    W = np.zeros((H, synth.ATTN_WIDTH), np.uint16)
    n = np.arange(H)
    W[n, (n * 3 + 1) % synth.ATTN_WIDTH] = 0x3F80
    return W


def test_out_proj_guard_and_gate_rows():
    M = 14
    d = synth.out_proj_inputs(M, seed=3, weight=_one_hot_o_weight())
    gates = np.array([0, 1, 2, -1, 0.5, 4, -2, 1, 1], np.float32)
    d["gate"] = synth.Table(synth.to_bf16_bits(np.repeat(gates[:, None], H, 1)).reshape(-1), 0, 9, H)
    d["gate_index"] = np.array([-1, 9, 10, -(1 << 31), (1 << 31) - 1, 0, 1, 2, 3, 4, 5, 6, 7, 8], np.int32)
    out = oracle.out_proj(d)
    res = d["residual"].reshape(M, H)
    for m in range(6):                                     # guarded or gate 0: out == residual
        assert np.array_equal(out[m], res[m])
    n = np.arange(H)
    o = bf16_val(d["attn_out"].reshape(M, -1)[:, (n * 3 + 1) % synth.ATTN_WIDTH])   # bf16(o) exact
    r = bf16_val(res)
    for m in range(6, M):
        g = gates[d["gate_index"][m]]
        assert is_nearest_bf16(out[m], r[m] + g * o[m]).all(), m     # g*o exact for these gates


def test_out_proj_matches_float64_matmul():
    M = 2
    d = synth.out_proj_inputs(M, seed=4)
    d["gate"] = synth.Table(np.full(9 * H, 0x3F80, np.uint16), 0, 9, H)
    d["gate_index"] = np.array([0, 3], np.int32)
    d["residual"] = np.zeros((M, H), np.uint16)
    out = oracle.out_proj(d)
    ref = bf16_val(d["attn_out"].reshape(M, -1)) @ bf16_val(d["o_weight"]).reshape(H, -1).T
    assert is_nearest_bf16(out, ref, rtol=1e-10).all()


# ---------------------------------------------------------------- FP8 MLP

def _mlp_one_hot(M=4, seed=21):
    W1 = np.zeros((synth.FC1_ROWS, H), np.uint8)
    n = np.arange(synth.FC1_ROWS)
    W1[n, (n * 7 + 2) % H] = 0x38                          # e4m3 1.0
    W2 = np.zeros((H, synth.INTER), np.uint8)
    n2 = np.arange(H)
    W2[n2, (n2 * 11 + 5) % synth.INTER] = 0x38
    w = (W1, np.ones(synth.FC1_ROWS, np.float32), W2, np.ones(H, np.float32))
    d = synth.mlp_inputs(M, seed=seed, weights=w, bad_index_frac=0.0)
    return d


def test_mlp_guard_rows():
    M = 5
    d = _mlp_one_hot(M)
    d["adaln_index"][:] = [-1, 2, INT64_MIN, INT64_MAX, 1]
    o = oracle.mlp(d)
    res = d["residual"].reshape(M, H)
    for m in range(4):
        assert np.all(o["a_q"][m] == 0) and o["a_scale"][m] == 0
        assert np.all(o["y"][m] == 0) and o["y_scale"][m] == 0 and np.all(o["y_q"][m] == 0)
        assert np.array_equal(o["out"][m], res[m])
    assert o["a_scale"][4] > 0


def test_mlp_activation_quant_properties():
    M = 3
    d = _mlp_one_hot(M)
    o = oracle.mlp(d)
    # a from the same rows via the pre-attention oracle's workspace (same norm + AdaLN reading)
    for m in range(M):
        codes = o["a_q"][m]
        s = np.float32(o["a_scale"][m])
        cv = e4m3_val(codes)
        k = np.argmax(np.abs(cv))
        assert abs(cv[k]) == 448.0 and np.max(np.abs(cv)) == 448.0
    # codes are torch's e4m3 conversion of the fp32 quotients a/s (library), reconstructed
    # from the one-hot FC1: h[n] = bf16(a_q[k(n)] * s_a), so a_q codes are observable too
    n = np.arange(synth.FC1_ROWS)
    k = (n * 7 + 2) % H
    for m in range(M):
        s = float(o["a_scale"][m])
        h_exact = e4m3_val(o["a_q"][m][k]) * s
        # y = bf16(bf16(silu(h_g)) * h_u) with library silu
        hg = bf16_val(synth.to_bf16_bits(h_exact[:synth.INTER].astype(np.float32)))
        hu = bf16_val(synth.to_bf16_bits(h_exact[synth.INTER:].astype(np.float32)))
        assert is_nearest_bf16(synth.to_bf16_bits(h_exact.astype(np.float32)), h_exact).all()
        silu = torch.nn.functional.silu(torch.from_numpy(hg)).numpy()
        sb = synth.to_bf16_bits(silu.astype(np.float32))
        assert is_nearest_bf16(sb, silu, rtol=1e-6).all()
        assert is_nearest_bf16(o["y"][m], bf16_val(sb) * hu, rtol=1e-12).all()


def test_mlp_codes_match_library_conversion():
    M = 3
    d = _mlp_one_hot(M)
    o = oracle.mlp(d)
    # reference a from the pre-attention oracle's workspace with the MLP's tables
    dp = {"M": M, "x": d["x"], "x_norm_weight": d["x_norm_weight"], "adaln_scale": d["adaln_scale"],
          "adaln_shift": d["adaln_shift"], "adaln_index": d["adaln_index"], "qkv_weight": _one_hot_qkv_weight(),
          "q_norm_weight": np.full(HD, 0x3F80, np.uint16), "k_norm_weight": np.full(HD, 0x3F80, np.uint16),
          "rope_cos_sin": np.tile(np.array([0x3F80] * 48 + [0] * 48, np.uint16), (M, 1)), "S": M,
          "rope_positions": None, "eps": d["eps"], "qk_eps": d["eps"]}
    a_bits, _ = oracle.pre_attn(dp)
    a = bf16_val(a_bits).astype(np.float32)
    for m in range(M):
        s = np.float32(np.max(np.abs(a[m])) / np.float32(448.0))       # fp32 division
        assert np.float32(o["a_scale"][m]) == s
        q = (a[m] / s).astype(np.float32)                               # fp32 division
        assert np.array_equal(o["a_q"][m], torch_e4m3(q))
        err = np.abs(a[m] - e4m3_val(o["a_q"][m]) * s)
        assert np.all(err <= 2.0 ** -4 * np.abs(a[m]) + 2.0 ** -10 * s)
    for m in range(M):
        y = bf16_val(o["y"][m]).astype(np.float32)
        s = np.float32(np.max(np.abs(y)) / np.float32(448.0))
        assert np.float32(o["y_scale"][m]) == s
        assert np.array_equal(o["y_q"][m], torch_e4m3((y / s).astype(np.float32)))


def test_mlp_subnormal_row_scale_codes_match_library_division():
    # a table row with scale -1 (bf16(1 + scale) = 0) and shift ~1e-37: a = shift exactly, so
    # s_a = RN(amax / 448) is a subnormal fp32 below 2^-128 (1 / s_a overflows); the codes must
    # still be the library e4m3 of the IEEE fp32 quotients a / s_a
    M = 2
    d = _mlp_one_hot(M, seed=23)
    sc, sh = d["adaln_scale"], d["adaln_shift"]
    base = sc.base.copy()
    base[sc.offset + sc.row_stride:sc.offset + sc.row_stride + H] = 0xBF80
    tiny = synth.to_bf16_bits(synth.normal(24, "tiny", (H,), 1e-37))
    base[sh.offset + sh.row_stride:sh.offset + sh.row_stride + H] = tiny
    for t in ("adaln_scale", "adaln_shift", "gate"):
        d[t] = synth.Table(base, d[t].offset, d[t].rows, d[t].row_stride)
    d["adaln_index"][:] = [1, 0]
    o = oracle.mlp(d)
    a = bf16_val(tiny).astype(np.float32)
    s = np.float32(np.max(np.abs(a)) / np.float32(448.0))
    with np.errstate(over="ignore"):
        assert 0 < s < 2.0 ** -128 and not np.isfinite(np.float32(1.0) / s)
    assert np.float32(o["a_scale"][0]) == s
    assert np.array_equal(o["a_q"][0], torch_e4m3((a / s).astype(np.float32)))
    assert np.max(np.abs(e4m3_val(o["a_q"][0]))) == 448.0


def test_mlp_fc2_gated_residual_closed_forms():
    M = 4
    d = _mlp_one_hot(M)
    gates = np.array([0.0, 1.0], np.float32)
    wide = np.zeros((2, 6 * H), np.float32)
    base_old = d["adaln_scale"].base
    # keep scale/shift as drawn, replace only the gate chunk with constant rows 0 and 1
    wide_bits = base_old.copy().reshape(2, 6 * H)
    wide_bits[:, 5 * H:] = synth.to_bf16_bits(np.repeat(gates[:, None], H, 1))
    base = wide_bits.reshape(-1)
    d["adaln_shift"] = synth.Table(base, 3 * H, 2, 6 * H)
    d["adaln_scale"] = synth.Table(base, 4 * H, 2, 6 * H)
    d["gate"] = synth.Table(base, 5 * H, 2, 6 * H)
    d["adaln_index"][:] = [0, 1, 1, 0]
    o = oracle.mlp(d)
    res = bf16_val(d["residual"].reshape(M, H))
    n2 = np.arange(H)
    kk = (n2 * 11 + 5) % synth.INTER
    for m in range(M):
        oo = e4m3_val(o["y_q"][m][kk]) * float(o["y_scale"][m])        # one-hot FC2, unit scales
        ob = bf16_val(synth.to_bf16_bits(oo.astype(np.float32)))
        assert is_nearest_bf16(synth.to_bf16_bits(oo.astype(np.float32)), oo).all()
        if d["adaln_index"][m] == 0:
            assert np.array_equal(o["out"][m], d["residual"].reshape(M, H)[m])
        else:
            assert is_nearest_bf16(o["out"][m], res[m] + ob).all()


def test_mlp_fc2_stage_on_given_codes_closed_forms():
    # the FC2 + gated residual stage alone, on random codes and scales (not the oracle's own):
    # with the one-hot W2 and unit scales, o = bf16(y_q[k(n)] s_y) and out = bf16(res + bf16(g o))
    M = 4
    d = _mlp_one_hot(M)
    gates = np.array([0.0, 1.0], np.float32)
    wide_bits = d["adaln_scale"].base.copy().reshape(2, 6 * H)
    wide_bits[:, 5 * H:] = synth.to_bf16_bits(np.repeat(gates[:, None], H, 1))
    base = wide_bits.reshape(-1)
    d["gate"] = synth.Table(base, 5 * H, 2, 6 * H)
    d["adaln_index"][:] = [0, 1, -1, 1]
    g = np.random.default_rng(3)
    y_q = g.integers(0, 256, (M, synth.INTER)).astype(np.uint8)
    y_q[(y_q & 0x7F) == 0x7F] = 0x38                                   # no NaN codes
    y_s = (g.random(M) * 0.1 + 0.01).astype(np.float32)
    out = oracle.mlp_fc2(y_q, y_s, d)
    res = bf16_val(d["residual"].reshape(M, H))
    kk = (np.arange(H) * 11 + 5) % synth.INTER
    for m in range(M):
        oo = e4m3_val(y_q[m][kk]) * float(y_s[m])
        ob = bf16_val(synth.to_bf16_bits(oo.astype(np.float32)))
        if d["adaln_index"][m] != 1:                                   # gate 0, or a guarded row
            assert np.array_equal(out[m], d["residual"].reshape(M, H)[m])
        else:
            assert is_nearest_bf16(out[m], res[m] + ob).all()
    # on the full oracle's own codes it reproduces the full oracle's out
    o = oracle.mlp(d)
    assert np.array_equal(oracle.mlp_fc2(o["y_q"], o["y_scale"], d), o["out"])


# ---------------------------------------------------------------- cross-check with brute force

@pytest.mark.parametrize("M", [1, 2])
def test_brute_force_pre_attn(M):
    d = _pre(M, _random_qkv_weight(), rows=2, wide_tables=True, bad_index_frac=0.0, S=16, positions="random",
             n_bad_positions=1)
    ws, out = oracle.pre_attn(d)
    bws, bout = brute.pre_attn(d, np.arange(M))
    assert ulp_diff_bf16(ws, bws).max() <= 1 and np.mean(ws != bws) < 1e-3
    assert ulp_diff_bf16(out, bout).max() <= 1 and np.mean(out != bout) < 1e-3


def test_brute_force_out_proj():
    M = 2
    d = synth.out_proj_inputs(M, seed=9)
    d["gate_index"] = np.array([2, 10], np.int32)
    out = oracle.out_proj(d)
    bout = brute.out_proj(d, np.arange(M))
    assert ulp_diff_bf16(out, bout).max() <= 1 and np.mean(out != bout) < 1e-3


_MLP_W = {}


def _mlp_random_weights():
    if "w" not in _MLP_W:
        _MLP_W["w"] = synth.mlp_weights(13)
    return _MLP_W["w"]


@pytest.mark.parametrize("M", [1, 2])
def test_brute_force_mlp(M):
    d = synth.mlp_inputs(M, seed=14, weights=_mlp_random_weights(), bad_index_frac=0.0)
    if M == 2:
        d["adaln_index"][1] = -1
    o = oracle.mlp(d)
    b = brute.mlp(d, np.arange(M))
    for k in ("y", "out"):
        assert ulp_diff_bf16(o[k], b[k]).max() <= 1 and np.mean(o[k] != b[k]) < 1e-3, k
    for k in ("a_q", "y_q"):
        assert np.abs(ordered_e4m3(o[k]) - ordered_e4m3(b[k])).max() <= 1 and np.mean(o[k] != b[k]) < 1e-3, k
    for k in ("a_scale", "y_scale"):
        assert np.array_equal(o[k], b[k]), k


# --- Ulysses destination-major pack (bf16 pre-attention page: out [P, M, 56 // P, 3, 128]) ---

@pytest.mark.parametrize("P", [1, 2, 4, 8])
def test_ulysses_pack_index_definition(P):
    """Element by element: packed[p, m, j, kind, d] is head p * (56 // P) + j of token m."""
    g = np.random.default_rng(50 + P)
    a = g.integers(0, 1 << 16, size=(3, 56, 3, 128), dtype=np.uint16)
    packed = oracle.ulysses_pack(a, P)
    assert packed.shape == (P, 3, 56 // P, 3, 128)
    for p in range(P):
        for m in range(3):
            for j in range(56 // P):
                for kind in range(3):
                    assert np.array_equal(packed[p, m, j, kind], a[m, p * (56 // P) + j, kind])


def test_ulysses_pack_degree_one_is_identity_and_blocks_partition_heads():
    g = np.random.default_rng(60)
    a = g.integers(0, 1 << 16, size=(5, 56, 3, 128), dtype=np.uint16)
    assert np.array_equal(oracle.ulysses_pack(a, 1)[0], a)
    for P in (2, 4, 8):
        packed = oracle.ulysses_pack(a, P)
        # the destinations' head blocks, in order, are exactly the 56 heads once each
        assert np.array_equal(np.concatenate(list(packed), axis=1), a)
    with pytest.raises(ValueError):
        oracle.ulysses_pack(a, 3)


# ---------------------------------------------------------------- e4m3 output mode

def _random_out_bits(g, shape):
    """bf16 bit patterns of a packed pre-attention output, |v| spanning the e4m3 range and
    beyond (saturation), with some exact zeros of both signs."""
    v = (g.standard_normal(shape) * np.exp2(g.integers(-12, 11, size=shape))).astype(np.float32)
    v.flat[::97] = 0.0
    v.flat[1::97] = -0.0
    return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_quant_out_e4m3_matches_library_conversion_per_kind():
    # torch's float8_e4m3fn conversion (a library routine) of the fp32 quotient, after clamping
    # to the largest code; each kind sliced from the [.., 3, 128] axes with its own descale
    g = np.random.Generator(np.random.PCG64(41))
    bits = _random_out_bits(g, (2, 5, 7, 3, HD))
    descale = (np.float32(0.37), np.float32(2.5), np.float32(0.0625))
    got = oracle.quant_out_e4m3(bits, *descale)
    v = bf16_val(bits)
    for kind in range(3):
        q = (v[..., kind, :].astype(np.float32) / descale[kind]).astype(np.float32)
        ref = torch_e4m3(np.clip(q, -448.0, 448.0))
        assert np.array_equal(got[..., kind, :], ref), kind


def test_quant_out_e4m3_unit_descale_inverts_the_code_table():
    # every finite e4m3 value is a bf16 value; with descale 1 it must come back as its own code
    rows = _golden("e4m3fn_codes.txt")
    bits = np.zeros((len(rows), 3, HD), np.uint16)
    for i, (v, _) in enumerate(rows):
        bits[i] = oracle.round_bf16(v)
    got = oracle.quant_out_e4m3(bits, 1.0, 1.0, 1.0)
    for i, (v, c) in enumerate(rows):
        assert np.all(got[i] == c), (v, hex(c))


def test_quant_out_e4m3_divides_and_saturates():
    bits = np.full((1, 3, HD), oracle.round_bf16(1.0), np.uint16)
    got = oracle.quant_out_e4m3(bits, 0.5, 0.25, 2.0)          # 1/0.5, 1/0.25, 1/2
    assert np.all(got[0, 0] == 0x40) and np.all(got[0, 1] == 0x48) and np.all(got[0, 2] == 0x30)
    big = np.full((1, 3, HD), oracle.round_bf16(1000.0), np.uint16)
    assert np.all(oracle.quant_out_e4m3(big, 1.0, 1.0, 1.0) == 0x7E)
    assert np.all(oracle.quant_out_e4m3(big | 0x8000, 1.0, 1.0, 1.0) == 0xFE)
    tie = np.full((1, 3, HD), oracle.round_bf16(1.0625), np.uint16)   # midway 1 and 1.125
    assert np.all(oracle.quant_out_e4m3(tie, 1.0, 1.0, 1.0) == 0x38)  # ties to even


# ---------------------------------------------------------------- MXFP4 (OCP Microscaling)

E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def test_e2m1_values_match_the_bit_fields():
    # OCP MX v1.0, FP4 E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is
    # subnormal (m * 2^-1)
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        v = m / 2.0 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2.0)
        v = -v if s else v
        got = oracle.e2m1_value(c)
        assert got == v and math.copysign(1.0, got) == math.copysign(1.0, v), c


def test_golden_e2m1_encodings():
    for v, c in _golden("e2m1_codes.txt"):
        assert oracle.round_e2m1(v) == c, (v, hex(c), hex(oracle.round_e2m1(v)))


def test_round_e2m1_is_nearest_with_the_sign_kept():
    rng = np.random.default_rng(11)
    grid = np.array(E2M1_GRID)
    for v in np.concatenate([rng.uniform(-9, 9, 3000), rng.uniform(-1, 1, 1000)]):
        c = oracle.round_e2m1(float(v))
        got = oracle.e2m1_value(c)
        assert abs(abs(v) - abs(got)) <= np.min(np.abs(abs(v) - grid)) + 0.0
        assert math.copysign(1.0, got) == math.copysign(1.0, v)
    # monotone in v
    vs = np.linspace(-8, 8, 4001)
    vals = [oracle.e2m1_value(oracle.round_e2m1(float(v))) for v in vs]
    assert all(a <= b for a, b in zip(vals, vals[1:]))


def test_mx_scale_exp_closed_forms():
    assert oracle.mx_scale_exp(0.0) == 0
    for k in range(-125, 128, 3):
        for f in (1.0, 1.25, 1.5, 1.99609375):
            assert oracle.mx_scale_exp(f * 2.0 ** k) == k - 2 + 127, (k, f)
    assert oracle.mx_scale_exp(2.0 ** -126) == 0          # below the byte range: clamped
    assert oracle.mx_scale_exp(2.0 ** -133) == 0          # smallest bf16 subnormal
    assert oracle.mx_scale_exp(2.0 ** 200) == 254         # above it


def _mx_exact_rows(rng, R, K):
    """bf16 rows whose every 32-block is exactly representable in MXFP4 with scale 2^k: E2M1
    grid values times 2^k, one element of magnitude 4 or 6 (so floor(log2 amax) = k + 2)."""
    k = rng.integers(-8, 3, (R, K // 32))
    mag = rng.choice(np.array(E2M1_GRID), (R, K))
    sign = rng.choice([-1.0, 1.0], (R, K))
    v = mag * sign
    v[:, ::32] = rng.choice([-6.0, -4.0, 4.0, 6.0], (R, K // 32))
    v = v * np.exp2(np.repeat(k, 32, axis=1))
    return synth.to_bf16_bits(v.astype(np.float32)), k


def test_mx_quant_fp4_is_exact_on_representable_blocks():
    rng = np.random.default_rng(12)
    x, k = _mx_exact_rows(rng, 6, 512)
    codes, scales = oracle.mx_quant_fp4(x)
    assert np.array_equal(scales.astype(np.int64), k + 127)
    assert np.array_equal(oracle.mx_values(codes, scales), bf16_val(x))


def test_mx_quant_fp4_worked_block():
    # one 32-block: amax 7 -> floor(log2 7) = 2 -> E = 127 (X = 1); 7 saturates to 6, 0.3 -> 0.5,
    # -2 -> -2, 2.5 -> 2 (tie to even), -0.1 -> -0, the rest 0
    v = np.zeros(32, np.float32)
    v[:6] = [1.0, -2.0, 0.3, 7.0, 2.5, -0.1]
    codes, scales = oracle.mx_quant_fp4(synth.to_bf16_bits(v)[None, :])
    assert scales.tolist() == [[127]]
    nib = [(int(b) >> s) & 15 for b in codes[0] for s in (0, 4)]   # element 2j in the low nibble
    assert nib[:6] == [0x2, 0xC, 0x1, 0x7, 0x4, 0x8] and nib[6:] == [0] * 26
    # scaled: the same block times 2^-20 gets E = 107 and the same codes
    codes2, scales2 = oracle.mx_quant_fp4(synth.to_bf16_bits(v * np.float32(2.0 ** -20))[None, :])
    assert scales2.tolist() == [[107]] and np.array_equal(codes2, codes)


def test_mx_quant_fp4_block_properties():
    rng = np.random.default_rng(13)
    R, K = 8, 1024
    v = rng.standard_normal((R, K)) * np.exp2(rng.integers(-30, 30, (R, 1)))
    v[0, 64:96] = 0.0                                         # an all-zero block
    x = synth.to_bf16_bits(v.astype(np.float32))
    codes, scales = oracle.mx_quant_fp4(x)
    xv = bf16_val(x).reshape(R, K // 32, 32)
    q = oracle.mx_values(codes, scales).reshape(R, K // 32, 32)
    amax = np.abs(xv).max(axis=2)
    X = np.exp2(scales.astype(np.float64) - 127)
    assert scales[0, 2] == 0 and np.all(q[0, 2] == 0)
    nz = amax > 0
    assert np.all((amax[nz] / X[nz] >= 4) & (amax[nz] / X[nz] < 8))
    # every element is within half a grid step of its value (or saturated at 6 X)
    y = np.abs(xv) / X[:, :, None]
    step = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    err = np.abs(np.abs(q) / X[:, :, None] - np.minimum(y, 6.0))
    assert np.all(err <= step / 2 + 1e-12)


def _mx_d(rng, M, gate_rows=9):
    g = rng.standard_normal((gate_rows, H)).astype(np.float32)
    gate = synth.Table(synth.to_bf16_bits(g), 0, gate_rows, H)
    return {"M": M, "gate": gate,
            "gate_index": rng.integers(-1, gate_rows + 1, M).astype(np.int32),
            "residual": synth.to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32))}


def test_out_proj_mxfp4_equals_the_bf16_oracle_on_representable_inputs():
    # attn and W exactly representable in MXFP4: the W4A4 out-projection of their codes must give
    # the bf16 out-projection's result bit for bit
    rng = np.random.default_rng(14)
    M = 3
    attn, _ = _mx_exact_rows(rng, M, synth.ATTN_WIDTH)
    W, _ = _mx_exact_rows(rng, H, synth.ATTN_WIDTH)
    d = _mx_d(rng, M)
    d["gate_index"][:3] = [0, -1, 8]
    d.update(attn_out=attn, o_weight=W)
    ac, asc = oracle.mx_quant_fp4(attn)
    wc, wsc = oracle.mx_quant_fp4(W)
    got = oracle.out_proj_mxfp4(ac, asc, wc, wsc, d)
    assert np.array_equal(got, oracle.out_proj(d))


def test_out_proj_mxfp4_matches_float64_matmul_of_the_values():
    # gate 1 and residual 0: out = bf16(o) = bf16(A . W), A and W the MXFP4 values
    rng = np.random.default_rng(15)
    M = 2
    a = rng.integers(0, 256, (M, synth.ATTN_WIDTH // 2)).astype(np.uint8)
    a_s = rng.integers(118, 130, (M, synth.ATTN_WIDTH // 32)).astype(np.uint8)
    w = rng.integers(0, 256, (H, synth.ATTN_WIDTH // 2)).astype(np.uint8)
    w_s = rng.integers(118, 130, (H, synth.ATTN_WIDTH // 32)).astype(np.uint8)
    d = {"M": M, "gate": synth.Table(synth.to_bf16_bits(np.ones((1, H), np.float32)), 0, 1, H),
         "gate_index": np.zeros(M, np.int32), "residual": np.zeros((M, H), np.uint16)}
    got = oracle.out_proj_mxfp4(a, a_s, w, w_s, d)
    A = torch.from_numpy(oracle.mx_values(a, a_s))
    Wv = torch.from_numpy(oracle.mx_values(w, w_s))
    want = (A @ Wv.T).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_brute_force_mx_quant_matches_the_oracle():
    # an independent NumPy reading of the MXFP4 conversion, bit for bit
    x = _mx_exact_rows(np.random.default_rng(16), 3, 512)[0]
    rng = np.random.default_rng(17)
    y = synth.to_bf16_bits((rng.standard_normal((5, 1024)) * np.exp2(rng.integers(-20, 20, (5, 1)))).astype(np.float32))
    y[0, 96:128] = synth.to_bf16_bits(np.float32(-0.0))
    for v in (x, y, synth.to_bf16_bits(np.resize(np.float32([0.25, -0.75, 5.0, 4.0, 7.5, 1.25]), (1, 256)))):
        c, s = oracle.mx_quant_fp4(v)
        bc, bs = brute.mx_quant(v)
        assert np.array_equal(c, bc) and np.array_equal(s, bs)


@pytest.mark.parametrize("M", [1, 2])
def test_brute_force_pre_attn_mxfp4(M):
    d = _pre(M, _random_qkv_weight(), rows=2, wide_tables=True, bad_index_frac=0.0, S=16, positions="random",
             n_bad_positions=1)
    wc, wsc = oracle.mx_quant_fp4(d["qkv_weight"])
    ws, c, s, out = oracle.pre_attn_mxfp4(d, wc, wsc)
    assert np.array_equal(ws, oracle.pre_attn(d)[0])             # the same workspace a
    bout = brute.qkv_mxfp4(d, np.arange(M), c, s, wc, wsc)
    assert ulp_diff_bf16(out, bout).max() <= 1 and np.mean(out != bout) < 1e-3
