"""The GPU parity bars must reject plausible mistakes.  Each test plants a mistake in the
oracle's inputs or outputs, on the CPU, and checks that the bar the GPU tests use fails on it,
while the oracle against itself passes."""
from __future__ import annotations

import numpy as np

import oracle
import synth
from tests.helpers import bf16_val, e4m3_half_step, gated_tolerance_ok, qkv_check, rope_elem_bound, ulp_bf16

M = 3


def _d(seed=31, **kw):
    return synth.pre_attn_inputs(M, seed=seed, rows=2, S=16, positions="random", n_bad_positions=0,
                                 bad_index_frac=0.0, **kw)


def _cs(d):
    return d["rope_cos_sin"].reshape(-1, 96)[np.clip(d["rope_positions"], 0, d["S"] - 1)]


_REF = {}


def _ref():
    if "r" not in _REF:
        d = _d()
        _REF["r"] = (d, oracle.pre_attn(d)[1])
    return _REF["r"]


def test_qkv_bar_accepts_the_oracle_itself():
    d, out = _ref()
    ok, rel, mx, n_rel, worst = qkv_check(out, out, _cs(d), max_relaxed=0)
    assert ok and rel == 0.0 and n_rel == 0


def test_qkv_bar_rejects_a_rope_sign_error():
    d, out = _ref()
    bad = dict(d)
    cs = bf16_val(d["rope_cos_sin"]).copy()
    cs[:, 48:] *= -1.0                      # o_j = u c + w s instead of u c - w s
    bad["rope_cos_sin"] = synth.to_bf16_bits(cs.astype(np.float32))
    _, wrong = oracle.pre_attn(bad)
    assert not qkv_check(wrong, out, _cs(d), max_relaxed=4)[0]


def test_qkv_bar_rejects_a_shifted_frequency():
    d, out = _ref()
    bad = dict(d)
    cs = d["rope_cos_sin"].reshape(-1, 96).copy()
    cs[:, :48] = np.roll(cs[:, :48], 1, axis=1)
    cs[:, 48:] = np.roll(cs[:, 48:], 1, axis=1)
    bad["rope_cos_sin"] = cs
    _, wrong = oracle.pre_attn(bad)
    assert not qkv_check(wrong, out, _cs(d), max_relaxed=4)[0]


def test_qkv_bar_rejects_a_wrong_position():
    d, out = _ref()
    bad = dict(d, rope_positions=(d["rope_positions"] + 1) % d["S"])
    _, wrong = oracle.pre_attn(bad)
    assert not qkv_check(wrong, out, _cs(d), max_relaxed=4)[0]


def test_qkv_bar_rejects_a_dropped_qk_norm_weight():
    d, out = _ref()
    bad = dict(d, q_norm_weight=np.full(128, 0x3F80, np.uint16))
    _, wrong = oracle.pre_attn(bad)
    assert not qkv_check(wrong, out, _cs(d), max_relaxed=4)[0]


def test_rope_bound_is_a_few_ulps_of_u():
    # the derived bound must stay at the scale of a few bf16 ulps of the pair, far below the
    # plain 1e-2 (1 + |o|) bar's absolute term for unit-scale heads
    d, out = _ref()
    b = rope_elem_bound(out, _cs(d))[:, :, :2, :96]
    o = bf16_val(out)[:, :, :2, :96]
    pair = np.hypot(o[..., :48], o[..., 48:])
    pair = np.concatenate([pair, pair], axis=-1)
    assert np.all(b <= 8.0 * ulp_bf16(pair * 1.02) + ulp_bf16(o) + 1e-30)
    assert np.all(np.isinf(rope_elem_bound(out, _cs(d))[:, :, 2]))


def test_rope_bound_covers_a_one_ulp_flip_of_v():
    # move one v element of a q head by one bf16 ulp through a one-hot workspace probe: with
    # cos = 1 and sin = 0 the output is u, and flipping the bf16 input of a pair member moves
    # the rotated outputs by no more than the bound
    d, out = _ref()
    W = d["qkv_weight"].copy()
    rng = np.random.default_rng(5)
    rows = rng.choice(2 * 7168, 64, replace=False)
    W[rows] = np.where(W[rows] & 0x7FFF, W[rows] + 1, W[rows]).astype(np.uint16)   # one ulp per weight
    _, moved = oracle.pre_attn(dict(d, qkv_weight=W))
    g, r = bf16_val(moved), bf16_val(out)
    err = np.abs(g - r)
    plain = err <= 1e-2 * (1 + np.abs(r))
    assert np.all(plain | (err <= rope_elem_bound(out, _cs(d))))


def test_e4m3_half_step():
    s = np.float64(0.5)
    # codes at 1.0 * s are spaced 2^-3 s apart, subnormal codes 2^-9 s
    assert e4m3_half_step(np.array([0.5, 0.75, 2.0 ** -8]), s).tolist() == [2.0 ** -5, 2.0 ** -5, 2.0 ** -11]


def _gated(seed=5, n=4000):
    g = np.random.default_rng(seed)
    res = synth.to_bf16_bits(g.standard_normal(n).astype(np.float32))
    gate = bf16_val(synth.to_bf16_bits((g.standard_normal(n) * 0.5).astype(np.float32)))
    o = bf16_val(synth.to_bf16_bits(g.standard_normal(n).astype(np.float32)))
    go = bf16_val(synth.to_bf16_bits((gate * o).astype(np.float32)))
    ref = synth.to_bf16_bits((bf16_val(res) + go).astype(np.float32))
    return res, gate, o, go, ref


def test_gated_bar_accepts_the_reference_itself():
    res, gate, _, _, ref = _gated()
    ok, rel, mx, n_far, _ = gated_tolerance_ok(ref, ref, res, gate)
    assert ok and rel == 0.0 and n_far == 0


def _cancelling(k):
    """_gated()'s elements with the first k made cancelling: g = 1, bf16(g o) = 3 and res = -3 +
    1/16, so out = 1/16; got takes bf16(g o) one bf16 ulp up (o one ulp off), which moves out by
    2^-6: far past 1e-2 (1 + |out|), within the carried bound."""
    res, gate, _, go, _ = _gated()
    res, gate, go = bf16_val(res).copy(), gate.copy(), go.copy()
    gate[:k], go[:k], res[:k] = 1.0, 3.0, -3.0 + 0.0625
    res_b = synth.to_bf16_bits(res.astype(np.float32))
    ref = synth.to_bf16_bits((bf16_val(res_b) + go).astype(np.float32))
    go_up = go.copy()
    go_up[:k] += 2.0 ** -6
    got = synth.to_bf16_bits((bf16_val(res_b) + go_up).astype(np.float32))
    return got, ref, res_b, gate


def test_gated_bar_covers_a_cancelling_residual():
    got, ref, res, gate = _cancelling(1)
    err = abs(bf16_val(got)[0] - bf16_val(ref)[0])
    assert err > 1e-2 * (1 + abs(bf16_val(ref)[0]))
    ok, _, _, n_far, worst = gated_tolerance_ok(got, ref, res, gate)
    assert ok and n_far == 1 and worst <= 1.0


def test_gated_bar_rejects_a_dropped_gate():
    res, gate, o, _, ref = _gated()
    wrong = synth.to_bf16_bits((bf16_val(res) + o).astype(np.float32))
    assert not gated_tolerance_ok(wrong, ref, res, gate)[0]


def test_gated_bar_rejects_another_rows_residual():
    res, gate, _, go, ref = _gated()
    wrong = synth.to_bf16_bits((np.roll(bf16_val(res), 1) + go).astype(np.float32))
    assert not gated_tolerance_ok(wrong, ref, res, gate)[0]


def test_gated_bar_caps_the_elements_past_the_plain_bar():
    # 4000 elements allow 4 + 0.04 past the plain bar
    assert gated_tolerance_ok(*_cancelling(4))[0]
    assert not gated_tolerance_ok(*_cancelling(5))[0]
