"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded
inputs.

Bars (bf16 pre-attention, out-projection and fp8 MLP):
  - the AdaLN workspace within 1 bf16 ulp at each rounding point of a = bf16(shift + n*s1):
    |a_gpu - a_ref| <= ulp(a_ref) + 2 ulp(a_ref - shift), at most 1e-4 of elements differing
    (n's own rounding may land on the other neighbour; shift can cancel n*s1);
  - every bf16 output: relative L2 error <= 2e-3 and |err| <= 1e-2 * (1 + |ref|) per element.
    A gated-residual output (out-projection, MLP) whose residual cancels the gated term may
    instead meet that bar carried from o, helpers.gated_tolerance_ok, for at most 4 + 1e-5 of
    the elements.  The MLP's out must meet these bars everywhere against the oracle's FC2 stage
    fed the GPU's own y_q and s_y; against the full oracle, elements outside them may only lie in
    rows whose s_y is not the oracle's (the whole row of y requantised).
    A RoPE-rotated q/k element may instead meet the derived bound of
    helpers.rope_elem_bound (an FP32-accumulated v may round to the other bf16 neighbour, and
    the rotation can carry that ulp of a large u into a small output), but at most
    4 + 4e-6 of the rotated elements may need it;
  - e4m3 activation codes within one code step and per-token activation scales within 1 bf16
    ulp of the oracle's; where the AdaLN shift cancels n*s1, a code may instead lie within the
    workspace bar carried through the division (that distance over s_a plus both half code
    steps), for at most 4 + 1e-5 of the codes;
  - the bf16 intermediate y: the same 1e-2 * (1 + |ref|) bar, relaxed to 4 ulp(ref) for at most
    1e-4 of its elements (y is three roundings past an FP32-accumulated GEMM);
  - the y quantisation: s_y == RN(amax|y_gpu|/448) and y_q == e4m3(y_gpu/s_y) on the GPU's own
    y; against the oracle, s_y bit-equal on every row whose amax|y| equals the oracle's and
    within |amax_gpu - amax_ref| / 448 (plus one fp32 ulp) elsewhere, and y_q bit-equal
    wherever y and s_y agree bit for bit, within |y_gpu - y_ref| plus both half code steps in
    value elsewhere (near zero a code step of y/s_y is 2^-9 s_y, far below the GEMM's
    accumulation error in y, so a code-step count is no bar there);
  - rows with a guarded index: workspace/codes exactly zero, outputs zero (pre-attention) or
    equal to the residual (out-projection, MLP).
At the full workload sizes the oracle runs on a sampled row set (rows are independent, so
this is exact parity on those rows): the first 256 rows, the whole last 256-row tile, every
guarded row, every clamped-position row and 512 seeded random rows.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import (bf16_val, gated_outside, gated_tolerance_ok, e4m3_half_step, e4m3_val, ordered_e4m3, qkv_check,
                           torch_e4m3, ulp_bf16, ulp_diff_bf16, workspace_ok)

pytestmark = pytest.mark.gpu

H = synth.HIDDEN
INT64_MIN, INT64_MAX = -(1 << 63), (1 << 63) - 1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import diffusion_transformer_adaln_rmsnorm_amd as dit
    dit.load_library()


def _say(msg):
    print(f"[parity] {msg}", file=sys.stderr, flush=True)


def _dit():
    import diffusion_transformer_adaln_rmsnorm_amd as dit
    return dit


def sample_rows(M, d=None, n_random=512, seed=0):
    rows = set(range(min(M, 256)))
    rows |= set(range(((M - 1) // 256) * 256, M))
    if d is not None:
        idx = d.get("adaln_index")
        if idx is not None:
            rows |= set(np.nonzero((idx < 0) | (idx >= d.get("rows", 1 << 62)))[0].tolist())
        gi = d.get("gate_index")
        if gi is not None:
            rows |= set(np.nonzero((gi < 0) | (gi >= d["gate"].rows))[0][:128].tolist())
        pos = d.get("rope_positions")
        if pos is not None:
            rows |= set(np.nonzero((pos < 0) | (pos >= d["S"]))[0].tolist())
    g = np.random.Generator(np.random.PCG64(seed))
    rows |= set(g.choice(M, size=min(n_random, M), replace=False).tolist())
    return np.array(sorted(rows), np.int64)


# ---------------------------------------------------------------- runners

def run_pre(d, out=None, workspace=None, P=1):
    t = synth.to_torch("pre_attn", d)
    M = d["M"]
    if out is None:
        out = torch.empty((P, M, 56 // P, 3, 128), dtype=torch.bfloat16, device="cuda")
    _dit().dit_pre_attn_bf16(t["x"], t["x_norm_weight"], t["adaln_scale"], t["adaln_shift"], t["adaln_index"],
                             t["qkv_weight"], t["q_norm_weight"], t["k_norm_weight"], t["rope_cos_sin"],
                             ulysses_degree=P, out=out, eps=t["eps"], qk_eps=t["qk_eps"],
                             rope_positions=t["rope_positions"], workspace=workspace)
    torch.cuda.synchronize()
    return t, out


def run_pre_e4m3(d, descale, P=1):
    t = synth.to_torch("pre_attn", d)
    M = d["M"]
    out = torch.empty((P, M, 56 // P, 3, 128), dtype=torch.uint8, device="cuda")
    _dit().dit_pre_attn_e4m3(t["x"], t["x_norm_weight"], t["adaln_scale"], t["adaln_shift"], t["adaln_index"],
                             t["qkv_weight"], t["q_norm_weight"], t["k_norm_weight"], t["rope_cos_sin"],
                             ulysses_degree=P, out=out, q_descale=descale[0], k_descale=descale[1],
                             v_descale=descale[2], eps=t["eps"], qk_eps=t["qk_eps"],
                             rope_positions=t["rope_positions"])
    torch.cuda.synchronize()
    return out.cpu().numpy()


def e4m3_of_bf16(bits, descale):
    """e4m3(fl32(v / descale_kind)) of bf16 bit patterns [..., 3, 128], saturating, by torch's
    float8_e4m3fn conversion (a library routine)."""
    v = bf16_val(bits).astype(np.float32)
    out = np.empty(bits.shape, np.uint8)
    for kind in range(3):
        q = (v[..., kind, :] / np.float32(descale[kind])).astype(np.float32)
        out[..., kind, :] = torch_e4m3(np.clip(q, -448.0, 448.0))
    return out


def row_cos_sin(d, rows):
    """Each selected row's [96] cos/sin cache row: position clamp(pos[m], 0, S-1), or m."""
    pos = d.get("rope_positions")
    p = rows if pos is None else np.clip(pos[rows], 0, d["S"] - 1)
    return d["rope_cos_sin"].reshape(-1, 96)[p]


def max_relaxed_qk(n_rows):
    """Ceiling on the rotated q/k elements allowed past the plain bar (4 + 4e-6 of them)."""
    return 4 + int(4e-6 * n_rows * 56 * 2 * 96)


def check_qkv(got, ref, cs_rows, label):
    ok, rel, mx, n_rel, worst = qkv_check(got, ref, cs_rows, max_relaxed=max_relaxed_qk(got.shape[0]))
    _say(f"  {label}: relL2={rel:.2e} max|err|={mx:.3e} past the plain bar={n_rel} "
         f"(ceiling {max_relaxed_qk(got.shape[0])}, worst err/derived bound {worst:.2f})")
    assert ok, (label, rel, mx, n_rel, worst)
    return rel, mx, n_rel


def check_pre(d, ws_gpu, out_gpu, rows=None, max_mismatch=1e-4):
    M = d["M"]
    rows = np.arange(M) if rows is None else rows
    ws_ref, out_ref = oracle.pre_attn(d, rows_sel=rows)
    ws = synth.bits(ws_gpu)[rows]
    out = synth.bits(out_gpu).reshape(M, 56, 3, 128)[rows]
    idx = d["adaln_index"][rows]
    bad = (idx < 0) | (idx >= d["adaln_scale"].rows)
    shift = bf16_val(d["adaln_shift"].dense())[np.where(bad, 0, idx)]
    wok, wmis, wratio = workspace_ok(ws[~bad], ws_ref[~bad], shift[~bad], max_mismatch=max_mismatch)
    du = ulp_diff_bf16(ws, ws_ref)
    _say(f"pre_attn M={M} rows={rows.size} ws max ulp={du.max()} ws mismatch={wmis:.2e} (err/bound {wratio:.2f}) "
         f"guarded={bad.sum()} v mismatch={np.mean(out[:, :, 2] != out_ref[:, :, 2]):.2e}")
    assert wok, f"workspace: mismatch {wmis:.2e}, worst err/bound {wratio:.2f}"
    assert np.all(ws[bad] == 0), "guarded workspace rows must be +0"
    assert np.all(bf16_val(out[bad]) == 0.0), "guarded output rows must be zero"
    check_qkv(out, out_ref, row_cos_sin(d, rows), f"pre_attn M={M} out")
    return ws, out


def run_out_proj(d, alias=False):
    t = synth.to_torch("out_proj", d)
    out = t["residual"] if alias else None
    out = _dit().dit_out_proj_gated_bf16(t["attn_out"], t["o_weight"], t["gate"], t["gate_index"], t["residual"],
                                         out=out)
    torch.cuda.synchronize()
    return out


def check_out_proj(d, out_gpu, rows=None):
    M = d["M"]
    rows = np.arange(M) if rows is None else rows
    ref = oracle.out_proj(d, rows_sel=rows)
    got = synth.bits(out_gpu)[rows]
    gi = d["gate_index"][rows]
    bad = (gi < 0) | (gi >= d["gate"].rows)
    assert np.array_equal(got[bad], d["residual"].reshape(M, H)[rows][bad]), "guarded rows must equal residual"
    res = d["residual"].reshape(M, H)[rows]
    g = np.where(bad[:, None], 0.0, bf16_val(d["gate"].dense())[np.where(bad, 0, gi)])
    ok, rel, mx, n_far, worst = gated_tolerance_ok(got, ref, res, g)
    _say(f"out_proj M={M} rows={rows.size} relL2={rel:.2e} max|err|={mx:.3e} mismatch={np.mean(got != ref):.2e} "
         f"past the plain bar={n_far} (worst {worst:.2f} of the carried bound)")
    assert ok, (rel, mx, n_far, worst)


def run_mlp(d, alias=None):
    t = synth.to_torch("mlp", d)
    M = d["M"]
    ws = {"workspace_a_q": torch.empty((M, H), dtype=torch.float8_e4m3fn, device="cuda"),
          "workspace_a_scale": torch.empty((M,), dtype=torch.float32, device="cuda"),
          "workspace_y": torch.empty((M, synth.INTER), dtype=torch.bfloat16, device="cuda"),
          "workspace_y_q": torch.empty((M, synth.INTER), dtype=torch.float8_e4m3fn, device="cuda"),
          "workspace_y_scale": torch.empty((M,), dtype=torch.float32, device="cuda")}
    out = None if alias is None else t[alias]
    out = _dit().dit_mlp_fp8(t["x"], t["x_norm_weight"], t["adaln_scale"], t["adaln_shift"], t["adaln_index"],
                             t["gate"], t["residual"], t["fc1_weight_q"], t["fc1_weight_scale"], t["fc2_weight_q"],
                             t["fc2_weight_scale"], out=out, eps=t["eps"], **ws)
    torch.cuda.synchronize()
    return out, ws


def check_y_quant(y, y_q, y_s, ref, label):
    """The y quantisation against the GPU's own y and against the oracle (see the module
    docstring).  y, y_q, y_s: the GPU's y bits, codes and scales of the checked rows."""
    yg, yr = bf16_val(y), bf16_val(ref["y"])
    s_r = ref["y_scale"].astype(np.float32)
    # on the GPU's own y: s_y = RN(amax/448) exactly, and every code is e4m3(y/s_y)
    amax_g = np.max(np.abs(yg), axis=1)
    amax_r = np.max(np.abs(yr), axis=1)
    assert np.array_equal(y_s, (amax_g.astype(np.float32) / np.float32(448.0)).astype(np.float32)), \
        "s_y != RN(amax|y|/448)"
    nz = y_s > 0
    q_lib = np.zeros_like(y_q)
    q_lib[nz] = torch_e4m3((yg[nz].astype(np.float32) / y_s[nz, None]).astype(np.float32))
    assert np.array_equal(y_q, q_lib), "y_q != e4m3(y/s_y) on the GPU's own y"
    # against the oracle: s_y
    same_amax = amax_g == amax_r
    assert np.array_equal(y_s[same_amax], s_r[same_amax]), "s_y differs on a row whose amax|y| is the oracle's"
    lip = np.abs(amax_g - amax_r) / 448.0 * (1 + 2.0 ** -22) + np.spacing(s_r).astype(np.float64)
    assert np.all(np.abs(y_s.astype(np.float64) - s_r) <= lip), "s_y beyond |d amax| / 448"
    s_ulps = np.abs(y_s.astype(np.float64) - s_r) / ulp_bf16(np.maximum(s_r, 2.0 ** -126))
    # y_q: bit-equal where y and s_y are; in value space elsewhere
    same = (y == ref["y"]) & (y_s == s_r)[:, None]
    assert np.array_equal(y_q[same], ref["y_q"][same]), "y_q differs where y and s_y equal the oracle's"
    vg = e4m3_val(y_q) * y_s[:, None].astype(np.float64)
    vr = e4m3_val(ref["y_q"]) * s_r[:, None].astype(np.float64)
    bound = np.abs(yg - yr) + e4m3_half_step(yg, y_s[:, None].astype(np.float64)) + \
        e4m3_half_step(yr, s_r[:, None].astype(np.float64))
    assert np.all(np.abs(vg - vr) <= bound * (1 + 1e-9)), "y_q beyond |dy| + half code steps"
    step = np.abs(ordered_e4m3(y_q) - ordered_e4m3(ref["y_q"]))
    _say(f"  {label} y_q: mismatch={np.mean(y_q != ref['y_q']):.2e} beyond one step={np.mean(step > 1):.2e} "
         f"(max step {step.max()}); s_y: rows equal={np.mean(y_s == s_r):.3f}, max off {s_ulps.max():.2f} bf16 ulp")


def check_mlp(d, out_gpu, ws, rows=None):
    M = d["M"]
    rows = np.arange(M) if rows is None else rows
    ref = oracle.mlp(d, rows_sel=rows)
    a_q = synth.bits(ws["workspace_a_q"])[rows]
    a_s = ws["workspace_a_scale"].cpu().numpy()[rows]
    y = synth.bits(ws["workspace_y"])[rows]
    y_q = synth.bits(ws["workspace_y_q"])[rows]
    y_s = ws["workspace_y_scale"].cpu().numpy()[rows]
    out = synth.bits(out_gpu)[rows]
    assert np.all(np.abs(a_s.astype(np.float64) - ref["a_scale"]) <= ulp_bf16(np.maximum(ref["a_scale"], 2.0 ** -126))), \
        "a_scale beyond 1 bf16 ulp"
    # a_q: one code step, except where the AdaLN shift cancels n*s1.  There the GPU's a may sit
    # the workspace bar's ulp(a) + 2 ulp(a - shift) from the oracle's a (n one bf16 ulp off, from
    # the FP32 sum of squares), which a / s_a carries into many code steps of a small quotient;
    # such codes must lie within that distance plus both half code steps in value.
    da = np.abs(ordered_e4m3(a_q) - ordered_e4m3(ref["a_q"]))
    idx = d["adaln_index"][rows]
    bad = (idx < 0) | (idx >= d["adaln_scale"].rows)
    if np.any(da > 1):
        dn = {k: d[k] for k in ("M", "x", "x_norm_weight", "adaln_scale", "adaln_shift", "adaln_index", "eps")}
        a_r = bf16_val(oracle.norm_adaln(dn, rows_sel=rows))
        shift = bf16_val(d["adaln_shift"].dense())[np.where(bad, 0, idx)]
        s = a_s[:, None].astype(np.float64)
        bound_a = ulp_bf16(a_r) + 2.0 * ulp_bf16(a_r - shift)
        bound = bound_a + e4m3_half_step(np.abs(a_r) + bound_a, s) + e4m3_half_step(a_r, s)
        dv = np.abs(e4m3_val(a_q) - e4m3_val(ref["a_q"])) * s
        far = da > 1
        assert np.all(dv[far] <= bound[far] * (1 + 1e-9)), "a_q beyond the carried workspace bar"
        assert far.sum() <= 4 + 1e-5 * da.size, f"{far.sum()} a_q codes beyond one step"
        _say(f"  a_q: {far.sum()} codes beyond one step (max {da.max()}), all within the carried workspace bar "
             f"(worst {float((dv[far] / bound[far]).max()):.2f} of it)")
    # y: 1e-2 (1 + |ref|), or 4 ulp(ref) for at most 1e-4 of the elements
    yg, yr = bf16_val(y), bf16_val(ref["y"])
    erry = np.abs(yg - yr)
    rely = np.linalg.norm(yg - yr) / max(np.linalg.norm(yr), 1e-30)
    plain = erry <= 1e-2 * (1.0 + np.abs(yr))
    n_relaxed = int(np.sum(~plain))
    assert rely <= 2e-3 and np.all(plain | (erry <= 4.0 * ulp_bf16(yr))), ("y", rely, float(erry.max()))
    assert n_relaxed <= 4 + 1e-4 * erry.size, f"{n_relaxed} y elements past the plain bar"
    check_y_quant(y, y_q, y_s, ref, f"mlp M={M}")
    assert np.all(a_q[bad] == 0) and np.all(a_s[bad] == 0) and np.all(y_s[bad] == 0)
    res = d["residual"].reshape(M, H)[rows]
    assert np.array_equal(out[bad], res[bad]), "guarded rows must equal the residual"
    g = np.where(bad[:, None], 0.0, bf16_val(d["gate"].dense())[np.where(bad, 0, idx)])
    # out against the FC2 stage of the oracle fed the GPU's own y_q and s_y: the plain bar (or
    # the carried one where the residual cancels), everywhere
    stage = oracle.mlp_fc2(y_q, y_s, d, rows_sel=rows)
    ok_s, rel_s, mx_s, n_far_s, worst_s = gated_tolerance_ok(out, stage, res, g)
    assert ok_s, ("out against the FC2 stage on the GPU's own y_q", rel_s, mx_s, n_far_s, worst_s)
    # against the full oracle: relative L2, and the same bars except in rows whose s_y is not the
    # oracle's (an amax one ulp off requantises the whole row of y, which moves o by more than its
    # plain bar; the stage check above covers those rows), at most 4 + 1e-5 of the elements
    ok, rel, mx, n_far, worst = gated_tolerance_ok(out, ref["out"], res, g)
    outside = gated_outside(out, ref["out"], res, g)
    requant = (y_s != ref["y_scale"])[:, None]
    assert rel <= 2e-3, ("out relL2", rel)
    assert not np.any(outside & ~requant), "out outside the bar in a row whose s_y is the oracle's"
    assert n_far <= 4 + 1e-5 * out.size, f"{n_far} out elements past the plain bar"
    _say(f"mlp M={M} rows={rows.size} a_q mismatch={np.mean(a_q != ref['a_q']):.2e} "
         f"a_s exact={np.mean(a_s == ref['a_scale']):.3f} y relL2={rely:.2e} y max|err|={erry.max():.3e} "
         f"y past plain bar={n_relaxed} out relL2={rel:.2e} max|err|={mx:.3e} out past the plain bar={n_far} "
         f"({int(outside.sum())} outside the carried bound, all in rows with a requantised y; against the FC2 "
         f"stage on the GPU's y_q: relL2={rel_s:.2e}, past the plain bar {n_far_s}) guarded={bad.sum()}")
    return ref


# ---------------------------------------------------------------- pre-attention

def test_pre_attn_config0_full():
    _say("config 0: pre_attn M=16 (rows=4 tables, guard -1 and 4)")
    kind, d = synth.config(0)
    ws = torch.empty((16, H), dtype=torch.bfloat16, device="cuda")
    t, out = run_pre(d, workspace=ws)
    check_pre(d, ws, out)


@pytest.mark.parametrize("M", [1, 2, 3, 16, 17, 255, 256, 257])
def test_pre_attn_small_M_random_positions(M):
    _say(f"pre_attn small M={M}, random positions with clamps, rows=2 wide tables")
    d = synth.pre_attn_inputs(M, seed=100 + M, rows=2, S=64, positions="random", n_bad_positions=min(8, M),
                              bad_index_frac=0.05, weight=_shared_weight())
    ws = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    _, out = run_pre(d, workspace=ws)
    check_pre(d, ws, out)


def test_every_entry_point_treats_M_zero_as_a_no_op():
    """M = 0 (zero-row views whose data pointers are those of real buffers): every entry point
    returns without an error and writes nothing -- the buffers behind the views keep their
    sentinel bytes.  The fp8 MLP's range starts at M = 1 (its page's limits) and is refused."""
    dit = _dit()
    _say("M = 0 through every entry point")
    d = synth.pre_attn_inputs(2, seed=5, rows=2, S=4, positions="random", n_bad_positions=0,
                              weight=_shared_weight())
    t = synth.to_torch("pre_attn", d)
    z = lambda a: a[:0]   # noqa: E731
    sent = lambda shape, dt: torch.full(shape, 0x5A, dtype=torch.uint8, device="cuda").view(dt)  # noqa: E731
    out_b = sent((1, 2, 56, 3, 256), torch.uint8)            # room for two bf16 rows
    out_bf = out_b.view(torch.bfloat16)[:, :0]
    out_e = sent((1, 2, 56, 3, 128), torch.uint8)
    ws = sent((2, H * 2), torch.uint8)
    ws_bf = ws.view(torch.bfloat16)[:0]
    before = [b.clone() for b in (out_b, out_e, ws)]
    common = (z(t["x"]), t["x_norm_weight"], t["adaln_scale"], t["adaln_shift"], z(t["adaln_index"]))
    rope = dict(rope_positions=z(t["rope_positions"]), qk_eps=t["qk_eps"])
    dit.dit_pre_attn_bf16(*common, t["qkv_weight"], t["q_norm_weight"], t["k_norm_weight"], t["rope_cos_sin"],
                          ulysses_degree=1, out=out_bf, eps=t["eps"], workspace=ws_bf, **rope)
    dit.dit_pre_attn_bf16_static_ws(*common, t["qkv_weight"], t["q_norm_weight"], t["k_norm_weight"],
                                    t["rope_cos_sin"], ulysses_degree=2, out=out_b.view(torch.bfloat16)[:, :0]
                                    .reshape(2, 0, 28, 3, 128), eps=t["eps"], **rope)
    dit.dit_pre_attn_e4m3(*common, t["qkv_weight"], t["q_norm_weight"], t["k_norm_weight"], t["rope_cos_sin"],
                          ulysses_degree=1, out=out_e[:, :0], q_descale=1.0, k_descale=1.0, v_descale=1.0,
                          eps=t["eps"], workspace=ws_bf, **rope)
    dit.dit_norm_adaln_bf16(*common, workspace=ws_bf, eps=t["eps"])
    dit.dit_qkv_rope_pack_bf16(ws_bf, t["qkv_weight"], t["q_norm_weight"], t["k_norm_weight"], t["rope_cos_sin"],
                               ulysses_degree=4, out=out_bf.reshape(4, 0, 14, 3, 128), **rope)
    dit.dit_qkv_rope_pack_e4m3(ws_bf, t["qkv_weight"], t["q_norm_weight"], t["k_norm_weight"], t["rope_cos_sin"],
                               ulysses_degree=1, out=out_e[:, :0], q_descale=1.0, k_descale=1.0, v_descale=1.0,
                               **rope)
    wq = torch.zeros((synth.QKV_ROWS, H // 2), dtype=torch.uint8, device="cuda")
    wqs = torch.zeros((dit.dit_mx_scale_bytes(synth.QKV_ROWS, H),), dtype=torch.uint8, device="cuda")
    mx_sc = sent((1024,), torch.uint8)
    before.append(mx_sc.clone())
    dit.dit_pre_attn_mxfp4(*common, wq, wqs, t["q_norm_weight"], t["k_norm_weight"], t["rope_cos_sin"],
                           ulysses_degree=1, out=out_bf, eps=t["eps"], ws_codes=ws[:0, : H // 2],
                           ws_scales=mx_sc[:0], **rope)
    # out-projections and the quantiser
    to = synth.to_torch("out_proj", synth.out_proj_inputs(2, seed=6))
    res = sent((2, H * 2), torch.uint8)
    res_bf = res.view(torch.bfloat16)[:0]
    ac = sent((2, synth.ATTN_WIDTH // 2), torch.uint8)
    before += [res.clone(), ac.clone()]
    dit.dit_out_proj_gated_bf16(z(to["attn_out"]), to["o_weight"], to["gate"], z(to["gate_index"]), res_bf,
                                out=res_bf)
    wo = torch.zeros((H, synth.ATTN_WIDTH // 2), dtype=torch.uint8, device="cuda")
    wos = torch.zeros((dit.dit_mx_scale_bytes(H, synth.ATTN_WIDTH),), dtype=torch.uint8, device="cuda")
    dit.dit_out_proj_gated_mxfp4(z(to["attn_out"]), wo, wos, to["gate"], z(to["gate_index"]), res_bf, out=res_bf,
                                 act_codes=ac[:0], act_scales=mx_sc[:0])
    dit.dit_mx_quant_fp4(z(to["attn_out"]), codes=ac[:0], scales=mx_sc[:0])
    torch.cuda.synchronize()
    for b0, b1 in zip(before, [out_b, out_e, ws, mx_sc, res, ac]):
        assert torch.equal(b0, b1), "an M = 0 call wrote to its buffers"
    with pytest.raises(dit.DitError) as err:
        dit.dit_mlp_fp8(z(t["x"]), t["x_norm_weight"], t["adaln_scale"], t["adaln_shift"], z(t["adaln_index"]),
                        t["adaln_scale"], z(t["x"]),
                        torch.zeros((synth.FC1_ROWS, H), dtype=torch.float8_e4m3fn, device="cuda"),
                        torch.ones((synth.FC1_ROWS,), dtype=torch.float32, device="cuda"),
                        torch.zeros((H, synth.INTER), dtype=torch.float8_e4m3fn, device="cuda"),
                        torch.ones((H,), dtype=torch.float32, device="cuda"))
    assert err.value.status == 2, err.value.status          # DIT_ERR_SHAPE: M below the range


def test_large_M_tiles_equal_their_repeated_4096_row_block():
    """Byte offsets far past 2^32: the pre-attention at M = 2^20 (out 45 GB) and the
    out-projection at M = 2^19 (out 5.6 GB), with inputs built by repeating a 4096-row block.
    Every 256-row tile then holds the same rows as a tile of the M = 4096 run, so sampled
    tiles (the first, those holding the 2^32- and 2^33-byte offsets of out, one in the middle
    and the last) must equal that run bit for bit; the M = 4096 runs themselves are held to the
    oracle (configs 1 and 3 tests)."""
    B = 4096
    d = synth.pre_attn_inputs(B, seed=21, rows=2, S=B, positions="random", weight=_shared_weight())
    t = synth.to_torch("pre_attn", d)
    ws0 = torch.empty((B, H), dtype=torch.bfloat16, device="cuda")
    out0 = torch.empty((1, B, 56, 3, 128), dtype=torch.bfloat16, device="cuda")
    args = (t["x_norm_weight"], t["adaln_scale"], t["adaln_shift"])
    rest = (t["qkv_weight"], t["q_norm_weight"], t["k_norm_weight"], t["rope_cos_sin"])
    _dit().dit_pre_attn_bf16(t["x"], *args, t["adaln_index"], *rest, ulysses_degree=1, out=out0, eps=t["eps"],
                             qk_eps=t["qk_eps"], rope_positions=t["rope_positions"], workspace=ws0)
    M = 1 << 20
    reps = M // B
    _say(f"pre_attn M={M} from a repeated {B}-row block (out {M * 56 * 3 * 128 * 2 / 2**30:.0f} GiB)")
    xb = t["x"].repeat(reps, 1)
    wsb = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    outb = torch.empty((1, M, 56, 3, 128), dtype=torch.bfloat16, device="cuda")
    _dit().dit_pre_attn_bf16(xb, *args, t["adaln_index"].repeat(reps), *rest, ulysses_degree=1, out=outb,
                             eps=t["eps"], qk_eps=t["qk_eps"], rope_positions=t["rope_positions"].repeat(reps),
                             workspace=wsb)
    torch.cuda.synchronize()
    row_bytes = 56 * 3 * 128 * 2
    tiles = sorted({0, (1 << 32) // row_bytes // 256, (1 << 33) // row_bytes // 256, M // 512, M // 256 - 1})
    for ti in tiles:
        r0, b0 = ti * 256, (ti * 256) % B
        assert torch.equal(outb[0, r0:r0 + 256].view(torch.int16), out0[0, b0:b0 + 256].view(torch.int16)), ti
        assert torch.equal(wsb[r0:r0 + 256].view(torch.int16), ws0[b0:b0 + 256].view(torch.int16)), ti
    del xb, wsb, outb
    torch.cuda.empty_cache()

    o = synth.out_proj_inputs(B, seed=22)
    to = synth.to_torch("out_proj", o)
    out0 = _dit().dit_out_proj_gated_bf16(to["attn_out"], to["o_weight"], to["gate"], to["gate_index"],
                                          to["residual"])
    M = 1 << 19
    reps = M // B
    _say(f"out_proj M={M} from a repeated {B}-row block")
    outb = _dit().dit_out_proj_gated_bf16(to["attn_out"].repeat(reps, 1), to["o_weight"], to["gate"],
                                          to["gate_index"].repeat(reps), to["residual"].repeat(reps, 1))
    torch.cuda.synchronize()
    tiles = sorted({0, (1 << 32) // (H * 2) // 256, M // 512, M // 256 - 1})
    for ti in tiles:
        r0, b0 = ti * 256, (ti * 256) % B
        assert torch.equal(outb[r0:r0 + 256].view(torch.int16), out0[b0:b0 + 256].view(torch.int16)), ti
    del outb
    torch.cuda.empty_cache()


def test_persistent_gemms_on_two_streams_at_once():
    """Each persistent GEMM launch takes its own set of tile counters: a pre-attention and an
    out-projection enqueued on two streams without a sync between them (so that they may run
    at the same time) give the same bits as the two run one after the other."""
    dit = _dit()
    d = synth.pre_attn_inputs(4096, seed=31, rows=2, S=4096, positions="random", weight=_shared_weight())
    o = synth.out_proj_inputs(4096, seed=32)
    t, to = synth.to_torch("pre_attn", d), synth.to_torch("out_proj", o)
    outs = [torch.empty((1, 4096, 56, 3, 128), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    ws = [torch.empty((4096, H), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    po = [torch.empty((4096, H), dtype=torch.bfloat16, device="cuda") for _ in range(2)]

    def pre(i):
        dit.dit_pre_attn_bf16(t["x"], t["x_norm_weight"], t["adaln_scale"], t["adaln_shift"], t["adaln_index"],
                              t["qkv_weight"], t["q_norm_weight"], t["k_norm_weight"], t["rope_cos_sin"],
                              ulysses_degree=1, out=outs[i], eps=t["eps"], qk_eps=t["qk_eps"],
                              rope_positions=t["rope_positions"], workspace=ws[i])

    def oproj(i):
        dit.dit_out_proj_gated_bf16(to["attn_out"], to["o_weight"], to["gate"], to["gate_index"], to["residual"],
                                    out=po[i])

    pre(0)
    oproj(0)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        for b in outs[1:] + po[1:]:
            b.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            pre(1)
        with torch.cuda.stream(s2):
            oproj(1)
        torch.cuda.synchronize()
        assert torch.equal(outs[1].view(torch.int16), outs[0].view(torch.int16)), rep
        assert torch.equal(po[1].view(torch.int16), po[0].view(torch.int16)), rep


def test_counter_sets_are_left_at_zero_for_their_next_use():
    """The tile counters come from a pool of 4096 sets in rotation, and the last workgroup of
    each launch puts its set back to zero: 4200 out-projection launches (every set used twice
    over, some three times) all give the bits of the first."""
    dit = _dit()
    o = synth.out_proj_inputs(300, seed=34)
    to = synth.to_torch("out_proj", o)
    outs = [torch.empty((300, H), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    dit.dit_out_proj_gated_bf16(to["attn_out"], to["o_weight"], to["gate"], to["gate_index"], to["residual"],
                                out=outs[0])
    torch.cuda.synchronize()
    for i in range(4200):
        dit.dit_out_proj_gated_bf16(to["attn_out"], to["o_weight"], to["gate"], to["gate_index"], to["residual"],
                                    out=outs[1])
        if i % 700 == 699:
            torch.cuda.synchronize()
            assert torch.equal(outs[1].view(torch.int16), outs[0].view(torch.int16)), i
            outs[1].zero_()


def test_persistent_gemm_replayed_from_a_captured_graph():
    """The pre-attention (norm, counter zeroing, persistent QKV GEMM) captured in a HIP graph:
    every replay, with eager work and synchronisations between replays, equals the eager run."""
    dit = _dit()
    d = synth.pre_attn_inputs(2048, seed=33, rows=2, S=2048, positions="random", weight=_shared_weight())
    t = synth.to_torch("pre_attn", d)
    out = torch.empty((1, 2048, 56, 3, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((2048, H), dtype=torch.bfloat16, device="cuda")

    def pre():
        dit.dit_pre_attn_bf16(t["x"], t["x_norm_weight"], t["adaln_scale"], t["adaln_shift"], t["adaln_index"],
                              t["qkv_weight"], t["q_norm_weight"], t["k_norm_weight"], t["rope_cos_sin"],
                              ulysses_degree=1, out=out, eps=t["eps"], qk_eps=t["qk_eps"],
                              rope_positions=t["rope_positions"], workspace=ws)

    pre()
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pre()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        pre()
    for rep in range(4):
        out.zero_()
        ws.zero_()
        pre() if rep == 2 else None             # eager work between replays
        torch.cuda.synchronize()
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), rep


@pytest.mark.parametrize("P", [2, 4, 8])
def test_pre_attn_ulysses_pack_is_the_degree_one_output_repacked(P):
    """P destinations: the same values as P = 1, bit for bit, in the destination-major layout
    [P, M, 56 // P, 3, 128] (two m-tiles with a ragged tail, random positions, guarded rows)."""
    M = 300
    _say(f"pre_attn ulysses P={P}, M={M}")
    d = synth.pre_attn_inputs(M, seed=400 + P, rows=2, S=512, positions="random", n_bad_positions=4,
                              bad_index_frac=0.02, weight=_shared_weight())
    _, out1 = run_pre(d, P=1)
    _, outp = run_pre(d, P=P)
    one = synth.bits(out1).reshape(M, 56, 3, 128)
    got = synth.bits(outp)
    assert got.shape == (P, M, 56 // P, 3, 128)
    assert np.array_equal(got, oracle.ulysses_pack(one, P))


# descales that put the q/k outputs (RMS ~1 after the norm) and the v outputs (~N(0,1)) over
# most of the e4m3 range, with some saturation
E4M3_DESCALE = (1.0 / 96.0, 0.015, 0.0075)


@pytest.mark.parametrize("P", [1, 2])
def test_pre_attn_e4m3_codes_are_the_bf16_output_quantised(P):
    """e4m3 output mode: every code is e4m3(fl32(o / descale)) of the bf16 mode's own output o
    (the same fp32 quotient decides the code on both sides), in the same layout; two m-tiles
    with a ragged tail, random positions, guarded rows."""
    M = 300
    _say(f"pre_attn e4m3 output, P={P}, M={M}")
    d = synth.pre_attn_inputs(M, seed=500 + P, rows=2, S=512, positions="random", n_bad_positions=4,
                              bad_index_frac=0.02, weight=_shared_weight())
    _, outb = run_pre(d, P=P)
    codes = run_pre_e4m3(d, E4M3_DESCALE, P=P)
    ref = e4m3_of_bf16(synth.bits(outb), E4M3_DESCALE)
    assert codes.shape == ref.shape == (P, M, 56 // P, 3, 128)
    mism = np.mean(codes != ref)
    _say(f"  codes != e4m3(bf16 out / descale): {mism:.2e}; saturated {np.mean((codes & 0x7F) == 0x7E):.2e}")
    assert np.array_equal(codes, ref)


def test_pre_attn_e4m3_against_oracle():
    """config 0 (M = 16, guarded rows, rows=4 tables) in e4m3 mode against the oracle's codes of
    its own bf16 output: within one code step (the bf16 values may differ by an ulp), guarded
    rows exactly zero."""
    _say("config 0, e4m3 output")
    kind, d = synth.config(0)
    codes = run_pre_e4m3(d, E4M3_DESCALE).reshape(16, 56, 3, 128)
    _, out_ref = oracle.pre_attn(d)
    ref = oracle.quant_out_e4m3(out_ref, *E4M3_DESCALE)
    step = np.abs(ordered_e4m3(codes) - ordered_e4m3(ref))
    idx = d["adaln_index"]
    bad = (idx < 0) | (idx >= d["adaln_scale"].rows)
    _say(f"  code mismatch {np.mean(codes != ref):.2e}, max step {step.max()}, guarded rows {bad.sum()}")
    assert step.max() <= 1
    assert np.all(codes[bad] == 0)


def test_pre_attn_ulysses_degree8_against_oracle():
    """P = 8 on the M = 16 workload (guarded rows, rows=4 tables), checked against the oracle's
    output after the oracle's destination-major pack."""
    _say("config 0 with ulysses_degree 8")
    kind, d = synth.config(0)
    ws = torch.empty((16, H), dtype=torch.bfloat16, device="cuda")
    _, outp = run_pre(d, workspace=ws, P=8)
    got = synth.bits(outp)
    ws_ref, out_ref = oracle.pre_attn(d)
    assert got.shape == (8, 16, 7, 3, 128)
    # destination p holds heads [7 p, 7 p + 7): put them back side by side and compare per row
    unpacked = np.concatenate(list(got), axis=1)
    check_qkv(unpacked, out_ref, row_cos_sin(d, np.arange(16)), "P=8")
    idx = d["adaln_index"]
    bad = (idx < 0) | (idx >= d["adaln_scale"].rows)
    assert np.all(bf16_val(got[:, bad]) == 0.0), "guarded rows must be zero in every destination"


_W = {}


def _shared_weight():
    if "w" not in _W:
        _W["w"] = synth.to_bf16_bits(synth.normal(1, "qkv_weight", (synth.QKV_ROWS, H), 1 / np.sqrt(H)))
    return _W["w"]


def test_pre_attn_identity_positions_ragged():
    M = 300
    _say(f"pre_attn identity positions M={M}")
    d = synth.pre_attn_inputs(M, seed=7, rows=3, S=M, positions="identity", bad_index_frac=0.02,
                              bad_index_values=(-1, 3, INT64_MIN, INT64_MAX, 1 << 32), weight=_shared_weight())
    ws = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    _, out = run_pre(d, workspace=ws)
    check_pre(d, ws, out)


def _eps_visible_inputs(M, seed, eps, qk_eps):
    """Pre-attention inputs on which eps and qk_eps both move the result by far more than an ulp:
    rows 0-63 of x scaled by 1e-2 (mean(x^2) ~ 1e-4 ~ eps), rows 64-67 constant
    (2^-8, 2^-7, -2^-6, 2^-5: c^2 within a few decades of eps), the q and k weight rows of heads
    0-3 scaled by 0.2 (mean(v^2) ~ 0.04 ~ qk_eps) and of heads 4-7 by 0.01 (mean(v^2) ~ 1e-4)."""
    d = synth.pre_attn_inputs(M, seed=seed, rows=2, S=512, positions="random", n_bad_positions=4,
                              bad_index_frac=0.02, weight=_shared_weight())
    x = bf16_val(d["x"]).reshape(M, H)
    x[:64] *= 0.01
    for r, c in zip(range(64, 68), (2.0 ** -8, 2.0 ** -7, -(2.0 ** -6), 2.0 ** -5)):
        x[r] = c
    d["x"] = synth.to_bf16_bits(x.astype(np.float32))
    W = _shared_weight().copy()
    for kind in (0, 1):
        for h, f in [(h, 0.2) for h in range(4)] + [(h, 0.01) for h in range(4, 8)]:
            r0 = kind * 7168 + h * 128
            W[r0:r0 + 128] = synth.to_bf16_bits((bf16_val(W[r0:r0 + 128]) * f).astype(np.float32))
    d["qkv_weight"] = W
    d["eps"], d["qk_eps"] = eps, qk_eps
    return d


def test_pre_attn_eps_and_qk_eps_are_both_visible():
    """eps = 1e-4 and qk_eps = 0.05 on rows and heads whose mean squares are of the same order
    (_eps_visible_inputs), against the oracle.  The oracle run with eps and qk_eps swapped (a
    mistake planted on the CPU) must fail the same bars, so the test tells the two apart."""
    M = 300
    eps, qk_eps = 1e-4, 0.05
    _say(f"pre_attn eps={eps} qk_eps={qk_eps}, M={M}")
    d = _eps_visible_inputs(M, 710, eps, qk_eps)
    ws = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    _, out = run_pre(d, workspace=ws)
    check_pre(d, ws, out)
    rows = np.r_[np.arange(0, 8), np.arange(64, 72)]
    _, swapped = oracle.pre_attn(dict(d, eps=qk_eps, qk_eps=eps), rows_sel=rows)
    got = synth.bits(out).reshape(M, 56, 3, 128)[rows]
    assert not qkv_check(got, swapped, row_cos_sin(d, rows))[0], "the bar cannot tell eps from qk_eps"


def test_pre_attn_qk_eps_none_means_eps():
    """qk_eps=None through the binding: the q/k heads are normalised with eps (the page's
    default), checked against the oracle with qk_eps = eps; the oracle with qk_eps = 0.05 must fail."""
    M = 257
    eps = 1e-4
    _say(f"pre_attn qk_eps=None, eps={eps}, M={M}")
    d = _eps_visible_inputs(M, 711, eps, None)
    ws = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    _, out = run_pre(d, workspace=ws)
    check_pre(d, ws, out)
    rows = np.arange(0, 16)
    _, other = oracle.pre_attn(dict(d, qk_eps=0.05), rows_sel=rows)
    got = synth.bits(out).reshape(M, 56, 3, 128)[rows]
    assert not qkv_check(got, other, row_cos_sin(d, rows))[0]


def test_pre_attn_one_hot_pack_bit_exact():
    # one-hot W: qkv[n] = a[k(n)] exactly, so V heads are bit copies of workspace entries
    M = 260
    _say("pre_attn one-hot weight pack check")
    W = np.zeros((synth.QKV_ROWS, H), np.uint16)
    n = np.arange(synth.QKV_ROWS)
    k = (n * 5 + 3) % H
    W[n, k] = 0x3F80
    d = synth.pre_attn_inputs(M, seed=8, rows=2, S=M, positions="identity", bad_index_frac=0.0, weight=W)
    ws = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    _, out = run_pre(d, workspace=ws)
    wsb = synth.bits(ws)
    ob = synth.bits(out).reshape(M, 56, 3, 128)
    v_expect = wsb[:, k[2 * 7168:]].reshape(M, 56, 128)
    assert np.array_equal(ob[:, :, 2], v_expect)
    check_pre(d, ws, out)


def test_pre_attn_exact_rope_angles():
    # with (cos, sin) in {(1,0),(0,1),(-1,0),(0,-1)} RoPE is a permutation/negation of u; the
    # GPU's output must be exactly that transform of its own cos=1, sin=0 output
    M = 64
    _say("pre_attn exact RoPE angles")
    d = synth.pre_attn_inputs(M, seed=9, rows=2, S=M, positions="identity", bad_index_frac=0.0,
                              weight=_shared_weight())
    d["rope_cos_sin"] = synth.to_bf16_bits(np.concatenate([np.ones((M, 48)), np.zeros((M, 48))], 1).astype(np.float32))
    ws = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    _, out_u = run_pre(d, workspace=ws)
    u = bf16_val(synth.bits(out_u).reshape(M, 56, 3, 128))
    check_pre(d, ws, out_u)
    pairs = np.array([[1, 0], [0, 1], [-1, 0], [0, -1]], np.float32)
    sel = (np.arange(M)[:, None] + np.arange(48)[None, :]) % 4
    c, s_ = pairs[sel, 0], pairs[sel, 1]
    d["rope_cos_sin"] = synth.to_bf16_bits(np.concatenate([c, s_], axis=1).astype(np.float32))
    _, out = run_pre(d, workspace=ws)
    o = bf16_val(synth.bits(out).reshape(M, 56, 3, 128))
    for kind in (0, 1):
        lo, hi = u[:, :, kind, :48], u[:, :, kind, 48:96]
        cc, ss = c[:, None, :], s_[:, None, :]
        assert np.array_equal(o[:, :, kind, :48], lo * cc - hi * ss)
        assert np.array_equal(o[:, :, kind, 48:96], hi * cc + lo * ss)
        assert np.array_equal(o[:, :, kind, 96:], u[:, :, kind, 96:])
    assert np.array_equal(o[:, :, 2], u[:, :, 2])
    check_pre(d, ws, out)


def test_pre_attn_config1_sampled():
    _say("config 1: pre_attn M=4096, S=8192 random positions with 8 clamps, ~0.5% guarded")
    kind, d = synth.config(1)
    ws = torch.empty((d["M"], H), dtype=torch.bfloat16, device="cuda")
    _, out = run_pre(d, workspace=ws)
    check_pre(d, ws, out, sample_rows(d["M"], d))


def test_pre_attn_config2_sampled_and_deterministic():
    _say("config 2: pre_attn M=32760 identity positions (the measured workload)")
    kind, d = synth.config(2)
    ws = torch.empty((d["M"], H), dtype=torch.bfloat16, device="cuda")
    _, out = run_pre(d, workspace=ws)
    ws1, out1 = synth.bits(ws), synth.bits(out)
    _, out2 = run_pre(d, workspace=ws)
    assert np.array_equal(out1, synth.bits(out2)) and np.array_equal(ws1, synth.bits(ws)), "not deterministic"
    check_pre(d, ws, out, sample_rows(d["M"], d))


# ---------------------------------------------------------------- out-projection

@pytest.mark.parametrize("M", [1, 3, 257])
def test_out_proj_small_M(M):
    _say(f"out_proj small M={M}")
    d = synth.out_proj_inputs(M, seed=200 + M)
    out = run_out_proj(d)
    check_out_proj(d, out)


def test_out_proj_alias_residual():
    M = 300
    _say("out_proj out is residual")
    d = synth.out_proj_inputs(M, seed=5)
    out = run_out_proj(d, alias=True)
    check_out_proj(d, out)


def test_out_proj_config3_sampled():
    _say("config 3: out_proj M=32760")
    kind, d = synth.config(3)
    out = run_out_proj(d)
    o1 = synth.bits(out)
    out2 = run_out_proj(d)
    assert np.array_equal(o1, synth.bits(out2)), "not deterministic"
    check_out_proj(d, out, sample_rows(d["M"], d))


# ---------------------------------------------------------------- MXFP4 W4A4 out-projection

def mx_scales_rowmajor(scales_gpu, R, K):
    """Scales in the MX scale layout (as include/dit.h states it) read back as [R, K/32]
    row-major bytes, plus the bytes of the padding rows up to a multiple of 128."""
    sc = scales_gpu.cpu().numpy()
    R_pad = (R + 127) // 128 * 128
    r = np.arange(R_pad)[:, None]
    b = np.arange(K // 32)[None, :]
    lane = r % 32 + 32 * (b % 2)
    off = ((r // 128) * (K // 256) + b // 8) * 1024 + lane * 16 + 4 * ((r % 128) // 32) + (b % 8) // 2
    assert sc.size == R_pad * (K // 32) and np.array_equal(np.sort(off.ravel()), np.arange(sc.size))
    full = sc[off]
    return full[:R], full[R:]


def _bf16_cuda(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _mx_special_rows(R, K, seed):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((R, K)) * np.exp2(rng.integers(-40, 40, (R, 1)))
    v[0, :32] = 0.0                                                    # zero block
    v[0, 32:64] = -0.0                                                 # negative zeros
    v[1, :32] = rng.integers(-3, 4, 32) * 2.0 ** -131                  # bf16 subnormals
    v[1, 32:64] = rng.uniform(-3e38, 3e38, 32)                         # near the bf16 maximum
    k = 2.0 ** -5                                                      # exact E2M1 midpoints, amax 4 k
    v[2, :32] = np.resize([4.0, 0.25, -0.75, 1.25, 1.75, -2.5, 3.5, 5.0, 0.3, -5.5], 32) * k
    v[2, 32:64] = np.resize([7.0, -6.5, 7.99, 0.1], 32)                # saturation (amax in [4, 8))
    return synth.to_bf16_bits(v.astype(np.float32))


@pytest.mark.parametrize("R,K", [(300, 7168), (3, 256), (128, 512)])
def test_mx_quant_fp4_matches_the_oracle_bit_for_bit(R, K):
    _say(f"mx quant R={R} K={K}")
    x = _mx_special_rows(R, K, seed=R + K)
    codes, scales = _dit().dit_mx_quant_fp4(_bf16_cuda(x))
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.mx_quant_fp4(x)
    assert np.array_equal(codes.cpu().numpy(), c_ref), "codes"
    rm, pad = mx_scales_rowmajor(scales, R, K)
    assert np.array_equal(rm, s_ref), "scales"
    assert np.all(pad == 0), "padding rows' scales"


def test_mx_quant_fp4_every_finite_bf16_value_at_every_scale():
    # For each scale byte E = 0 .. 252 (252 is the largest a finite bf16 maximum gives), blocks
    # led by 2^(E - 125), whose exponent field E + 2 sets the block scale to E, and filled with
    # every finite bf16 value of both signs with an exponent field up to E + 2: each finite value
    # quantised at every scale its block can have, about 8.6 million values in all.
    blocks, want_E = [], []
    mags = np.arange(0x7F80, dtype=np.uint16)                         # finite magnitudes
    for E in range(253):
        vals = mags[(mags >> 7) <= E + 2]
        vals = np.concatenate([vals, vals | 0x8000])
        n = -(-vals.size // 31)
        b = np.zeros((n, 32), np.uint16)
        b[:, 0] = (E + 2) << 7
        b[:, 1:].reshape(-1)[:vals.size] = vals
        blocks.append(b)
        want_E.append(np.full(n, E, np.uint8))
    blocks, want_E = np.concatenate(blocks), np.concatenate(want_E)
    K = 7168
    per_row = K // 32
    R = -(-blocks.shape[0] // per_row)
    x = np.zeros((R * per_row, 32), np.uint16)
    x[:blocks.shape[0]] = blocks
    x = x.reshape(R, K)
    _say(f"mx quant, every finite bf16 value at every scale: R={R} K={K}")
    codes, scales = _dit().dit_mx_quant_fp4(_bf16_cuda(x))
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.mx_quant_fp4(x)
    assert np.array_equal(s_ref.reshape(-1)[:want_E.size], want_E), "oracle scale bytes"
    rm, pad = mx_scales_rowmajor(scales, R, K)
    assert np.array_equal(rm, s_ref), "scales"
    assert np.array_equal(codes.cpu().numpy(), c_ref), "codes"


def test_norm_adaln_one_plus_scale_for_every_finite_bf16_scale():
    # x = 1, w = 1 and shift = 0 make n = bf16(r) = 1 exactly (r = 1 / sqrt(1 + eps) rounds to the
    # bf16 1), so the workspace is a = bf16(1 + scale) itself: every finite bf16 scale, bit for bit
    pat = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    pat = pat[((pat >> 7) & 0xFF) != 0xFF]
    rows = -(-pat.size // H)
    sc = np.zeros((rows, H), np.uint16)
    sc.reshape(-1)[:pat.size] = pat
    zeros = np.zeros((rows, H), np.uint16)
    one_x = np.full((rows, H), 0x3F80, np.uint16)
    one_w = np.full(H, 0x3F80, np.uint16)
    idx = np.arange(rows, dtype=np.int64)
    _say(f"norm_adaln, 1 + scale for {pat.size} scale values")
    ws = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda")
    _dit().dit_norm_adaln_bf16(_bf16_cuda(one_x), _bf16_cuda(one_w), _bf16_cuda(sc), _bf16_cuda(zeros),
                               torch.from_numpy(idx).cuda(), workspace=ws, eps=1e-6)
    torch.cuda.synchronize()
    d = {"M": rows, "x": one_x, "x_norm_weight": one_w, "adaln_scale": synth.Table(sc.reshape(-1), 0, rows, H),
         "adaln_shift": synth.Table(zeros.reshape(-1), 0, rows, H), "adaln_index": idx, "eps": 1e-6}
    ref = oracle.norm_adaln(d)
    want = synth.to_bf16_bits((1.0 + bf16_val(sc)).astype(np.float32))
    assert np.array_equal(ref, want), "oracle: bf16(1 + scale)"
    assert np.array_equal(synth.bits(ws), ref), "workspace"


_MXW = {}


def _mx_weight():
    """A bf16 o_weight, its MXFP4 form from the GPU quantiser and from the oracle's (checked equal)."""
    if "w" not in _MXW:
        W = synth.to_bf16_bits(synth.normal(91, "o_weight", (H, synth.ATTN_WIDTH), 1.0 / np.sqrt(synth.ATTN_WIDTH)))
        wc, ws = _dit().dit_mx_quant_fp4(_bf16_cuda(W))
        torch.cuda.synchronize()
        wc_ref, ws_ref = oracle.mx_quant_fp4(W)
        assert np.array_equal(wc.cpu().numpy(), wc_ref)
        rm, _ = mx_scales_rowmajor(ws, H, synth.ATTN_WIDTH)
        assert np.array_equal(rm, ws_ref)
        _MXW["w"] = (W, wc, ws, wc_ref, ws_ref)
    return _MXW["w"]


def run_out_proj_mx(d, alias=False):
    W, wc, ws, _, _ = _mx_weight()
    t = synth.to_torch("out_proj", d)
    M = d["M"]
    ac = torch.empty((M, synth.ATTN_WIDTH // 2), dtype=torch.uint8, device="cuda")
    asc = torch.empty((_dit().dit_mx_scale_bytes(M, synth.ATTN_WIDTH),), dtype=torch.uint8, device="cuda")
    out = t["residual"] if alias else None
    out = _dit().dit_out_proj_gated_mxfp4(t["attn_out"], wc, ws, t["gate"], t["gate_index"], t["residual"], out=out,
                                          act_codes=ac, act_scales=asc)
    torch.cuda.synchronize()
    return out, ac, asc


def check_out_proj_mx(d, out_gpu, ac, asc, rows):
    M = d["M"]
    _, _, _, wc_ref, ws_ref = _mx_weight()
    a_c, a_s = oracle.mx_quant_fp4(d["attn_out"].reshape(M, synth.ATTN_WIDTH)[rows])
    assert np.array_equal(ac.cpu().numpy()[rows], a_c), "activation codes"
    rm, pad = mx_scales_rowmajor(asc, M, synth.ATTN_WIDTH)
    assert np.array_equal(rm[rows], a_s) and np.all(pad == 0), "activation scales"
    ref = oracle.out_proj_mxfp4(a_c, a_s, wc_ref, ws_ref, dict(d, M=rows.size, gate_index=d["gate_index"][rows],
                                                                residual=d["residual"].reshape(M, H)[rows]))
    got = synth.bits(out_gpu)[rows]
    gi = d["gate_index"][rows]
    bad = (gi < 0) | (gi >= d["gate"].rows)
    assert np.array_equal(got[bad], d["residual"].reshape(M, H)[rows][bad]), "guarded rows must equal residual"
    res = d["residual"].reshape(M, H)[rows]
    g = np.where(bad[:, None], 0.0, bf16_val(d["gate"].dense())[np.where(bad, 0, gi)])
    ok, rel, mx, n_far, worst = gated_tolerance_ok(got, ref, res, g)
    _say(f"out_proj mxfp4 M={M} rows={rows.size} relL2={rel:.2e} max|err|={mx:.3e} mismatch={np.mean(got != ref):.2e} "
         f"past the plain bar={n_far}")
    assert ok, (rel, mx, n_far, worst)


@pytest.mark.parametrize("M", [1, 300])
def test_out_proj_mxfp4_against_oracle(M):
    _say(f"out_proj mxfp4 M={M}")
    d = synth.out_proj_inputs(M, seed=400 + M, weight=_mx_weight()[0])
    out, ac, asc = run_out_proj_mx(d)
    rows = np.arange(M) if M <= 4 else np.unique(np.r_[np.arange(8), np.arange(250, 262), np.arange(M - 12, M),
                                                       np.nonzero(d["gate_index"] < 0)[0][:4]])
    check_out_proj_mx(d, out, ac, asc, rows)


def test_out_proj_mxfp4_alias_residual_and_full_size():
    M = 32760
    _say(f"out_proj mxfp4 M={M}, out is residual")
    d = synth.out_proj_inputs(M, seed=7, weight=_mx_weight()[0])
    again = synth.bits(run_out_proj_mx(d)[0])
    out, ac, asc = run_out_proj_mx(d, alias=True)
    assert np.array_equal(synth.bits(out), again), "not deterministic (or aliasing changed the result)"
    g = np.random.default_rng(8)
    rows = np.unique(np.r_[np.arange(16), np.arange(M - 16, M), np.nonzero(d["gate_index"] < 0)[0][:16],
                           g.choice(M, 24, replace=False)])
    check_out_proj_mx(d, out, ac, asc, rows)


# ---------------------------------------------------------------- MXFP4 W4A4 pre-attention

_MXQ = {}


def _mx_qkv_weight():
    """The shared qkv weight's MXFP4 form from the GPU quantiser and from the oracle's (checked equal)."""
    if "w" not in _MXQ:
        W = _shared_weight()
        wc, ws = _dit().dit_mx_quant_fp4(_bf16_cuda(W))
        torch.cuda.synchronize()
        wc_ref, ws_ref = oracle.mx_quant_fp4(W)
        assert np.array_equal(wc.cpu().numpy(), wc_ref)
        rm, _ = mx_scales_rowmajor(ws, synth.QKV_ROWS, H)
        assert np.array_equal(rm, ws_ref)
        _MXQ["w"] = (wc, ws, wc_ref, ws_ref)
    return _MXQ["w"]


def run_pre_mx(d, P=1):
    t = synth.to_torch("pre_attn", d)
    wc, ws, _, _ = _mx_qkv_weight()
    M = d["M"]
    out = torch.empty((P, M, 56 // P, 3, 128), dtype=torch.bfloat16, device="cuda")
    wsc = torch.empty((M, H // 2), dtype=torch.uint8, device="cuda")
    wss = torch.empty((_dit().dit_mx_scale_bytes(M, H),), dtype=torch.uint8, device="cuda")
    _dit().dit_pre_attn_mxfp4(t["x"], t["x_norm_weight"], t["adaln_scale"], t["adaln_shift"], t["adaln_index"], wc, ws,
                              t["q_norm_weight"], t["k_norm_weight"], t["rope_cos_sin"], ulysses_degree=P, out=out,
                              eps=t["eps"], qk_eps=t["qk_eps"], rope_positions=t["rope_positions"], ws_codes=wsc,
                              ws_scales=wss)
    # the bf16 workspace of the same rows: the fused quantisation must be its MXFP4
    wsb = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    _dit().dit_norm_adaln_bf16(t["x"], t["x_norm_weight"], t["adaln_scale"], t["adaln_shift"], t["adaln_index"],
                               workspace=wsb, eps=t["eps"])
    torch.cuda.synchronize()
    return out, wsc, wss, wsb


def check_pre_mx(d, out, wsc, wss, wsb, rows):
    M = d["M"]
    c_ref, s_ref = oracle.mx_quant_fp4(synth.bits(wsb)[rows])
    assert np.array_equal(wsc.cpu().numpy()[rows], c_ref), "workspace codes"
    rm, pad = mx_scales_rowmajor(wss, M, H)
    assert np.array_equal(rm[rows], s_ref) and np.all(pad == 0), "workspace scales"
    _, _, wc_ref, ws_ref = _mx_qkv_weight()
    ref = oracle.qkv_mxfp4(c_ref, s_ref, wc_ref, ws_ref, d, rows_sel=rows)
    got = synth.bits(out).reshape(M, 56, 3, 128)[rows]
    idx = d["adaln_index"][rows]
    bad = (idx < 0) | (idx >= d["adaln_scale"].rows)
    assert np.all(bf16_val(got[bad]) == 0.0), "guarded output rows must be zero"
    _say(f"pre_attn mxfp4 M={M} rows={rows.size} mismatch={np.mean(got != ref):.2e} guarded={bad.sum()}")
    check_qkv(got, ref, row_cos_sin(d, rows), f"pre_attn mxfp4 M={M} out")


def test_pre_attn_mxfp4_against_oracle():
    M = 300
    _say(f"pre_attn mxfp4 M={M}")
    d = synth.pre_attn_inputs(M, seed=600, rows=2, S=512, positions="random", n_bad_positions=4,
                              bad_index_frac=0.02, weight=_shared_weight())
    out, wsc, wss, wsb = run_pre_mx(d)
    bad = np.nonzero((d["adaln_index"] < 0) | (d["adaln_index"] >= 2))[0]
    rows = np.unique(np.r_[np.arange(8), np.arange(250, 262), np.arange(M - 8, M), bad[:4]])
    check_pre_mx(d, out, wsc, wss, wsb, rows)


@pytest.mark.parametrize("M", [1, 129])
def test_pre_attn_mxfp4_small_M(M):
    # one row (127 padding scale rows), and one row past a 128-row scale block
    _say(f"pre_attn mxfp4 M={M}")
    d = synth.pre_attn_inputs(M, seed=603 + M, rows=2, S=64, positions="random", n_bad_positions=1,
                              bad_index_frac=0.05, weight=_shared_weight())
    out, wsc, wss, wsb = run_pre_mx(d)
    rows = np.unique(np.r_[np.arange(min(M, 4)), np.arange(max(M - 6, 0), M)])
    check_pre_mx(d, out, wsc, wss, wsb, rows)


def test_pre_attn_mxfp4_ulysses_pack():
    M = 300
    _say(f"pre_attn mxfp4 P=2, 4, 8 against P=1, M={M}")
    d = synth.pre_attn_inputs(M, seed=601, rows=2, S=512, positions="random", n_bad_positions=4,
                              weight=_shared_weight())
    one = synth.bits(run_pre_mx(d, P=1)[0]).reshape(M, 56, 3, 128)
    for P in (2, 4, 8):
        got = synth.bits(run_pre_mx(d, P=P)[0])
        assert got.shape == (P, M, 56 // P, 3, 128)
        assert np.array_equal(got, oracle.ulysses_pack(one, P)), P


def test_pre_attn_mxfp4_full_size_sampled():
    M = 32760
    _say(f"pre_attn mxfp4 M={M}")
    d = synth.pre_attn_inputs(M, seed=602, rows=2, S=M, positions="identity", weight=_shared_weight())
    out, wsc, wss, wsb = run_pre_mx(d)
    out2, wsc2, wss2, _ = run_pre_mx(d)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)) and torch.equal(wsc, wsc2) and \
        torch.equal(wss, wss2), "not deterministic"
    g = np.random.default_rng(9)
    rows = np.unique(np.r_[np.arange(8), np.arange(M - 8, M), g.choice(M, 16, replace=False)])
    check_pre_mx(d, out, wsc, wss, wsb, rows)


# ---------------------------------------------------------------- FP8 MLP

_MW = {}


def _mlp_weights():
    if "w" not in _MW:
        _MW["w"] = synth.mlp_weights(33)
    return _MW["w"]


@pytest.mark.parametrize("M", [1, 2, 257])
def test_mlp_small_M(M):
    _say(f"mlp small M={M}")
    d = synth.mlp_inputs(M, seed=300 + M, weights=_mlp_weights(), bad_index_frac=0.02,
                         bad_index_values=(-1, 2, INT64_MIN, INT64_MAX))
    out, ws = run_mlp(d)
    check_mlp(d, out, ws)


@pytest.mark.parametrize("alias", ["residual", "x"])
def test_mlp_alias(alias):
    M = 40
    _say(f"mlp out is {alias}")
    d = synth.mlp_inputs(M, seed=400, weights=_mlp_weights(), bad_index_frac=0.05)
    out, ws = run_mlp(d, alias=alias)
    check_mlp(d, out, ws)


def test_mlp_subnormal_scales_and_visible_eps():
    """Per-token scales below 2^-126, where 1 / s overflows fp32, and eps = 1e-4 on rows with
    mean(x^2) ~ 1e-4.
    - Table row 2 has scale -1 (bf16(1 + scale) = 0) and shift values ~1e-37, so a = shift
      exactly, amax ~ 3e-37 and s_a = RN(amax / 448) is subnormal: the codes must equal the
      oracle's e4m3(fl32(a / s_a)) and the scales must be bit-equal.
    - A second run scales every FC1 column scale by 2^-63, so y ~ 1e-38 and s_y is subnormal
      (the y quantisation's own division path), checked with check_mlp's bars."""
    M = 40
    _say(f"mlp subnormal scales, eps visible, M={M}")
    d = synth.mlp_inputs(M, seed=420, rows=3, weights=_mlp_weights(), bad_index_frac=0.0)
    sc, sh = d["adaln_scale"], d["adaln_shift"]
    base = sc.base.copy()
    base[sc.offset + 2 * sc.row_stride:sc.offset + 2 * sc.row_stride + H] = 0xBF80          # -1.0
    tiny = synth.normal(421, "tiny_shift", (H,), 1e-37)
    base[sh.offset + 2 * sh.row_stride:sh.offset + 2 * sh.row_stride + H] = synth.to_bf16_bits(tiny)
    for t in ("adaln_scale", "adaln_shift", "gate"):
        d[t] = synth.Table(base, d[t].offset, d[t].rows, d[t].row_stride)
    d["adaln_index"][:8] = 2
    x = bf16_val(d["x"]).reshape(M, H)
    x[8:16] *= 0.01
    d["x"] = synth.to_bf16_bits(x.astype(np.float32))
    d["eps"] = 1e-4
    out, ws = run_mlp(d)
    ref = check_mlp(d, out, ws)
    a_q = synth.bits(ws["workspace_a_q"])
    a_s = ws["workspace_a_scale"].cpu().numpy()
    assert np.all((a_s[:8] > 0) & (a_s[:8] < 2.0 ** -128)), "row scales meant to be subnormal"
    assert np.array_equal(a_s[:8], ref["a_scale"][:8]) and np.array_equal(a_q[:8], ref["a_q"][:8])
    # subnormal s_y
    q1, s1, q2, s2 = _mlp_weights()
    d2 = dict(d, fc1_scale=(s1 * np.float32(2.0 ** -63)).astype(np.float32))
    out2, ws2 = run_mlp(d2)
    ref2 = check_mlp(d2, out2, ws2)
    y_s = ws2["workspace_y_scale"].cpu().numpy()
    live = ref2["y_scale"] > 0
    _say(f"  subnormal s_y: {live.sum()} rows with y != 0, {np.sum(live & (y_s < 2.0 ** -128))} of them below "
         f"2^-128, max {y_s.max():.3e}")
    assert live.sum() >= 16 and np.all(y_s[live] < 2.0 ** -126), "y scales meant to be subnormal"
    assert np.any(y_s[live] < 2.0 ** -128), "some 1 / s_y meant to overflow"
    # at this scale the bar's 1e-2 absolute term says nothing about y: hold its normal-range
    # elements to 4 ulp of the oracle's
    yg, yr = bf16_val(synth.bits(ws2["workspace_y"])), bf16_val(ref2["y"])
    normal = np.abs(yr) >= 2.0 ** -125
    assert normal.sum() > 1000
    assert np.all(np.abs(yg - yr)[normal] <= 4.0 * ulp_bf16(yr[normal])), "y at 1e-38"


def test_mlp_maximum_M():
    """M = 149796, the largest M the MLP page allows: 586 m-tiles, the last one ragged
    (36 rows).  Sampled rows (the first 256, the last m-tile, every guarded row, 32 random)
    against the oracle."""
    M = 149796
    _say(f"fp8 MLP at the maximum M={M}")
    d = synth.mlp_inputs(M, seed=900, bad_index_frac=0.0002)
    out, ws = run_mlp(d)
    check_mlp(d, out, ws, sample_rows(M, d, n_random=32))


@pytest.mark.parametrize("M", [8192, 16300])
def test_mlp_y_quant_inside_fc2(M):
    """M whose m tiles split into whole groups of four per XCD (32 and 64 m tiles), where FC2
    quantises y in its own launch: one group per XCD (all units before the tiles), and two
    groups per XCD (the second group's units among the first group's tiles) with a ragged last
    m tile (172 rows).  Sampled rows against the oracle (codes, scales, y and out), and a
    second run bit-identical."""
    _say(f"fp8 MLP, y quantised inside FC2, M={M}")
    d = synth.mlp_inputs(M, seed=950 + M % 97, weights=_mlp_weights(), bad_index_frac=0.001)
    out, ws = run_mlp(d)
    out2, ws2 = run_mlp(d)
    assert np.array_equal(synth.bits(out), synth.bits(out2)), "out not deterministic"
    for k in ("workspace_y_q", "workspace_y_scale"):
        assert torch.equal(ws[k].view(torch.uint8), ws2[k].view(torch.uint8)), f"{k} not deterministic"
    check_mlp(d, out, ws, sample_rows(M, d, n_random=96))


def test_mlp_config4_sampled_and_deterministic():
    _say("config 4: fp8 MLP M=32760")
    kind, d = synth.config(4)
    out, ws = run_mlp(d)
    o1 = synth.bits(out)
    y1 = synth.bits(ws["workspace_y_q"])
    out2, ws2 = run_mlp(d)
    assert np.array_equal(o1, synth.bits(out2)) and np.array_equal(y1, synth.bits(ws2["workspace_y_q"]))
    check_mlp(d, out, ws, sample_rows(d["M"], d))
