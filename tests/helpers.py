"""Shared test helpers: format properties and tolerance checks.

These encode properties of the number formats (what "nearest bf16" or "nearest e4m3"
means), never the stages' formulas, so they can judge the oracle as well as the HIP path.
"""
from __future__ import annotations

import numpy as np
import torch

import synth


def bf16_val(bits):
    return synth.bf16_bits_to_f32(np.asarray(bits, np.uint16)).astype(np.float64)


def _bf16_neighbors(bits):
    b = np.asarray(bits, np.uint16).astype(np.int64)
    sign = b & 0x8000
    mag = b & 0x7FFF
    up = bf16_val((sign | np.minimum(mag + 1, 0x7F7F)).astype(np.uint16))
    down = np.where(mag > 0, bf16_val((sign | np.maximum(mag - 1, 0)).astype(np.uint16)),
                    -bf16_val(np.ones_like(mag, dtype=np.uint16)))
    return down, up


def is_nearest_bf16(bits, exact, rtol=1e-12):
    """True where bits encode a bf16 value at least as close to `exact` as its two neighbours.

    rtol absorbs the float64 error of the library value `exact` at exact ties.
    """
    exact = np.asarray(exact, np.float64)
    r = bf16_val(bits)
    down, up = _bf16_neighbors(bits)
    d = np.abs(exact - r)
    slack = rtol * np.abs(exact) + 1e-300
    return (d <= np.abs(exact - down) + slack) & (d <= np.abs(exact - up) + slack)


def ulp_diff_bf16(a_bits, b_bits):
    """|difference| in bf16 units in the last place (ordered integer distance)."""
    def ordered(b):
        b = np.asarray(b, np.uint16).astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def e4m3_val(codes):
    return synth.e4m3_codes_to_f32(np.asarray(codes, np.uint8)).astype(np.float64)


def torch_e4m3(v32):
    """float8_e4m3fn codes of fp32 values |v| <= 448 by torch's conversion (a library routine)."""
    return torch.from_numpy(np.ascontiguousarray(v32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def ordered_e4m3(c):
    c = np.asarray(c, np.uint8).astype(np.int64)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def bf16_tolerance_ok(got_bits, ref_bits, max_rel_l2=2e-3, elem=1e-2):
    """The acceptance bar for bf16 outputs: relative L2 error and |err| <= elem*(1+|ref|)."""
    g = bf16_val(got_bits).ravel()
    r = bf16_val(ref_bits).ravel()
    m = np.abs(r)
    err = np.abs(g - r)
    rel_l2 = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
    ok_elem = np.all(err <= elem * (1.0 + m))
    return bool(rel_l2 <= max_rel_l2 and ok_elem), float(rel_l2), float(err.max() if err.size else 0.0)


def gated_tolerance_ok(got_bits, ref_bits, res_bits, gate_vals, max_rel_l2=2e-3, elem=1e-2):
    """The bar for gated-residual bf16 outputs out = bf16(res + bf16(g*o)).

    The plain bar holds per element: relative L2 error <= max_rel_l2 and |err| <= elem (1 + |ref|).
    Where the residual cancels the gated term, out is small while the error of the gated term
    keeps its own size.  Carried from o meeting the plain bar (|do| <= elem (1 + |o|)) through
    the two roundings, such an element may instead meet
        |err| <= elem (|g| + |ref - res| + ulp(ref)) + ulp(ref) + ulp(ref - res),
    with |ref - res| standing for |g*o| (within an ulp), for at most 4 + 1e-5 of the elements.
    Returns (ok, rel_l2, max_err, n_carried, worst err / carried bound).
    """
    err, rel_l2, plain, carried = _gated_terms(got_bits, ref_bits, res_bits, gate_vals, elem)
    n_far = int(np.sum(~plain))
    worst = float((err[~plain] / carried[~plain]).max()) if n_far else 0.0
    ok = rel_l2 <= max_rel_l2 and np.all(plain | (err <= carried)) and n_far <= 4 + 1e-5 * err.size
    return bool(ok), float(rel_l2), float(err.max() if err.size else 0.0), n_far, worst


def _gated_terms(got_bits, ref_bits, res_bits, gate_vals, elem):
    g = bf16_val(got_bits)
    r = bf16_val(ref_bits)
    res = bf16_val(res_bits)
    gv = np.abs(np.asarray(gate_vals, np.float64))
    err = np.abs(g - r)
    rel_l2 = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
    plain = err <= elem * (1.0 + np.abs(r))
    carried = elem * (gv + np.abs(r - res) + ulp_bf16(r)) + ulp_bf16(r) + ulp_bf16(r - res)
    return err, rel_l2, plain, carried


def gated_outside(got_bits, ref_bits, res_bits, gate_vals, elem=1e-2):
    """Mask of the elements (shape of got_bits) outside both the plain and the carried bar of
    gated_tolerance_ok."""
    err, _, plain, carried = _gated_terms(got_bits, ref_bits, res_bits, gate_vals, elem)
    return ~plain & (err > carried)


def rope_elem_bound(out_ref_bits, cos_sin_bits):
    """Derived per-element bound for the RoPE-rotated q/k outputs [R, 56, 3, 128].

    cos_sin_bits [R, 96] holds each row's cache row (cos in [0, 48), sin in [48, 96)).  The
    GEMM accumulates in FP32 (the pages' precision), so v = bf16(acc) may sit one bf16 ulp
    from the oracle's bf16(exact acc).  Through u = bf16(v * r2 * w) that is at most two ulps
    of u (ulp(v) |r2 w| <= 2 ulp(u)), plus one more where u's own rounding flips: |du| <= 3
    ulp(u).  The rotation o_j = bf16(u_j c - u_{j+48} s) carries it as |c| du_j + |s| du_{j+48},
    and o's rounding may flip once more.  So
        |o_gpu - o_ref| <= 3 (|c| ulp(u_j) + |s| ulp(u_{j+48})) + ulp(o_ref)   (j < 48)
    and the same with u_j, u_{j+48} exchanged for o_{j+48}.  u is recovered from the oracle's
    o by the inverse rotation; its magnitude is raised by 2^-6 (the bf16 rounding of o, c and
    s) so that the ulp taken is never below u's own.  Returns the bound for the q/k rotated
    dims and +inf elsewhere (those elements are held to the plain bar only)."""
    o = bf16_val(out_ref_bits)
    cs = bf16_val(cos_sin_bits)
    c = np.abs(cs[:, None, None, :48])
    s = cs[:, None, None, 48:96]
    cc = cs[:, None, None, :48]
    lo, hi = o[:, :, :2, :48], o[:, :, :2, 48:96]
    u_lo = lo * cc + hi * s
    u_hi = hi * cc - lo * s
    grow = 1.0 + 2.0 ** -6
    ul_lo = ulp_bf16(np.abs(u_lo) * grow + 2.0 ** -133)
    ul_hi = ulp_bf16(np.abs(u_hi) * grow + 2.0 ** -133)
    sa = np.abs(s)
    bound = np.full(o.shape, np.inf)
    bound[:, :, :2, :48] = 3.0 * (c * ul_lo + sa * ul_hi) + ulp_bf16(lo)
    bound[:, :, :2, 48:96] = 3.0 * (c * ul_hi + sa * ul_lo) + ulp_bf16(hi)
    return bound


def qkv_check(got_bits, ref_bits, cos_sin_bits, max_rel_l2=2e-3, elem=1e-2, max_relaxed=None):
    """The QKV output bar: relative L2 <= max_rel_l2, and each element within the plain
    elem * (1 + |ref|) or, for a RoPE-rotated q/k element, within rope_elem_bound.  The number of
    elements that need the derived bound is returned and, when max_relaxed is given, must not
    exceed it.  Returns (ok, rel_l2, max|err|, n_relaxed, worst err/bound over relaxed elements)."""
    g = bf16_val(got_bits)
    r = bf16_val(ref_bits)
    err = np.abs(g - r)
    rel_l2 = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
    plain = err <= elem * (1.0 + np.abs(r))
    bound = rope_elem_bound(ref_bits, cos_sin_bits)
    derived = err <= bound
    ok_elem = np.all(plain | derived)
    relaxed = ~plain
    n_relaxed = int(relaxed.sum())
    worst = float((err[relaxed] / bound[relaxed]).max()) if n_relaxed else 0.0
    ok = bool(rel_l2 <= max_rel_l2 and ok_elem and (max_relaxed is None or n_relaxed <= max_relaxed))
    return ok, float(rel_l2), float(err.max() if err.size else 0.0), n_relaxed, worst


def e4m3_half_step(v, s):
    """Half the e4m3 code spacing at |v| / s, in v's units (s the per-row scale): 2^(e-4) s for
    a normal quotient in [2^e, 2^(e+1)), 2^-10 s in the subnormal range (below 2^-6)."""
    q = np.abs(np.asarray(v, np.float64)) / np.where(s > 0, s, 1.0)
    e = np.floor(np.log2(np.maximum(q, 2.0 ** -6)))
    return np.exp2(e - 4) * s


def ulp_bf16(v):
    """Spacing of the bf16 grid at |v| (2^(e-7) for |v| in [2^e, 2^(e+1)); subnormal floor)."""
    v = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -126)))
    return np.exp2(e - 7)


def workspace_ok(got_bits, ref_bits, shift_vals, max_mismatch=1e-3):
    """The AdaLN workspace bar: 1 bf16 ulp at each rounding point of a = bf16(shift + n*s1).

    The GPU's n may sit one bf16 ulp from the oracle's (its sum of squares is FP32, as the
    pages fix); that step reaches a as |s1| * ulp(n) <= 2 ulp(a - shift), which dwarfs ulp(a)
    when shift cancels n*s1.  So each element must satisfy
        |a_gpu - a_ref| <= ulp(a_ref) + 2 ulp(a_ref - shift),
    and at most `max_mismatch` of the elements may differ at all.
    Returns (ok, mismatch fraction, worst ratio err / bound).
    """
    g = bf16_val(got_bits)
    r = bf16_val(ref_bits)
    err = np.abs(g - r)
    bound = ulp_bf16(r) + 2.0 * ulp_bf16(r - shift_vals)
    ratio = float((err / bound).max()) if err.size else 0.0
    mism = float(np.mean(g != r)) if err.size else 0.0
    return bool(np.all(err <= bound) and mism <= max_mismatch), mism, ratio
