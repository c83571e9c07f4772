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


def bf16_tolerance_ok(got_bits, ref_bits, max_rel_l2=2e-3, elem=1e-2, mag=None):
    """The acceptance bar for bf16 outputs: relative L2 error and |err| <= elem*(1+|ref|).

    mag, when given, replaces |ref| as the element's magnitude (same shape as ref)."""
    g = bf16_val(got_bits).ravel()
    r = bf16_val(ref_bits).ravel()
    m = np.abs(r) if mag is None else np.asarray(mag, np.float64).ravel()
    err = np.abs(g - r)
    rel_l2 = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
    ok_elem = np.all(err <= elem * (1.0 + m))
    return bool(rel_l2 <= max_rel_l2 and ok_elem), float(rel_l2), float(err.max() if err.size else 0.0)


def qkv_magnitude(out_ref_bits):
    """Per-element magnitude of packed q/k/v outputs [..., 3, 128] for the elementwise bar.

    RoPE rotates each (j, j+48) pair of q and k (j < 48) and preserves the pair's norm, so a
    rotated element is judged against that norm: a one-ulp difference in a large u_j may land
    in an output that the rotation made small.  V and the pass-through dims use |ref|."""
    r = bf16_val(out_ref_bits)
    mag = np.abs(r).copy()
    pair = np.hypot(r[..., :2, :48], r[..., :2, 48:96])
    mag[..., :2, :48] = pair
    mag[..., :2, 48:96] = pair
    return mag


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
