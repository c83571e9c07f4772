"""The no-allocation pre-attention entry point (dit_pre_attn_bf16_static_ws) against the
allocating one (dit_pre_attn_bf16) through the C ABI: the same kernels on the same inputs, so
the outputs must be equal bit for bit, on two calls in a row with the second one smaller (the
static workspace then still holds the first call's rows past M).  A few rows are also checked
against the oracle with the pre-attention bar."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import qkv_check

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[no-alloc] {msg}", file=sys.stderr, flush=True)


def _call(fn, t, P, out):
    return fn(t["x"], t["x_norm_weight"], t["adaln_scale"], t["adaln_shift"], t["adaln_index"], t["qkv_weight"],
              t["q_norm_weight"], t["k_norm_weight"], t["rope_cos_sin"], ulysses_degree=P, out=out, eps=t["eps"],
              qk_eps=t["qk_eps"], rope_positions=t["rope_positions"])


def test_static_workspace_matches_the_allocating_entry_point():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import diffusion_transformer_adaln_rmsnorm_amd as dit
    dit.load_library()
    assert dit.STATIC_WS_MAX_ROWS == 4096
    W = synth.to_bf16_bits(synth.normal(3, "qkv_weight", (synth.QKV_ROWS, synth.HIDDEN), 1 / np.sqrt(synth.HIDDEN)))
    for M, P, seed in ((4096, 1, 810), (300, 2, 811)):
        _say(f"M={M} P={P}")
        d = synth.pre_attn_inputs(M, seed=seed, rows=2, S=512, positions="random", n_bad_positions=4,
                                  bad_index_frac=0.02, weight=W)
        t = synth.to_torch("pre_attn", d)
        shape = (P, M, 56 // P, 3, 128)
        out_s = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        out_a = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        _call(dit.dit_pre_attn_bf16_static_ws, t, P, out_s)
        _call(dit.dit_pre_attn_bf16, t, P, out_a)
        torch.cuda.synchronize()
        assert torch.equal(out_s.view(torch.int16), out_a.view(torch.int16)), f"M={M}: outputs differ"
        rows = np.unique(np.r_[np.arange(4), np.arange(M - 4, M)])
        _, ref = oracle.pre_attn(d, rows_sel=rows)
        got = np.concatenate(list(synth.bits(out_s)), axis=1)[rows]
        cs = d["rope_cos_sin"][np.clip(d["rope_positions"][rows], 0, d["S"] - 1)]
        ok, rel, mx, n_rel, worst = qkv_check(got, ref, cs, max_relaxed=4)
        _say(f"  bit-equal to the allocating call; oracle rows relL2={rel:.2e} max|err|={mx:.3e}")
        assert ok, (rel, mx, n_rel, worst)
    with pytest.raises(dit.DitError, match="SHAPE"):
        M = 4097
        d = synth.pre_attn_inputs(M, seed=812, rows=2, S=M, positions="identity", weight=W)
        t = synth.to_torch("pre_attn", d)
        _call(dit.dit_pre_attn_bf16_static_ws, t, 1, torch.empty((1, M, 56, 3, 128), dtype=torch.bfloat16,
                                                                   device="cuda"))
