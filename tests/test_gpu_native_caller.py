"""The C ABI from a plain C program (tests/native/pre_attn_caller.c, built by
__graft_entry__.build()): the same bf16 pre-attention problem through the C caller, on a stream
of its own, and through the Python binding must give the same bits, and the C caller's error
paths must report their status without launching."""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest
import torch

import synth
from tests.native.build import BINARY

pytestmark = pytest.mark.gpu

H = synth.HIDDEN


def test_c_caller_matches_the_python_binding(tmp_path):
    assert os.path.exists(BINARY), "the C caller is built by __graft_entry__.build()"
    import diffusion_transformer_adaln_rmsnorm_amd as dit
    M, rows = 300, 2
    d = synth.pre_attn_inputs(M, seed=707, rows=rows, wide_tables=False, S=M, positions="identity",
                              bad_index_frac=0.02)
    assert d.get("rope_positions") is None
    files = {"x.bin": d["x"].reshape(M, H), "xw.bin": d["x_norm_weight"], "scale.bin": d["adaln_scale"].dense(),
             "shift.bin": d["adaln_shift"].dense(), "idx.bin": d["adaln_index"].astype(np.int64),
             "w.bin": d["qkv_weight"].reshape(synth.QKV_ROWS, H), "qw.bin": d["q_norm_weight"],
             "kw.bin": d["k_norm_weight"], "cs.bin": d["rope_cos_sin"].reshape(d["S"], 96)}
    for name, arr in files.items():
        np.ascontiguousarray(arr).tofile(tmp_path / name)
    eps, qk_eps = float(np.float32(d["eps"])), float(np.float32(d["qk_eps"] if d.get("qk_eps") is not None
                                                                 else d["eps"]))
    (tmp_path / "meta.txt").write_text(f"{M} {rows} {d['S']} {eps!r} {qk_eps!r}\n")
    print(f"[native] C caller, pre_attn M={M}", flush=True)
    r = subprocess.run([BINARY, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)
    ws_c = np.fromfile(tmp_path / "ws.bin", np.uint16).reshape(M, H)
    out_c = np.fromfile(tmp_path / "out.bin", np.uint16).reshape(1, M, 56, 3, 128)

    t = synth.to_torch("pre_attn", d)
    ws = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((1, M, 56, 3, 128), dtype=torch.bfloat16, device="cuda")
    dit.dit_pre_attn_bf16(t["x"], t["x_norm_weight"], t["adaln_scale"], t["adaln_shift"], t["adaln_index"],
                          t["qkv_weight"], t["q_norm_weight"], t["k_norm_weight"], t["rope_cos_sin"],
                          ulysses_degree=1, out=out, eps=eps, qk_eps=qk_eps, rope_positions=None, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(ws_c, synth.bits(ws)), "workspace: C caller != binding"
    assert np.array_equal(out_c, synth.bits(out)), "out: C caller != binding"
    bad = (d["adaln_index"] < 0) | (d["adaln_index"] >= rows)
    assert bad.any() and np.all(ws_c[bad] == 0)
