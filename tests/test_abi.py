"""C-ABI library checks that need no GPU: it loads, exports every declared entry point, and
rejects contract violations before anything is launched.  Also checks that the Python
binding refuses host tensors instead of computing anything on the CPU."""
from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch

import diffusion_transformer_adaln_rmsnorm_amd as dit

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dit.h")

OK, NULL, SHAPE, ALIGN, STRIDE, UNSUP, LAUNCH, VALUE = range(8)
A = 0x7F0000000000          # fake 16-byte aligned device addresses; never dereferenced
MAX_ROWS = 1 << 24          # row limit of the pre-attention and out-projection calls
MAX_S = (2 ** 32 - 1) // 192    # cos/sin cache rows whose byte offsets fit 32 bits
FLT_MIN = 2.0 ** -126


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dit_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("dit_pre_attn_bf16", "dit_pre_attn_bf16_static_ws", "dit_pre_attn_e4m3", "dit_qkv_rope_pack_e4m3", "dit_out_proj_gated_bf16",
              "dit_mlp_fp8", "dit_mlp_fp8_flags_elems", "dit_status_string", "dit_abi_version",
              "dit_mx_scale_bytes", "dit_mx_quant_fp4", "dit_out_proj_gated_mxfp4", "dit_pre_attn_mxfp4"):
        assert n in names


def test_header_states_the_limits_the_library_checks():
    src = open(HEADER).read()
    assert re.search(r"#define DIT_MAX_ROWS 16777216\b", src)
    assert re.search(r"#define DIT_MAX_ROPE_ROWS %d\b" % MAX_S, src)


def test_library_exports_every_declared_symbol():
    L = dit.load_library()
    for n in _declared():
        assert hasattr(L, n), n
    assert L.dit_abi_version() == 100
    assert L.dit_status_string(ALIGN) == b"pointer not aligned"
    assert L.dit_mlp_fp8_flags_elems(32760) == 0


def _T(ptr=A + 0x100000, rows=2, stride=6 * 5376):
    return dit.Table(ptr, rows, stride)


def _p(k):
    return ctypes.c_void_p(A + k * 0x1000000)


def pre(**kw):
    a = dict(x=_p(1), M=16, xw=_p(2), sc=_T(), sh=_T(A + 0x200000), idx=_p(3), W=_p(4), qw=_p(5), kw=_p(6),
             cs=_p(7), S=16, pos=None, P=1, eps=1e-5, qk_eps=1e-5, ws=_p(8), out=_p(9))
    a.update(kw)
    return dit.load_library().dit_pre_attn_bf16(a["x"], a["M"], a["xw"], a["sc"], a["sh"], a["idx"], a["W"],
                                                  a["qw"], a["kw"], a["cs"], a["S"], a["pos"], a["P"], a["eps"],
                                                  a["qk_eps"], a["ws"], a["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), NULL), (dict(ws=None), NULL), (dict(out=None), NULL), (dict(idx=None), NULL),
    (dict(sc=_T(ptr=0)), NULL),
    (dict(x=ctypes.c_void_p(A + 8)), ALIGN), (dict(out=ctypes.c_void_p(A + 2)), ALIGN),
    (dict(idx=ctypes.c_void_p(A + 4)), ALIGN), (dict(pos=ctypes.c_void_p(A + 4)), ALIGN),
    (dict(sc=_T(ptr=A + 8)), ALIGN),
    (dict(sc=_T(stride=5375 + 1 + 4)), STRIDE), (dict(sh=_T(stride=5368)), STRIDE),
    (dict(sc=_T(rows=0)), SHAPE), (dict(sc=_T(rows=3)), SHAPE),
    (dict(M=-1), SHAPE), (dict(M=1 << 40), SHAPE), (dict(S=0), SHAPE), (dict(S=15), SHAPE),
    (dict(P=2, M=0), OK), (dict(P=8, M=0), OK), (dict(P=3), VALUE), (dict(P=0), VALUE), (dict(P=16), VALUE),
    (dict(eps=0.0), VALUE), (dict(eps=-1e-5), VALUE), (dict(qk_eps=float("nan")), VALUE),
    (dict(eps=float("inf")), VALUE),
    (dict(M=0), OK),
    (dict(M=MAX_ROWS + 1, S=MAX_ROWS + 1), SHAPE), (dict(M=0, S=MAX_S), OK), (dict(M=0, S=MAX_S + 1), SHAPE),
    (dict(S=MAX_S + 1), SHAPE), (dict(S=1 << 40, pos=_p(10)), SHAPE),
])
def test_pre_attn_contract_checks(kw, status):
    assert pre(**kw) == status


def pre_static(**kw):
    a = dict(x=_p(1), M=16, xw=_p(2), sc=_T(), sh=_T(A + 0x200000), idx=_p(3), W=_p(4), qw=_p(5), kw=_p(6),
             cs=_p(7), S=16, pos=None, P=1, eps=1e-5, qk_eps=1e-5, out=_p(9))
    a.update(kw)
    return dit.load_library().dit_pre_attn_bf16_static_ws(a["x"], a["M"], a["xw"], a["sc"], a["sh"], a["idx"],
                                                            a["W"], a["qw"], a["kw"], a["cs"], a["S"], a["pos"],
                                                            a["P"], a["eps"], a["qk_eps"], a["out"], None)


# every check runs before the device is touched (these need no GPU): M beyond the static
# workspace, and each argument the allocating form checks
@pytest.mark.parametrize("kw,status", [
    (dict(M=4097, S=4097), SHAPE), (dict(M=-1), SHAPE), (dict(M=1 << 40), SHAPE), (dict(M=0), OK),
    (dict(x=None), NULL), (dict(out=None), NULL), (dict(idx=None), NULL),
    (dict(out=ctypes.c_void_p(A + 8)), ALIGN), (dict(sc=_T(rows=3)), SHAPE), (dict(S=15), SHAPE),
    (dict(M=4096, S=4095), SHAPE), (dict(S=MAX_S + 1), SHAPE), (dict(P=3), VALUE), (dict(eps=0.0), VALUE),
    (dict(M=0, S=1, pos=_p(10)), OK),
])
def test_pre_attn_static_ws_contract_checks(kw, status):
    assert pre_static(**kw) == status


def test_static_ws_limit_matches_the_header():
    assert re.search(r"#define DIT_STATIC_WS_MAX_ROWS %d\b" % dit.STATIC_WS_MAX_ROWS, open(HEADER).read())


def pre8(**kw):
    a = dict(x=_p(1), M=16, xw=_p(2), sc=_T(), sh=_T(A + 0x200000), idx=_p(3), W=_p(4), qw=_p(5), kw=_p(6),
             cs=_p(7), S=16, pos=None, P=1, eps=1e-5, qk_eps=1e-5, dq=0.5, dk=0.25, dv=2.0, ws=_p(8), out=_p(9))
    a.update(kw)
    return dit.load_library().dit_pre_attn_e4m3(a["x"], a["M"], a["xw"], a["sc"], a["sh"], a["idx"], a["W"],
                                                  a["qw"], a["kw"], a["cs"], a["S"], a["pos"], a["P"], a["eps"],
                                                  a["qk_eps"], a["dq"], a["dk"], a["dv"], a["ws"], a["out"], None)


def pack8(**kw):
    a = dict(ws=_p(8), M=16, W=_p(4), qw=_p(5), kw=_p(6), cs=_p(7), S=16, pos=None, P=1, qk_eps=1e-5, dq=0.5,
             dk=0.25, dv=2.0, out=_p(9))
    a.update(kw)
    return dit.load_library().dit_qkv_rope_pack_e4m3(a["ws"], a["M"], a["W"], a["qw"], a["kw"], a["cs"], a["S"],
                                                       a["pos"], a["P"], a["qk_eps"], a["dq"], a["dk"], a["dv"],
                                                       a["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dq=0.0), VALUE), (dict(dk=-1.0), VALUE), (dict(dv=float("nan")), VALUE), (dict(dq=float("inf")), VALUE),
    (dict(out=None), NULL), (dict(x=None), NULL), (dict(out=ctypes.c_void_p(A + 8)), ALIGN),
    (dict(P=3), VALUE), (dict(S=15), SHAPE), (dict(M=-1), SHAPE),
    (dict(M=0), OK), (dict(M=0, P=4), OK),
    # a descale must have a finite reciprocal: normal floats only
    (dict(dq=1e-39), VALUE), (dict(dk=2.0 ** -130), VALUE), (dict(dv=FLT_MIN / 2), VALUE),
    (dict(M=0, dq=FLT_MIN, dk=FLT_MIN, dv=FLT_MIN), OK), (dict(M=0, S=MAX_S + 1), SHAPE),
])
def test_pre_attn_e4m3_contract_checks(kw, status):
    assert pre8(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(dq=0.0), VALUE), (dict(dv=-2.0), VALUE), (dict(dk=float("nan")), VALUE),
    (dict(out=None), NULL), (dict(ws=None), NULL), (dict(out=ctypes.c_void_p(A + 4)), ALIGN),
    (dict(P=5), VALUE), (dict(qk_eps=0.0), VALUE), (dict(M=0), OK),
    (dict(dk=1e-40), VALUE), (dict(M=0, dq=FLT_MIN), OK), (dict(S=MAX_S + 1), SHAPE),
    (dict(M=MAX_ROWS + 1, S=MAX_ROWS + 1), SHAPE),
])
def test_qkv_rope_pack_e4m3_contract_checks(kw, status):
    assert pack8(**kw) == status


def test_pre_attn_positions_lift_the_S_ge_M_rule():
    # with explicit positions S may be smaller than M; M = 0 keeps the call a no-op
    assert pre(M=0, S=1, pos=_p(10)) == OK


def outp(**kw):
    a = dict(attn=_p(1), M=8, Wo=_p(2), gate=_T(rows=9, stride=5376), gi=_p(3), res=_p(4), out=_p(5))
    a.update(kw)
    return dit.load_library().dit_out_proj_gated_bf16(a["attn"], a["M"], a["Wo"], a["gate"], a["gi"], a["res"],
                                                        a["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(attn=None), NULL), (dict(gi=None), NULL), (dict(res=None), NULL), (dict(out=None), NULL),
    (dict(attn=ctypes.c_void_p(A + 4)), ALIGN), (dict(gi=ctypes.c_void_p(A + 2)), ALIGN),
    (dict(gate=_T(rows=0, stride=5376)), SHAPE), (dict(gate=_T(rows=9, stride=5380)), STRIDE),
    (dict(gate=_T(rows=1 << 31, stride=5376)), SHAPE),
    (dict(M=-3), SHAPE), (dict(M=0), OK), (dict(M=MAX_ROWS + 1), SHAPE),
])
def test_out_proj_contract_checks(kw, status):
    assert outp(**kw) == status


def test_mx_scale_bytes():
    L = dit.load_library()
    # rows padded to 128, one byte per 32 values
    assert L.dit_mx_scale_bytes(1, 256) == 128 * 8
    assert L.dit_mx_scale_bytes(128, 7168) == 128 * 224
    assert L.dit_mx_scale_bytes(129, 7168) == 256 * 224
    assert L.dit_mx_scale_bytes(32760, 7168) == 32768 * 224
    assert L.dit_mx_scale_bytes(0, 7168) == 0 and L.dit_mx_scale_bytes(-1, 7168) == 0


def mxq(**kw):
    a = dict(x=_p(1), R=8, K=7168, codes=_p(2), scales=_p(3))
    a.update(kw)
    return dit.load_library().dit_mx_quant_fp4(a["x"], a["R"], a["K"], a["codes"], a["scales"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=7000), SHAPE), (dict(K=128), SHAPE), (dict(K=0), SHAPE), (dict(R=-1), SHAPE),
    (dict(R=(1 << 31) // 224 + 1), SHAPE),
    (dict(x=None), NULL), (dict(codes=None), NULL), (dict(scales=None), NULL),
    (dict(x=ctypes.c_void_p(A + 2)), ALIGN), (dict(codes=ctypes.c_void_p(A + 8)), ALIGN),
    (dict(R=0), OK),
])
def test_mx_quant_contract_checks(kw, status):
    assert mxq(**kw) == status


def outp_mx(**kw):
    a = dict(attn=_p(1), M=8, wc=_p(2), ws=_p(3), gate=_T(rows=9, stride=5376), gi=_p(4), res=_p(5), ac=_p(6),
             as_=_p(7), out=_p(8))
    a.update(kw)
    return dit.load_library().dit_out_proj_gated_mxfp4(a["attn"], a["M"], a["wc"], a["ws"], a["gate"], a["gi"],
                                                         a["res"], a["ac"], a["as_"], a["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(attn=None), NULL), (dict(wc=None), NULL), (dict(ws=None), NULL), (dict(ac=None), NULL),
    (dict(as_=None), NULL), (dict(out=None), NULL),
    (dict(ws=ctypes.c_void_p(A + 4)), ALIGN), (dict(as_=ctypes.c_void_p(A + 4)), ALIGN),
    (dict(gi=ctypes.c_void_p(A + 2)), ALIGN),
    (dict(gate=_T(rows=0, stride=5376)), SHAPE), (dict(gate=_T(rows=9, stride=5380)), STRIDE),
    (dict(M=-3), SHAPE), (dict(M=(1 << 24) + 1), SHAPE), (dict(M=0), OK),
])
def test_out_proj_mxfp4_contract_checks(kw, status):
    assert outp_mx(**kw) == status


def pre_mx(**kw):
    a = dict(x=_p(1), M=16, xw=_p(2), sc=_T(), sh=_T(A + 0x200000), idx=_p(3), wc=_p(4), ws=_p(5), qw=_p(6),
             kw=_p(7), cs=_p(8), S=16, pos=None, P=1, eps=1e-5, qk_eps=1e-5, wsc=_p(9), wss=_p(10), out=_p(11))
    a.update(kw)
    return dit.load_library().dit_pre_attn_mxfp4(a["x"], a["M"], a["xw"], a["sc"], a["sh"], a["idx"], a["wc"],
                                                   a["ws"], a["qw"], a["kw"], a["cs"], a["S"], a["pos"], a["P"],
                                                   a["eps"], a["qk_eps"], a["wsc"], a["wss"], a["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(P=3), VALUE), (dict(eps=0.0), VALUE), (dict(qk_eps=float("nan")), VALUE),
    (dict(x=None), NULL), (dict(wc=None), NULL), (dict(ws=None), NULL), (dict(wsc=None), NULL),
    (dict(wss=None), NULL), (dict(out=None), NULL),
    (dict(ws=ctypes.c_void_p(A + 4)), ALIGN), (dict(wss=ctypes.c_void_p(A + 8)), ALIGN),
    (dict(pos=ctypes.c_void_p(A + 4)), ALIGN),
    (dict(S=8), SHAPE), (dict(sh=_T(rows=3)), SHAPE), (dict(M=-1), SHAPE),
    (dict(M=0), OK), (dict(S=MAX_S + 1), SHAPE), (dict(M=0, S=MAX_S), OK),
    (dict(M=MAX_ROWS + 1, S=MAX_ROWS + 1), SHAPE),
])
def test_pre_attn_mxfp4_contract_checks(kw, status):
    assert pre_mx(**kw) == status


def mlp(**kw):
    a = dict(x=_p(1), M=8, xw=_p(2), sc=_T(), sh=_T(A + 0x200000), g=_T(A + 0x300000), idx=_p(3), res=_p(4),
             w1=_p(5), s1=_p(6), w2=_p(7), s2=_p(8), eps=1e-5, aq=_p(9), as_=_p(10), y=_p(11), yq=_p(12), ys=_p(13),
             flags=None, out=_p(14))
    a.update(kw)
    return dit.load_library().dit_mlp_fp8(a["x"], a["M"], a["xw"], a["sc"], a["sh"], a["g"], a["idx"], a["res"],
                                          a["w1"], a["s1"], a["w2"], a["s2"], a["eps"], a["aq"], a["as_"], a["y"],
                                          a["yq"], a["ys"], a["flags"], a["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=0), SHAPE), (dict(M=149797), SHAPE), (dict(M=-1), SHAPE),
    (dict(eps=0.0), VALUE), (dict(eps=float("nan")), VALUE),
    (dict(x=None), NULL), (dict(y=None), NULL), (dict(ys=None), NULL), (dict(g=_T(ptr=0)), NULL),
    (dict(g=_T(rows=3)), SHAPE), (dict(sh=_T(stride=5376 * 7)), STRIDE),
    (dict(aq=ctypes.c_void_p(A + 8)), ALIGN), (dict(s1=ctypes.c_void_p(A + 2)), ALIGN),
])
def test_mlp_contract_checks(kw, status):
    assert mlp(**kw) == status


def test_binding_refuses_host_tensors():
    x = torch.zeros(4, dit.HIDDEN, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        dit.dit_out_proj_gated_bf16(torch.zeros(4, dit.ATTN_WIDTH, dtype=torch.bfloat16),
                                    torch.zeros(dit.HIDDEN, dit.ATTN_WIDTH, dtype=torch.bfloat16),
                                    torch.zeros(9, dit.HIDDEN, dtype=torch.bfloat16),
                                    torch.zeros(4, dtype=torch.int32), x)
    with pytest.raises(ValueError, match="GPU"):
        dit.dit_mx_quant_fp4(torch.zeros(4, dit.ATTN_WIDTH, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="GPU"):
        dit.dit_pre_attn_bf16(x, torch.zeros(dit.HIDDEN, dtype=torch.bfloat16), x[:1], x[:1],
                              torch.zeros(4, dtype=torch.int64), None, None, None, None, ulysses_degree=1, out=None)
