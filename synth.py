"""Seeded synthetic inputs for the MiniMax-H3 AdaLN projection stages.

This module only draws random tensors and encodes them in the storage formats the
operations take (bf16 bit patterns, float8_e4m3fn codes, int64/int32 indices).  It holds
none of the stages' arithmetic: encodings go through torch's CPU dtype conversions (a
library routine), and everything the stages compute is left to the oracle and the HIP path,
which both receive the same arrays from here.

Shapes and distributions follow the workloads described on the FlashInfer MiniMax-H3
diffusion_ops pages (bf16 pre-attention, nvfp4 out-proj, fp8 MLP):
hidden 5376, 56 heads x 128, QKV rows 21504 in [q_all | k_all | v_all] order, an
[S, 96] cos/sin cache, MLP intermediate 14336 (FC1 output 28672 = gate | up).

Random draws use numpy PCG64 streams spawned from one SeedSequence per (seed, tensor
name), filled in fixed 4 Mi-element chunks on a thread pool, so the bits depend only on the
seed, never on the thread count.
"""
from __future__ import annotations

import hashlib
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

HIDDEN = 5376
HEADS = 56
HEAD_DIM = 128
QKV_ROWS = 3 * HEADS * HEAD_DIM          # 21504
ATTN_WIDTH = HEADS * HEAD_DIM            # 7168
ROT_DIMS = 96
N_FREQ = 48
INTER = 14336
FC1_ROWS = 2 * INTER                     # 28672
ADALN_CHUNKS = 6
GATE_ROWS_OUTPROJ = 9
BASE_SEED = 20261202

_CHUNK = 1 << 22


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _stream_seed(seed: int, name: str) -> np.random.SeedSequence:
    h = int.from_bytes(hashlib.sha256(name.encode()).digest()[:8], "little")
    return np.random.SeedSequence([seed & 0xFFFFFFFF, h & 0xFFFFFFFF, h >> 32])


def normal(seed: int, name: str, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """float32 N(mean, std^2) of the given shape, reproducible from (seed, name)."""
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    nch = max(1, (n + _CHUNK - 1) // _CHUNK)
    seqs = _stream_seed(seed, name).spawn(nch)

    def fill(i):
        sl = out[i * _CHUNK:(i + 1) * _CHUNK]
        np.random.Generator(np.random.PCG64(seqs[i])).standard_normal(sl.shape[0], dtype=np.float32, out=sl)
        if std != 1.0:
            sl *= np.float32(std)
        if mean != 0.0:
            sl += np.float32(mean)

    if nch == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nch)))
    return out.reshape(shape)


def rng(seed: int, name: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(_stream_seed(seed, name)))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Encode float32 values as bf16 bit patterns (uint16), round-to-nearest-even (torch)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_e4m3_codes(a: np.ndarray) -> np.ndarray:
    """Encode float32 values (already within +-448) as float8_e4m3fn codes (uint8), via torch."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def e4m3_codes_to_f32(c: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(c, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float32).numpy()


def quantize_weight_rows_e4m3(w: np.ndarray):
    """Per-output-row e4m3 weight encoding used to make synthetic FP8 weights.

    The pages take FP8 weights from preparation helpers whose pages are missing; this
    stand-in scales each row by amax/448 (fp32) and encodes the quotient with torch's
    float8_e4m3fn conversion.  It only shapes the inputs.
    """
    w = np.ascontiguousarray(w, np.float32)
    amax = np.abs(w).max(axis=1)
    s = (amax / np.float32(448.0)).astype(np.float32)
    s[s == 0] = np.float32(1.0)
    q = np.empty(w.shape, np.uint8)
    step = 2048
    for r0 in range(0, w.shape[0], step):
        blk = w[r0:r0 + step] / s[r0:r0 + step, None]
        np.clip(blk, -448.0, 448.0, out=blk)
        q[r0:r0 + step] = to_e4m3_codes(blk)
    return q, s


class Table:
    """A [rows, 5376] view into a wider bf16 matrix: base array, element offset, row stride."""

    def __init__(self, base: np.ndarray, offset: int, rows: int, row_stride: int, cols: int = HIDDEN):
        self.base = base          # flat uint16 array owning the storage
        self.offset = offset
        self.rows = rows
        self.row_stride = row_stride
        self.cols = cols

    def dense(self) -> np.ndarray:
        """The table as a contiguous [rows, cols] uint16 copy (for inspection)."""
        out = np.empty((self.rows, self.cols), np.uint16)
        for r in range(self.rows):
            s = self.offset + r * self.row_stride
            out[r] = self.base[s:s + self.cols]
        return out


def _guarded_indices(g: np.random.Generator, M: int, rows: int, frac: float, bad_values):
    idx = g.integers(0, rows, size=M, dtype=np.int64)
    nbad = int(round(frac * M))
    if nbad > 0 and M > 0:
        where = g.choice(M, size=min(nbad, M), replace=False)
        bad = np.asarray(bad_values, np.int64)
        idx[where] = bad[np.arange(where.size) % bad.size]
    return idx


def rope_cache(seed: int, S: int) -> np.ndarray:
    """[S, 96] bf16 cache: columns [0,48) cos(theta), [48,96) sin(theta), theta ~ U[0, 2pi)."""
    theta = rng(seed, "rope_theta").uniform(0.0, 2.0 * math.pi, size=(S, N_FREQ))
    cs = np.concatenate([np.cos(theta), np.sin(theta)], axis=1).astype(np.float32)
    return to_bf16_bits(cs)


def pre_attn_inputs(M: int, *, seed: int, rows: int = 2, wide_tables: bool = True,
                    S: int | None = None, positions: str = "identity", bad_index_frac: float = 0.005,
                    bad_index_values=(-1, 2, 1 << 32, -(1 << 32)), n_bad_positions: int = 8,
                    weight: np.ndarray | None = None):
    """Inputs of the bf16 pre-attention stage.

    positions: "identity" (None, S >= M) or "random" (uniform in [0,S) plus out-of-range
    values for the clamp).  wide_tables: tables are column chunks of a [rows, 6*5376]
    modulation matrix (shift = chunk 0, scale = chunk 1), else two [rows, 5376] tables.
    """
    if S is None:
        S = max(M, 1)
    d = {"M": M, "rows": rows, "S": S, "seed": seed}
    d["x"] = to_bf16_bits(normal(seed, "x", (M, HIDDEN)))
    d["x_norm_weight"] = to_bf16_bits(normal(seed, "x_norm_weight", (HIDDEN,), 0.1, 1.0))
    if wide_tables:
        mod = to_bf16_bits(normal(seed, "modulation", (rows, ADALN_CHUNKS * HIDDEN), 0.1)).reshape(-1)
        ld = ADALN_CHUNKS * HIDDEN
        d["adaln_shift"] = Table(mod, 0 * HIDDEN, rows, ld)
        d["adaln_scale"] = Table(mod, 1 * HIDDEN, rows, ld)
    else:
        sc = to_bf16_bits(normal(seed, "adaln_scale", (rows, HIDDEN), 0.1)).reshape(-1)
        sh = to_bf16_bits(normal(seed, "adaln_shift", (rows, HIDDEN), 0.1)).reshape(-1)
        d["adaln_scale"] = Table(sc, 0, rows, HIDDEN)
        d["adaln_shift"] = Table(sh, 0, rows, HIDDEN)
    g = rng(seed, "adaln_index")
    d["adaln_index"] = _guarded_indices(g, M, rows, bad_index_frac, bad_index_values)
    if weight is None:
        weight = to_bf16_bits(normal(seed, "qkv_weight", (QKV_ROWS, HIDDEN), 1.0 / math.sqrt(HIDDEN)))
    d["qkv_weight"] = weight
    d["q_norm_weight"] = to_bf16_bits(normal(seed, "q_norm_weight", (HEAD_DIM,), 0.1, 1.0))
    d["k_norm_weight"] = to_bf16_bits(normal(seed, "k_norm_weight", (HEAD_DIM,), 0.1, 1.0))
    d["rope_cos_sin"] = rope_cache(seed, S)
    if positions == "identity":
        d["rope_positions"] = None
    else:
        gp = rng(seed, "rope_positions")
        pos = gp.integers(0, S, size=M, dtype=np.int64)
        nb = min(n_bad_positions, M)
        if nb:
            where = gp.choice(M, size=nb, replace=False)
            bad = np.array([-1, S, -(1 << 40), S + 12345, -7, 1 << 62, -(1 << 62), 2 * S], np.int64)
            pos[where] = bad[np.arange(nb) % bad.size]
        d["rope_positions"] = pos
    d["eps"] = 1e-5
    d["qk_eps"] = 1e-5
    return d


def out_proj_inputs(M: int, *, seed: int, gate_rows: int = GATE_ROWS_OUTPROJ, weight: np.ndarray | None = None):
    d = {"M": M, "seed": seed}
    d["attn_out"] = to_bf16_bits(normal(seed, "attn_out", (M, ATTN_WIDTH)))
    if weight is None:
        weight = to_bf16_bits(normal(seed, "o_weight", (HIDDEN, ATTN_WIDTH), 1.0 / math.sqrt(ATTN_WIDTH)))
    d["o_weight"] = weight
    gate = to_bf16_bits(normal(seed, "gate", (gate_rows, HIDDEN), 0.5)).reshape(-1)
    d["gate"] = Table(gate, 0, gate_rows, HIDDEN)
    d["gate_index"] = rng(seed, "gate_index").integers(-1, 11, size=M, dtype=np.int64).astype(np.int32)
    d["residual"] = to_bf16_bits(normal(seed, "residual", (M, HIDDEN)))
    return d


def mlp_weights(seed: int):
    w1 = normal(seed, "fc1_weight", (FC1_ROWS, HIDDEN), 1.0 / math.sqrt(HIDDEN))
    q1, s1 = quantize_weight_rows_e4m3(w1)
    del w1
    w2 = normal(seed, "fc2_weight", (HIDDEN, INTER), 1.0 / math.sqrt(INTER))
    q2, s2 = quantize_weight_rows_e4m3(w2)
    return q1, s1, q2, s2


def mlp_inputs(M: int, *, seed: int, rows: int = 2, weights=None, bad_index_frac: float = 0.005,
               bad_index_values=(-1, 2, 1 << 32, -(1 << 32))):
    d = {"M": M, "rows": rows, "seed": seed}
    d["x"] = to_bf16_bits(normal(seed, "x", (M, HIDDEN)))
    d["x_norm_weight"] = to_bf16_bits(normal(seed, "x_norm_weight", (HIDDEN,), 0.1, 1.0))
    mod = to_bf16_bits(normal(seed, "modulation", (rows, ADALN_CHUNKS * HIDDEN), 0.1)).reshape(-1)
    ld = ADALN_CHUNKS * HIDDEN
    d["adaln_shift"] = Table(mod, 3 * HIDDEN, rows, ld)
    d["adaln_scale"] = Table(mod, 4 * HIDDEN, rows, ld)
    d["gate"] = Table(mod, 5 * HIDDEN, rows, ld)
    d["adaln_index"] = _guarded_indices(rng(seed, "adaln_index"), M, rows, bad_index_frac, bad_index_values)
    d["residual"] = to_bf16_bits(normal(seed, "residual", (M, HIDDEN)))
    if weights is None:
        weights = mlp_weights(seed)
    d["fc1_q"], d["fc1_scale"], d["fc2_q"], d["fc2_scale"] = weights
    d["eps"] = 1e-5
    return d


# The five workloads: config id -> (kind, builder).  Seeds are BASE_SEED + config id.
def config(cid: int, M: int | None = None, **kw):
    seed = BASE_SEED + cid
    if cid == 0:
        M = 16 if M is None else M
        d = pre_attn_inputs(M, seed=seed, rows=4, wide_tables=False, S=max(M, 16), positions="identity",
                            bad_index_frac=0.0, **kw)
        # two guarded entries: -1 and rows (= 4)
        if M >= 2:
            d["adaln_index"][3 % M] = -1
            d["adaln_index"][(11 % M) if M > 11 else M - 1] = 4
        return "pre_attn", d
    if cid == 1:
        M = 4096 if M is None else M
        return "pre_attn", pre_attn_inputs(M, seed=seed, rows=2, S=8192, positions="random", **kw)
    if cid == 2:
        M = 32760 if M is None else M
        return "pre_attn", pre_attn_inputs(M, seed=seed, rows=2, S=M, positions="identity", **kw)
    if cid == 3:
        M = 32760 if M is None else M
        return "out_proj", out_proj_inputs(M, seed=seed, **kw)
    if cid == 4:
        M = 32760 if M is None else M
        return "mlp", mlp_inputs(M, seed=seed, **kw)
    raise ValueError(f"unknown config {cid}")


# ---------------------------------------------------------------- device upload (no arithmetic)

def _t_bf16(a, device):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def _t_e4m3(a, device):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).view(torch.float8_e4m3fn).to(device)


def _t_table(t: Table, device, cache):
    key = id(t.base)
    if key not in cache:
        cache[key] = _t_bf16(t.base, device)
    base = cache[key]
    return base.as_strided((t.rows, t.cols), (t.row_stride, 1), t.offset)


def to_torch(kind: str, d: dict, device="cuda"):
    """The arrays of a synthetic input dict as torch tensors on `device` (bit copies)."""
    cache = {}
    M = d["M"]
    o = {"M": M}
    if kind == "pre_attn":
        o["x"] = _t_bf16(d["x"].reshape(M, HIDDEN), device)
        o["x_norm_weight"] = _t_bf16(d["x_norm_weight"], device)
        o["adaln_scale"] = _t_table(d["adaln_scale"], device, cache)
        o["adaln_shift"] = _t_table(d["adaln_shift"], device, cache)
        o["adaln_index"] = torch.from_numpy(np.ascontiguousarray(d["adaln_index"], np.int64)).to(device)
        o["qkv_weight"] = _t_bf16(d["qkv_weight"].reshape(QKV_ROWS, HIDDEN), device)
        o["q_norm_weight"] = _t_bf16(d["q_norm_weight"], device)
        o["k_norm_weight"] = _t_bf16(d["k_norm_weight"], device)
        o["rope_cos_sin"] = _t_bf16(d["rope_cos_sin"].reshape(-1, ROT_DIMS), device)
        pos = d.get("rope_positions")
        o["rope_positions"] = None if pos is None else torch.from_numpy(np.ascontiguousarray(pos, np.int64)).to(device)
        o["eps"] = d["eps"]
        o["qk_eps"] = d.get("qk_eps")
    elif kind == "out_proj":
        o["attn_out"] = _t_bf16(d["attn_out"].reshape(M, ATTN_WIDTH), device)
        o["o_weight"] = _t_bf16(d["o_weight"].reshape(HIDDEN, ATTN_WIDTH), device)
        o["gate"] = _t_table(d["gate"], device, cache)
        o["gate_index"] = torch.from_numpy(np.ascontiguousarray(d["gate_index"], np.int32)).to(device)
        o["residual"] = _t_bf16(d["residual"].reshape(M, HIDDEN), device)
    elif kind == "mlp":
        o["x"] = _t_bf16(d["x"].reshape(M, HIDDEN), device)
        o["x_norm_weight"] = _t_bf16(d["x_norm_weight"], device)
        o["adaln_scale"] = _t_table(d["adaln_scale"], device, cache)
        o["adaln_shift"] = _t_table(d["adaln_shift"], device, cache)
        o["gate"] = _t_table(d["gate"], device, cache)
        o["adaln_index"] = torch.from_numpy(np.ascontiguousarray(d["adaln_index"], np.int64)).to(device)
        o["residual"] = _t_bf16(d["residual"].reshape(M, HIDDEN), device)
        o["fc1_weight_q"] = _t_e4m3(d["fc1_q"], device)
        o["fc1_weight_scale"] = torch.from_numpy(np.ascontiguousarray(d["fc1_scale"], np.float32)).to(device)
        o["fc2_weight_q"] = _t_e4m3(d["fc2_q"], device)
        o["fc2_weight_scale"] = torch.from_numpy(np.ascontiguousarray(d["fc2_scale"], np.float32)).to(device)
        o["eps"] = d["eps"]
    else:
        raise ValueError(kind)
    return o


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a bf16 (uint16) or e4m3 (uint8) tensor, copied to the host."""
    if t.dtype == torch.bfloat16:
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.detach().view(torch.uint8).cpu().numpy()
    return t.detach().cpu().numpy()
