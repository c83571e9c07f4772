#!/usr/bin/env python3
"""Benchmark of the MiniMax-H3 AdaLN projection stages on one MI355X.

One step = one pass of the whole hot path over one batch of M = 32760 tokens:
  pre-attention (RMSNorm + AdaLN -> workspace; QKV GEMM + Q/K norm + RoPE + pack),
  gated-residual out-projection (bf16), and the FP8 W8A8 MLP block,
with the seeded synthetic inputs of the three M = 32760 workloads already resident in HBM.

The headline value is the pre-attention stage throughput: 2*M*21504*5376 flop over the wall
time of its two launches, from HIP events on the stream the kernels run on.  Each kernel
launch of the step is bracketed by events so the dominant kernel (the QKV GEMM) can be
priced against the bf16 MFMA peak.  The CPU oracle is timed on a bounded row sample of the
same pre-attention workload on the host's cores (cpu_baseline).

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

M_TOKENS = 32760
QKV_FLOP = 2.0 * M_TOKENS * 21504 * 5376          # 7.5745e12
OUTP_FLOP = 2.0 * M_TOKENS * 5376 * 7168           # 2.5248e12
MLP_FLOP = 2.0 * M_TOKENS * 28672 * 5376 + 2.0 * M_TOKENS * 5376 * 14336   # 1.5149e13
# Published MI355X dense peaks (TFLOP/s) and HBM bandwidth (GB/s).
PEAK_BF16 = 2500.0
PEAK_FP8 = 5000.0
PEAK_FP4 = 10100.0
PEAK_HBM = 8000.0
# Minimum HBM bytes of the norm/AdaLN launch per row: read x (5376 bf16), write the workspace
# (5376 bf16), read the int64 index; tables and the norm weight stay in cache.
NORM_BYTES_PER_ROW = 5376 * 2 * 2 + 8
FLUSH_BYTES = 512 << 20


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("gemm.hpp", "pre_attn.hip", "qk_epi.hpp", "common.hpp"):
        with open(os.path.join(ROOT, "diffusion_transformer_adaln_rmsnorm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per QKV GEMM launch from the committed counter summary, if it still
    describes the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "qkv_gemm_traffic_m32760.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(d, seconds_target=15.0):
    import numpy as np
    import oracle
    threads = max(1, os.cpu_count() or 1)
    # one warm call sizes the sample so that the timed call lasts about seconds_target
    t0 = time.perf_counter()
    oracle.pre_attn(d, rows_sel=np.arange(threads, dtype=np.int64), threads=threads)
    per_round = time.perf_counter() - t0
    rounds = max(1, int(seconds_target / max(per_round, 1e-3)))
    g = np.random.Generator(np.random.PCG64(12345))
    rows = np.sort(g.choice(d["M"], size=min(d["M"], rounds * threads), replace=False)).astype(np.int64)
    t0 = time.perf_counter()
    oracle.pre_attn(d, rows_sel=rows, threads=threads)
    dt = time.perf_counter() - t0
    flop = 2.0 * rows.size * 21504 * 5376
    rows_per_s = rows.size / dt
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "model": cpu_model(), "rows_per_s": round(rows_per_s, 2),
            "full_M_s_extrapolated": round(d["M"] / rows_per_s, 1),
            "sample": f"pre-attention oracle (fp64, C) on {rows.size} seeded random rows of the M={d['M']} workload, "
                      f"{dt:.1f} s wall on {threads} threads (os.cpu_count()); value = QKV flops of those rows / "
                      f"wall time; full_M_s_extrapolated = M / rows_per_s (rows are independent), not measured"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the first launches run at a lower shader clock while power management ramps up
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stages", default="pre_attn,out_proj,mlp")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device-to-device copy 3 times (reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: every stage here is data-parallel over rows and runs on a "
              f"single MI355X; --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    stages = [s for s in args.stages.split(",") if s]

    import numpy as np
    import torch

    if args.calibrate_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": 1 << 30, "copies": 3}))
        return

    import synth
    import diffusion_transformer_adaln_rmsnorm_amd as dit

    dit.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t_gen = time.perf_counter()
    log("generating seeded inputs (pre-attention M=32760)")
    _, d_pre = synth.config(2)
    tp = synth.to_torch("pre_attn", d_pre, dev)
    ws = torch.empty((M_TOKENS, 5376), dtype=torch.bfloat16, device=dev)
    out_qkv = torch.empty((1, M_TOKENS, 56, 3, 128), dtype=torch.bfloat16, device=dev)
    if "out_proj" in stages:
        log("generating seeded inputs (out-projection M=32760)")
        _, d_op = synth.config(3)
        to = synth.to_torch("out_proj", d_op, dev)
        out_op = torch.empty((M_TOKENS, 5376), dtype=torch.bfloat16, device=dev)
        del d_op
    if "mlp" in stages:
        log("generating seeded inputs (fp8 MLP M=32760)")
        _, d_mlp = synth.config(4)
        tm = synth.to_torch("mlp", d_mlp, dev)
        del d_mlp
        mws = {"workspace_a_q": torch.empty((M_TOKENS, 5376), dtype=torch.float8_e4m3fn, device=dev),
               "workspace_a_scale": torch.empty((M_TOKENS,), dtype=torch.float32, device=dev),
               "workspace_y": torch.empty((M_TOKENS, 14336), dtype=torch.bfloat16, device=dev),
               "workspace_y_q": torch.empty((M_TOKENS, 14336), dtype=torch.float8_e4m3fn, device=dev),
               "workspace_y_scale": torch.empty((M_TOKENS,), dtype=torch.float32, device=dev)}
        out_mlp = torch.empty((M_TOKENS, 5376), dtype=torch.bfloat16, device=dev)
    # cache flush between timed iterations: a 512 MiB device copy (1 GiB of traffic) evicts the
    # 4 MiB L2 of every XCD and the 256 MiB Infinity Cache, so no launch finds its inputs there
    flush_src = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    flush_dst = torch.empty_like(flush_src)

    def flush():
        flush_dst.copy_(flush_src)

    torch.cuda.synchronize()
    log(f"inputs resident in HBM ({time.perf_counter() - t_gen:.1f} s)")

    def step(ev):
        ev[0].record()
        dit.dit_norm_adaln_bf16(tp["x"], tp["x_norm_weight"], tp["adaln_scale"], tp["adaln_shift"],
                                tp["adaln_index"], workspace=ws, eps=tp["eps"])
        ev[1].record()
        dit.dit_qkv_rope_pack_bf16(ws, tp["qkv_weight"], tp["q_norm_weight"], tp["k_norm_weight"],
                                   tp["rope_cos_sin"], ulysses_degree=1, out=out_qkv, qk_eps=tp["qk_eps"],
                                   rope_positions=tp["rope_positions"])
        ev[2].record()
        if "out_proj" in stages:
            dit.dit_out_proj_gated_bf16(to["attn_out"], to["o_weight"], to["gate"], to["gate_index"],
                                        to["residual"], out=out_op)
        ev[3].record()
        if "mlp" in stages:
            dit.dit_mlp_fp8(tm["x"], tm["x_norm_weight"], tm["adaln_scale"], tm["adaln_shift"], tm["adaln_index"],
                            tm["gate"], tm["residual"], tm["fc1_weight_q"], tm["fc1_weight_scale"],
                            tm["fc2_weight_q"], tm["fc2_weight_scale"], out=out_mlp, eps=tm["eps"], **mws)
        ev[4].record()

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(5)]  # noqa: E731
    for i in range(args.warmup):
        flush()
        step(mk())
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps); timing {args.steps} steps")
    evs = [mk() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        flush()
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    seg = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(4)] for e in evs])   # ms
    def time_calls(fn, n, warm=3):
        """Mean event time (ms) of fn over n calls, each after a cache flush, on the stream the
        kernels run on (torch's current stream, which the binding passes to the library)."""
        for _ in range(warm):
            flush()
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in ev:
            flush()
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev]))

    n8 = max(3, min(args.steps, 10))
    # the e4m3 output mode of the QKV launch (same workspace and weights; not part of the step)
    out_e4m3 = torch.empty((1, M_TOKENS, 56, 3, 128), dtype=torch.uint8, device=dev)

    def qkv_e4m3():
        dit.dit_qkv_rope_pack_e4m3(ws, tp["qkv_weight"], tp["q_norm_weight"], tp["k_norm_weight"],
                                   tp["rope_cos_sin"], ulysses_degree=1, out=out_e4m3, q_descale=1.0 / 96.0,
                                   k_descale=0.015, v_descale=0.0075, qk_eps=tp["qk_eps"],
                                   rope_positions=tp["rope_positions"])
    e4m3_ms = time_calls(qkv_e4m3, n8)
    del out_e4m3
    # the MXFP4 W4A4 pre-attention on the same inputs (qkv weight quantised once, outside the
    # timing; each call runs the fused norm + quantisation and the block-scaled QKV GEMM)
    wq_c, wq_s = dit.dit_mx_quant_fp4(tp["qkv_weight"])
    ws_c = torch.empty((M_TOKENS, 2688), dtype=torch.uint8, device=dev)
    ws_s = torch.empty((dit.dit_mx_scale_bytes(M_TOKENS, 5376),), dtype=torch.uint8, device=dev)

    def pre_mx():
        dit.dit_pre_attn_mxfp4(tp["x"], tp["x_norm_weight"], tp["adaln_scale"], tp["adaln_shift"], tp["adaln_index"],
                               wq_c, wq_s, tp["q_norm_weight"], tp["k_norm_weight"], tp["rope_cos_sin"],
                               ulysses_degree=1, out=out_qkv, eps=tp["eps"], qk_eps=tp["qk_eps"],
                               rope_positions=tp["rope_positions"], ws_codes=ws_c, ws_scales=ws_s)
    pre_mx_ms = time_calls(pre_mx, n8)
    del wq_c, wq_s, ws_c, ws_s
    mx_ms = None
    if "out_proj" in stages:
        # the MXFP4 W4A4 out-projection on the same inputs (weight quantised once, outside the
        # timing; each call quantises attn_out and runs the block-scaled GEMM; not part of the step)
        w_c, w_s = dit.dit_mx_quant_fp4(to["o_weight"])
        a_c = torch.empty((M_TOKENS, 3584), dtype=torch.uint8, device=dev)
        a_s = torch.empty((dit.dit_mx_scale_bytes(M_TOKENS, 7168),), dtype=torch.uint8, device=dev)

        def op_mx():
            dit.dit_out_proj_gated_mxfp4(to["attn_out"], w_c, w_s, to["gate"], to["gate_index"], to["residual"],
                                         out=out_op, act_codes=a_c, act_scales=a_s)
        mx_ms = time_calls(op_mx, n8)
        del w_c, w_s, a_c, a_s
    # the two smaller pre-attention workloads (M = 16: W streaming, HBM-bound; M = 4096), each
    # with its own seeded inputs, both launches timed, a cache flush before each call
    small = {}
    for cid in (0, 1):
        _, dc = synth.config(cid)
        tc = synth.to_torch("pre_attn", dc, dev)
        Mc = dc["M"]
        wsc = torch.empty((Mc, 5376), dtype=torch.bfloat16, device=dev)
        outc = torch.empty((1, Mc, 56, 3, 128), dtype=torch.bfloat16, device=dev)

        def pre_c():
            dit.dit_pre_attn_bf16(tc["x"], tc["x_norm_weight"], tc["adaln_scale"], tc["adaln_shift"],
                                  tc["adaln_index"], tc["qkv_weight"], tc["q_norm_weight"], tc["k_norm_weight"],
                                  tc["rope_cos_sin"], ulysses_degree=1, out=outc, eps=tc["eps"], qk_eps=tc["qk_eps"],
                                  rope_positions=tc["rope_positions"], workspace=wsc)
        ms = time_calls(pre_c, 20, warm=5)
        idx = dc["adaln_index"]
        rows_touched = len(set(int(i) for i in idx if 0 <= i < dc["adaln_scale"].rows))
        # minimum bytes of both launches: x, workspace write + read, index, the touched table rows
        # (scale and shift), x_norm_weight, W, q/k norm weights, one cos/sin row per token, out
        byts = (Mc * (5376 * 2 * 3 + 8 + 192 + 21504 * 2) + rows_touched * 2 * 5376 * 2 + 5376 * 2
                + 21504 * 5376 * 2 + 2 * 128 * 2 + (Mc * 8 if dc["rope_positions"] is not None else 0))
        flop = 2.0 * Mc * 21504 * 5376
        small[cid] = (Mc, ms, byts, flop)
        log(f"config {cid}: pre-attn M={Mc} {ms * 1e3:.1f} us = {byts / ms / 1e6:.0f} GB/s, "
            f"{flop / ms / 1e9:.1f} TFLOP/s")
        del tc, wsc, outc, dc
    norm_ms, gemm_ms, op_ms, mlp_ms = seg.mean(axis=0)
    pre_ms = norm_ms + gemm_ms
    ms_per_step = wall * 1e3 / args.steps
    value = QKV_FLOP / (pre_ms * 1e-3) / 1e12
    gemm_tflops = QKV_FLOP / (gemm_ms * 1e-3) / 1e12
    log(f"pre-attn {pre_ms:.3f} ms (norm {norm_ms:.3f} + qkv gemm {gemm_ms:.3f}) = {value:.1f} TFLOP/s; "
        f"out-proj {op_ms:.3f} ms; mlp {mlp_ms:.3f} ms; step {ms_per_step:.3f} ms")
    traffic = load_traffic()
    res = {
        "metric": "pre-attn TFLOP/s at M=32760 bf16 and % of MI355X MFMA peak (1 GPU)",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded PCG64, shapes of the MiniMax-H3 block)",
        "config": {"workload": "bf16 pre-attention M=32760 (QKV 32760x21504x5376, rows=2 AdaLN tables, S=32760 "
                               "identity positions); step also runs the M=32760 bf16 gated out-projection and "
                               "fp8 W8A8 MLP", "tokens": M_TOKENS, "stages": stages,
                   "cache_flush": "512 MiB device copy before each step and each timed call, outside the "
                                  "kernel events (ms_per_step includes it)"},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16, 2),
        "roofline": {"bound": "mfma", "kernel": "k_qkv_gemm", "achieved": round(gemm_tflops, 2),
                     "peak": PEAK_BF16, "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_BF16, 4),
                     "traffic": traffic, "avg_launch_ms": round(float(gemm_ms), 4)},
        "stages_ms": {"norm_adaln": round(float(norm_ms), 4), "qkv_gemm": round(float(gemm_ms), 4),
                      "out_proj": round(float(op_ms), 4), "mlp_fp8": round(float(mlp_ms), 4),
                      "qkv_gemm_e4m3_out": round(float(e4m3_ms), 4)},
        "stage_rates": {
            "norm_adaln_GBps": round(NORM_BYTES_PER_ROW * M_TOKENS / (norm_ms * 1e-3) / 1e9, 1),
            "norm_adaln_frac_hbm": round(NORM_BYTES_PER_ROW * M_TOKENS / (norm_ms * 1e-3) / 1e9 / PEAK_HBM, 4),
            "qkv_gemm_e4m3_out_TFLOPs": round(QKV_FLOP / (e4m3_ms * 1e-3) / 1e12, 2),
            "qkv_gemm_e4m3_out_frac_bf16": round(QKV_FLOP / (e4m3_ms * 1e-3) / 1e12 / PEAK_BF16, 4),
        },
    }
    if "out_proj" in stages:
        r = OUTP_FLOP / (op_ms * 1e-3) / 1e12
        res["stage_rates"]["out_proj_TFLOPs"] = round(r, 2)
        res["stage_rates"]["out_proj_frac_bf16"] = round(r / PEAK_BF16, 4)
    r = QKV_FLOP / (pre_mx_ms * 1e-3) / 1e12
    res["stages_ms"]["pre_attn_mxfp4"] = round(float(pre_mx_ms), 4)
    res["stage_rates"]["pre_attn_mxfp4_TFLOPs"] = round(r, 2)
    res["stage_rates"]["pre_attn_mxfp4_frac_fp4"] = round(r / PEAK_FP4, 4)
    if mx_ms is not None:
        r = OUTP_FLOP / (mx_ms * 1e-3) / 1e12
        res["stages_ms"]["out_proj_mxfp4"] = round(float(mx_ms), 4)
        res["stage_rates"]["out_proj_mxfp4_TFLOPs"] = round(r, 2)
        res["stage_rates"]["out_proj_mxfp4_frac_fp4"] = round(r / PEAK_FP4, 4)
    M0, ms0, b0, f0 = small[0]
    res["stages_ms"]["pre_attn_m16"] = round(ms0, 5)
    res["stage_rates"]["pre_attn_m16_GBps"] = round(b0 / (ms0 * 1e-3) / 1e9, 1)
    res["stage_rates"]["pre_attn_m16_frac_hbm"] = round(b0 / (ms0 * 1e-3) / 1e9 / PEAK_HBM, 4)
    res["stage_rates"]["pre_attn_m16_bytes"] = b0
    M1, ms1, b1, f1 = small[1]
    res["stages_ms"]["pre_attn_m4096"] = round(ms1, 4)
    res["stage_rates"]["pre_attn_m4096_TFLOPs"] = round(f1 / (ms1 * 1e-3) / 1e12, 2)
    res["stage_rates"]["pre_attn_m4096_frac_bf16"] = round(f1 / (ms1 * 1e-3) / 1e12 / PEAK_BF16, 4)
    if "mlp" in stages:
        r = MLP_FLOP / (mlp_ms * 1e-3) / 1e12
        res["stage_rates"]["mlp_fp8_TFLOPs"] = round(r, 2)
        res["stage_rates"]["mlp_fp8_frac_fp8"] = round(r / PEAK_FP8, 4)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a row sample")
        res["cpu_baseline"] = cpu_baseline(d_pre)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
