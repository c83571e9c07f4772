"""Host-side logic of bench.py, on the CPU: the traffic figure it reports for the QKV GEMM and
its refusal of more than one GPU.  No device is touched."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUMMARY = os.path.join(ROOT, "profiles", "qkv_gemm_traffic_m32760.json")


def _summary():
    with open(SUMMARY) as fh:
        return json.load(fh)


def test_traffic_summary_is_self_consistent():
    """bytes_per_launch = FETCH_SIZE KiB x 1024 x the copy factor + WRITE_SIZE KiB x 1024 x its
    factor, and the algorithmic bytes are the workspace, the weight and the output once each."""
    t = _summary()
    fetch = t["fetch_kib_per_dispatch"] * 1024 * t["copy_fetch_factor"]
    write = t["write_kib_per_dispatch"] * 1024 * t["copy_write_factor"]
    assert abs(fetch + write - t["bytes_per_launch"]) <= 1e-4 * t["bytes_per_launch"]
    assert t["algorithmic_bytes_per_launch"] == 32760 * 5376 * 2 + 21504 * 5376 * 2 + 32760 * 21504 * 2
    # the counters read at least what the kernel must move (they count L2 misses, which include it)
    assert t["bytes_per_launch"] >= t["algorithmic_bytes_per_launch"]
    # a 1 GiB device copy reads and writes 1 GiB: the factors scale the counters to that
    assert 0.5 < t["copy_fetch_factor"] < 4 and 0.5 < t["copy_write_factor"] < 4


def test_traffic_is_reported_only_for_the_source_it_was_taken_on(monkeypatch):
    t = _summary()
    got = bench.load_traffic()
    if t["kernel_source_hash"] == bench.kernel_source_hash():
        assert got == t["bytes_per_launch"]
    else:
        assert got is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.load_traffic() is None


def test_kernel_source_hash_covers_the_qkv_sources(tmp_path, monkeypatch):
    """Any byte of gemm.hpp, pre_attn.hip, qk_epi.hpp or common.hpp changes the hash."""
    src = os.path.join(ROOT, "diffusion_transformer_adaln_rmsnorm_amd", "csrc")
    fake = tmp_path / "diffusion_transformer_adaln_rmsnorm_amd" / "csrc"
    fake.mkdir(parents=True)
    names = ("gemm.hpp", "pre_attn.hip", "qk_epi.hpp", "common.hpp")
    for n in names:
        (fake / n).write_bytes(open(os.path.join(src, n), "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    monkeypatch.setattr(bench, "ROOT", ROOT)
    assert h0 == bench.kernel_source_hash()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    for n in names:
        p = fake / n
        orig = p.read_bytes()
        p.write_bytes(orig + b" ")
        assert bench.kernel_source_hash() != h0, n
        p.write_bytes(orig)
    assert bench.kernel_source_hash() == h0


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)
    assert r.stdout.strip() == "" or not r.stdout.strip().startswith("{")
