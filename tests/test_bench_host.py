"""The bench's host-side contract, on the CPU: the multi-GPU refusal, the algorithmic work that
the roofline figures divide by, the guard that drops a traffic figure taken on other kernel
sources, and the shape of the CPU-oracle baseline object."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from moe_synth import CONFIGS, MoeConfig, make_inputs  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "single-GPU" in r.stderr and r.stdout == ""


def test_algorithmic_work_of_the_mixtral_workload():
    cfg = CONFIGS["mixtral_prefill"]          # T=4096, H=4096, I=14336, E=8, top-2
    P = 4096 * 2
    assert bench.gemm_flops(cfg, "gate_up") == 2 * 2 * 4096 * 14336 * P
    assert bench.gemm_flops(cfg, "down") == 2 * 4096 * 14336 * P
    # 8 active experts: all gate+up weights, x once, Hs written once
    w = 8 * 2 * 4096 * 14336 * 2
    assert bench.gemm_bytes(cfg, "gate_up", 8) == w + 4096 * 4096 * 2 + P * 14336 * 2
    assert bench.gemm_bytes(cfg, "down", 8) == w / 2 + P * 14336 * 2 + P * 4096 * 2


def test_algorithmic_work_of_the_lora_fold():
    cfg = CONFIGS["lora_prefill"]             # I=1408, H=4096, rank 16 padded to 64
    counts = [10, 7, 0, 3]                    # expert 2 adapted but idle, expert 1 not adapted
    flops, bytes_, rows = bench.fold_work(cfg, counts, [0, 2, 3])
    assert rows == 13
    assert flops == 2 * 16 * (1408 + 4096) * 13
    per_row = 1408 * 2 + 2 * 4096 * 2 + 2 * 64 * 2
    assert bytes_ == 13 * per_row + 2 * (64 * 1408 * 2 + 4096 * 64 * 2)


def test_roofline_bound_follows_the_ridge():
    r = bench.roofline(1e12, 1e9, 1.0, 2500.0, "k")       # 1000 flop/B > ridge 312.5
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and abs(r["achieved"] - 1000.0) < 1e-9
    assert abs(r["frac"] - 0.4) < 1e-12
    r = bench.roofline(1e10, 1e9, 1.0, 2500.0, "k")       # 10 flop/B
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and abs(r["achieved"] - 1000.0) < 1e-9


def test_algorithmic_bytes_of_gptq_weights():
    cfg = CONFIGS["decode_int4"]              # H=2048, I=1408, G=128
    K, N, G = 2048, 1408, 128
    per = K // 8 * N * 4 + K // G * N * 2 + K // G * N // 8 * 4
    assert bench.expert_weight_bytes(cfg, "gate_up") == 2 * per
    K, N = 1408, 2048
    assert bench.expert_weight_bytes(cfg, "down") == K // 8 * N * 4 + K // G * N * 2 + K // G * N // 8 * 4


def test_algorithmic_work_of_the_fp8_workload():
    cfg = CONFIGS["fp8_prefill"]              # mixtral_prefill's shape, E4M3 weights
    P = 4096 * 2
    assert bench.gemm_flops(cfg, "gate_up") == 2 * 2 * 4096 * 14336 * P
    # codes (1 byte) + one fp32 scale per output channel; activations read as 1-byte codes
    w = 8 * 2 * (4096 * 14336 + 14336 * 4)
    assert bench.gemm_bytes(cfg, "gate_up", 8) == w + 4096 * 4096 * 1 + P * 14336 * 2
    assert bench.expert_weight_bytes(cfg, "down") == 4096 * 14336 + 4096 * 4


def _write_traffic(tmp, src_files, sha, value):
    os.makedirs(os.path.join(tmp, "profiles"))
    with open(os.path.join(tmp, "profiles", "traffic_w.txt"), "w") as f:
        f.write("# header\n\n  indented: ignored\n")
        f.write(f"source_files: {' '.join(src_files)}\nsource_sha256: {sha}\n")
        f.write(f"gate_up.traffic_bytes: {value}\n")


def test_traffic_figure_only_for_the_profiled_sources(tmp_path, monkeypatch):
    tmp = str(tmp_path)
    csrc = os.path.join(tmp, "mixture_experts_routed_route_amd", "csrc")
    os.makedirs(csrc)
    with open(os.path.join(csrc, "k.hip"), "wb") as f:
        f.write(b"kernel source v1")
    sha = hashlib.sha256(b"kernel source v1").hexdigest()
    _write_traffic(tmp, ["k.hip"], sha, 12345)
    monkeypatch.setattr(bench, "ROOT", tmp)
    assert bench.measured_traffic("w", "gate_up") == 12345.0
    assert bench.measured_traffic("w", "down") is None          # no figure for that role
    assert bench.measured_traffic("other", "gate_up") is None   # no summary for that workload
    with open(os.path.join(csrc, "k.hip"), "wb") as f:
        f.write(b"kernel source v2")                           # the kernel changed since
    assert bench.measured_traffic("w", "gate_up") is None


def test_traffic_figure_per_role_sources(tmp_path, monkeypatch):
    """A role with its own source list is judged by those files alone: changing another role's
    kernel does not void it."""
    tmp = str(tmp_path)
    csrc = os.path.join(tmp, "mixture_experts_routed_route_amd", "csrc")
    os.makedirs(csrc)
    for name, body in (("g.hip", b"gemm v1"), ("f.hip", b"fold v1")):
        with open(os.path.join(csrc, name), "wb") as f:
            f.write(body)
    os.makedirs(os.path.join(tmp, "profiles"))
    with open(os.path.join(tmp, "profiles", "traffic_w.txt"), "w") as f:
        f.write("# test\n")
        f.write(f"gate_up.source_files: g.hip\ngate_up.source_sha256: {hashlib.sha256(b'gemm v1').hexdigest()}\n")
        f.write("gate_up.traffic_bytes: 111\n")
        f.write(f"lora_fold.source_files: f.hip\nlora_fold.source_sha256: {hashlib.sha256(b'fold v1').hexdigest()}\n")
        f.write("lora_fold.traffic_bytes: 222\n")
    monkeypatch.setattr(bench, "ROOT", tmp)
    assert bench.measured_traffic("w", "gate_up") == 111.0
    assert bench.measured_traffic("w", "lora_fold") == 222.0
    with open(os.path.join(csrc, "f.hip"), "wb") as f:
        f.write(b"fold v2")
    assert bench.measured_traffic("w", "lora_fold") is None
    assert bench.measured_traffic("w", "gate_up") == 111.0


def test_cpu_baseline_object():
    cfg = MoeConfig("bench_tiny", T=48, H=64, I=32, E=4, top_k=2, block_size=16, seed=3)
    d = make_inputs(cfg)
    cpu = bench.cpu_baseline(cfg, d, tokens=32, min_seconds=0.0, max_runs=2)
    assert set(cpu) == {"value", "unit", "cores", "kind", "sample"}
    assert cpu["kind"] == "oracle" and cpu["unit"] == "tokens/s"
    assert cpu["value"] > 0 and 1 <= cpu["cores"] <= len(os.sched_getaffinity(0))
    assert "32 of 48 tokens" in cpu["sample"]
