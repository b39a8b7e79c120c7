"""Benchmark of one routed-MoE expert layer on one MI355X.

One step = the whole path over one batch of synthetic tokens:
route -> align -> grouped gate/up + SiLU -> grouped down -> [LoRA fold] -> combine.

Prints ONE JSON line (metric = MoE layer tokens/s).  The grouped gate/up GEMM is
timed on its own with HIP events on the launch stream inside the timed region and
reported against the bf16 MFMA peak; the CPU oracle is timed on a bounded token
sample of the same workload on the host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)




def gemm_flops(cfg, op: str) -> float:
    """Algorithmic FLOPs of one grouped GEMM launch: 2*K*N per real (token, expert) pair and projection."""
    per_pair = {"gate_up": 2 * 2 * cfg.H * cfg.I, "down": 2 * cfg.H * cfg.I}[op]
    return float(per_pair) * cfg.P


def expert_weight_bytes(cfg, op: str) -> float:
    """Bytes of one expert's weights read by one launch (gate+up, or down)."""
    nproj = 2 if op == "gate_up" else 1
    if cfg.weights == "bf16":
        return float(nproj * cfg.H * cfg.I * 2)
    if cfg.weights == "fp8":   # codes + one fp32 scale per output channel
        N = cfg.I if op == "gate_up" else cfg.H
        return float(nproj * (cfg.H * cfg.I + N * 4))
    G = cfg.group_size
    K, N = (cfg.H, cfg.I) if op == "gate_up" else (cfg.I, cfg.H)
    per = K // 8 * N * 4 + K // G * N * 2 + K // G * N // 8 * 4   # qweight + fp16 scales + qzeros
    return float(nproj * per)


def gemm_bytes(cfg, op: str, active_experts: int) -> float:
    """Algorithmic HBM bytes of one grouped GEMM launch: the active experts' weights, the
    activation rows read once (x for gate/up, Hs for down; 1-byte codes on the fp8 path) and the
    rows written (Hs / Ys)."""
    w = active_experts * expert_weight_bytes(cfg, op)
    ab = 1 if cfg.weights == "fp8" else 2
    if op == "gate_up":
        act = cfg.T * cfg.H * ab + cfg.P * cfg.I * 2
    else:
        act = cfg.P * cfg.I * ab + cfg.P * cfg.H * 2
    return w + act


def clone_layer(layer):
    """Same weights in fresh buffers (so repeated steps cannot be served from the 256 MB MALL)."""
    import copy
    import mixture_experts_routed_route_amd as m
    c = copy.copy(layer)
    def cw(w):
        if isinstance(w, m.Bf16Weight):
            return m.Bf16Weight(w.w.clone())
        if isinstance(w, m.Fp8Weight):
            return m.Fp8Weight(w.codes.clone(), w.scales.clone())
        return m.GptqWeight(w.qweight.clone(), w.scales.clone(), w.qzeros.clone(), w.group_size)
    c.gate, c.up, c.down = cw(layer.gate), cw(layer.up), cw(layer.down)
    return c


def measured_traffic(workload: str, role: str):
    """HBM bytes per launch of one grouped GEMM from the committed FETCH_SIZE/WRITE_SIZE summary of
    this workload (already scaled by the copy calibration), or None when there is none or the
    kernel's source files have changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith((" ", "#")):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    files, want = kv.get("source_files", "").split(), kv.get("source_sha256")
    if not files or not want or f"{role}.traffic_bytes" not in kv:
        return None
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "mixture_experts_routed_route_amd", "csrc", f), "rb").read())
    return float(kv[f"{role}.traffic_bytes"]) if h.hexdigest() == want else None


def layer_flops(cfg) -> float:
    return 6.0 * cfg.H * cfg.I * cfg.P


def cpu_baseline(cfg, d, budget_tokens: int, min_seconds: float = 10.0, max_runs: int = 8):
    """The oracle as it stands, on the first ``budget_tokens`` tokens of the same workload, run
    repeatedly until at least ``min_seconds`` of host time have passed (at most ``max_runs`` runs)."""
    import oracle
    from threadpoolctl import threadpool_info
    T = min(cfg.T, budget_tokens)
    sub = dict(d)
    sub["cfg"] = cfg.with_(T=T)
    sub["logits"] = d["logits"][:T]
    sub["x"] = d["x"][:T]
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle.moe_layer(sub)
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or runs >= max_runs:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": runs * T / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{runs} run(s) of the first {T} of {cfg.T} tokens of {cfg.name}, whole layer (route, "
                      f"align, grouped GEMMs, combine) in fp64 numpy; {dt:.1f} s in total"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="mixtral_prefill")
    ap.add_argument("--cpu-tokens", type=int, default=4096, help="token sample of the CPU oracle leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotate", type=int, default=0,
                    help="independent weight copies cycled through (0: enough for >= 1 GiB of weights, max 4)")
    ap.add_argument("--graph", action="store_true",
                    help="time steps replayed from HIP graphs (one captured step per weight copy); the "
                         "per-kernel figures then come from an eager pass of the same steps")
    ap.add_argument("--fold", default="auto", choices=["auto", "grouped", "gather"],
                    help="LoRA fold over the sorted rows or slot by slot (auto: by the padding share)")
    ap.add_argument("--gate-up-lora", default="fused", choices=["fused", "unfused"],
                    help="gate/up LoRA folded in the gate/up GEMM's epilogue, or the page's unfused order")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (reference for the FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures the single-GPU path only; --gpus {args.gpus} is not supported "
              "(multi-GPU expert/tensor parallel sharding is not part of this build)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import mixture_experts_routed_route_amd as m
    from moe_synth import CONFIGS, make_inputs

    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    log(f"[bench] generating {cfg.name} inputs")
    d = make_inputs(cfg)
    layer = m.MoeLayer.from_arrays(d, dev, fold=args.fold, gate_up_fused=args.gate_up_lora == "fused")
    b = layer.plan(cfg.T, dev)
    wbytes = sum(expert_weight_bytes(cfg, op) for op in ("gate_up", "down")) * cfg.E
    rot = args.rotate or max(1, min(4, int(-(-(1 << 30) // wbytes))))
    layers = [layer] + [clone_layer(layer) for _ in range(rot - 1)]
    logits = torch.from_numpy(d["logits"]).to(dev)
    x = torch.from_numpy(d["x"]).view(torch.bfloat16).to(dev)
    torch.cuda.synchronize()

    def step(i, ev=None):
        layer = layers[i % rot]
        layer.route_align(logits, b)
        if ev is not None:
            ev[0].record()
        layer.gate_up_stage(x, b)
        if ev is not None:
            ev[1].record()
        layer.down_stage(b)
        if ev is not None:
            ev[2].record()
        layer.lora_fold(b)
        if ev is not None:
            ev[3].record()
        layer.combine(b)

    log(f"[bench] warmup {args.warmup}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    if args.graph:
        # the path allocates nothing and issues no memset, so a step captures as it runs eagerly
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        graphs = []
        for i in range(rot):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                step(i)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[i % rot].replay()
        torch.cuda.synchronize()
        log(f"[bench] timing {args.steps} graph replays")
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % rot].replay()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        log("[bench] per-kernel timing: eager pass")
        for i in range(args.steps):
            step(i, events[i])
        torch.cuda.synchronize()
    else:
        log(f"[bench] timing {args.steps} steps")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i, events[i])
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
    ms = dt * 1e3 / args.steps
    gu_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    dn_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    fold_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in events])) if layer.lora is not None else None
    gu_what = ("gemm_bf16_kernel<gate_up> with the gate/up LoRA epilogue (+ 2 shrinks)"
               if layer.gate_up_lora and layer.gate_up_fused
               else "gate/up stage: 2 gathered GEMMs, 2 LoRA folds, SiLU*up" if layer.gate_up_lora
               else "gate/up stage: x quantisation + gemm_fp8_kernel<gate_up>" if cfg.weights == "fp8"
               else ("gemm_bf16_kernel" if cfg.weights == "bf16" else "gemm_int4_kernel") + "<gate_up>")
    peak_mfma = PEAK_FP8_TFLOPS if cfg.weights == "fp8" else PEAK_BF16_TFLOPS
    tokens_s = cfg.T / (ms / 1e3)
    active = int((b.routing.counts > 0).sum().item())
    gu_bytes = gemm_bytes(cfg, "gate_up", active)
    gu_tflops = gemm_flops(cfg, "gate_up") / (gu_ms / 1e3) / 1e12
    dn_tflops = gemm_flops(cfg, "down") / (dn_ms / 1e3) / 1e12
    gemm_tflops = (gemm_flops(cfg, "gate_up") + gemm_flops(cfg, "down")) / ((gu_ms + dn_ms) / 1e3) / 1e12
    log(f"[bench] step {ms:.3f} ms; gate/up {gu_ms:.3f} ms ({gu_tflops:.1f} TFLOP/s); "
        f"down {dn_ms:.3f} ms ({dn_tflops:.1f} TFLOP/s); grouped GEMMs {gemm_tflops:.1f} TFLOP/s"
        + (f"; LoRA fold ({layer.fold_mode(b)}) {1e3 * fold_ms:.1f} us" if fold_ms is not None else ""))

    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.int16, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 1 GiB device-to-device copy done")

    ai = gemm_flops(cfg, "gate_up") / gu_bytes
    if ai >= peak_mfma * 1e12 / (PEAK_HBM_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": gu_tflops, "peak": peak_mfma, "unit": "TFLOP/s"}
    else:
        gbs = gu_bytes / (gu_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(cfg.name, "gate_up")
    roof["kernel"] = gu_what
    roof["algorithmic"] = {"flops": gemm_flops(cfg, "gate_up"), "bytes": gu_bytes, "active_experts": active,
                           "flop_per_byte": ai}
    log(f"[bench] gate/up roofline: {roof['bound']} {roof['achieved']:.1f} {roof['unit']} "
        f"({100 * roof['frac']:.1f}% of peak), AI {ai:.0f} flop/B, {active} active experts, rotate {rot}")

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] cpu oracle on {args.cpu_tokens} tokens")
        cpu = cpu_baseline(cfg, d, args.cpu_tokens)
        log(f"[bench] cpu oracle {cpu['value']:.2f} tokens/s on {cpu['cores']} threads")

    line = {
        "metric": "MoE layer tokens/s + grouped-GEMM TFLOP/s (% bf16 MFMA / HBM peak), 1 GPU",
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8 e4m3 x fp8 e4m3, fp32 accumulate"}.get(
            cfg.weights, "int4 weights x bf16, fp32 accumulate"),
        "data": "synthetic (seeded numpy PCG64; random-init expert weights)",
        "config": {"workload": cfg.name, "tokens": cfg.T, "hidden": cfg.H, "intermediate": cfg.I,
                   "experts": cfg.E, "top_k": cfg.top_k, "block_size": cfg.block_size,
                   "weights": cfg.weights, "lora_rank": cfg.lora_rank,
                   **({"lora_fold": layer.fold_mode(b)} if layer.lora is not None else {}),
                   **({"lora_gate_up": "fused" if layer.gate_up_fused else "unfused"} if layer.gate_up_lora else {}),
                   "launch": "hip_graph" if args.graph else "eager"},
        "grouped_gemm_tflops": gemm_tflops,
        "grouped_gemm_frac_mfma_peak": gemm_tflops / peak_mfma,
        "kernels_ms": {"gate_up": gu_ms, "down": dn_ms,
                       **({"lora_fold": fold_ms} if fold_ms is not None else {})},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
