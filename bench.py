"""Benchmark of one routed-MoE expert layer on one MI355X.

One step = the whole path over one batch of synthetic tokens:
route -> align -> grouped gate/up + SiLU -> grouped down -> [LoRA fold] -> combine.

By default the five workloads the metric is quoted on run one after the other (tiny,
mixtral_prefill, finegrained_skewed, decode_int4, lora_prefill), and ONE JSON line is printed:
``value`` is the tokens/s of mixtral_prefill (the largest prefill workload), ``roofline`` is its
dominant kernel (the grouped gate/up GEMM), and ``configs`` holds every workload's own figures:
tokens/s, per-kernel times, a roofline object per GEMM (and per LoRA fold), and the CPU oracle
timed on a bounded token sample of that workload on the host's cores.  ``--config NAME`` runs a
single workload (used for the rocprofv3 runs whose summaries sit in profiles/).

Each kernel is timed with HIP events recorded on the stream it is launched on (the current
torch stream, which the binding passes to every call), inside the timed region.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

WORKLOADS = ["tiny", "mixtral_prefill", "finegrained_skewed", "decode_int4", "lora_prefill"]
HEADLINE = "mixtral_prefill"
# token sample of the CPU oracle per workload, and the host seconds it is repeated for (bounded so the
# five samples together take well under a minute)
CPU_SAMPLE = {"tiny": (64, 2.0), "mixtral_prefill": (4096, 8.0), "finegrained_skewed": (2048, 4.0),
              "decode_int4": (16, 3.0), "lora_prefill": (1024, 4.0)}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- algorithmic work
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


def fold_work(cfg, counts, lora_ids, fused=False):
    """Algorithmic work of the down-projection LoRA fold: per adapted real row, the Hs row read,
    the Ys row read and written (not when the fold runs in the down GEMM's epilogue, which writes
    Ys once anyway) and the bf16 xa row written and read back (at the padded rank the kernels run),
    plus the A_e and B_e of every adapted expert that has rows; FLOPs at the real rank
    (2 * rank * (I + H) per adapted real row)."""
    R, r = cfg.lora_max_rank, cfg.lora_rank
    ad = [int(e) for e in lora_ids if int(e) < len(counts) and counts[int(e)] > 0]
    rows = int(sum(int(counts[e]) for e in ad))
    ys = 0 if fused else 2 * cfg.H * 2
    bytes_ = rows * (cfg.I * 2 + ys + 2 * R * 2) + len(ad) * (R * cfg.I * 2 + cfg.H * R * 2)
    return float(2 * r * (cfg.I + cfg.H) * rows), float(bytes_), rows


def roofline(flops: float, bytes_: float, ms: float, peak_mfma: float, kernel: str, traffic=None):
    """Roofline object of one kernel: the bound is chosen from its arithmetic intensity against the
    ridge of the MFMA peak and HBM."""
    ai = flops / bytes_ if bytes_ else float("inf")
    if ai >= peak_mfma * 1e12 / (PEAK_HBM_GBS * 1e9):
        ach = flops / (ms / 1e3) / 1e12
        r = {"bound": "mfma", "achieved": ach, "peak": peak_mfma, "unit": "TFLOP/s"}
    else:
        ach = bytes_ / (ms / 1e3) / 1e9
        r = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    r["frac"] = r["achieved"] / r["peak"]
    r["traffic"] = traffic
    r["kernel"] = kernel
    r["ms"] = ms
    r["algorithmic"] = {"flops": flops, "bytes": bytes_, "flop_per_byte": ai}
    return r


# ----------------------------------------------------------------------------- helpers
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
    """HBM bytes per launch of one kernel from the committed FETCH_SIZE/WRITE_SIZE summary of
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
    # a role's own source list and hash when the summary gives them, else the file-wide ones
    files = kv.get(f"{role}.source_files", kv.get("source_files", "")).split()
    want = kv.get(f"{role}.source_sha256", kv.get("source_sha256"))
    if not files or not want or f"{role}.traffic_bytes" not in kv:
        return None
    h = hashlib.sha256()
    for f in files:
        p = os.path.join(ROOT, "mixture_experts_routed_route_amd", "csrc", f)
        if not os.path.exists(p):
            return None
        h.update(open(p, "rb").read())
    return float(kv[f"{role}.traffic_bytes"]) if h.hexdigest() == want else None


def host_cores() -> int:
    """Host cores this process may run on (the CPU oracle's BLAS uses up to that many threads)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(cfg, d, tokens: int, min_seconds: float, max_runs: int = 200):
    """The oracle as it stands, on the first ``tokens`` tokens of the same workload, run repeatedly
    until at least ``min_seconds`` of host time have passed (at most ``max_runs`` runs)."""
    import oracle
    from threadpoolctl import threadpool_info
    T = min(cfg.T, tokens)
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
    cores = host_cores()
    blas = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": runs * T / dt, "unit": "tokens/s", "cores": min(cores, blas), "kind": "oracle",
            "sample": f"{runs} run(s) of the first {T} of {cfg.T} tokens of {cfg.name}, whole layer (route, "
                      f"align, grouped GEMMs, {'LoRA fold, ' if cfg.lora_rank else ''}combine) in fp64 numpy; "
                      f"{dt:.1f} s in total; {cores} host cores available, BLAS threads {blas}"}


# ----------------------------------------------------------------------------- measured ceilings
def measure_ceilings(dev) -> dict:
    """What this chip delivers, measured beside the datasheet peaks: a 1 GiB device copy (torch's
    copy kernel; read + write bytes), a 2 GiB streaming read and a register-only bf16 MFMA loop
    (include/moe_probes.h).  Each is the best of five timed launches after one warm-up."""
    import torch
    import mixture_experts_routed_route_amd as m
    from mixture_experts_routed_route_amd._lib import check, lib

    def best(fn, n=5):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return min(ts)

    stream = torch.cuda.current_stream(dev).cuda_stream
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(3)
    dst = torch.empty_like(src)
    copy_ms = best(lambda: dst.copy_(src))
    del dst
    big = torch.empty(2 << 30, dtype=torch.uint8, device=dev).fill_(5)
    blocks = 256 * 8
    sink = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    read_ms = best(lambda: check(lib().moe_probe_stream_read(big.data_ptr(), big.numel(), sink.data_ptr(), blocks,
                                                             stream)))
    del big, src
    iters, mblocks = 20000, 512          # 2 workgroups of 4 waves per compute unit
    fsink = torch.empty(mblocks * 256, dtype=torch.float32, device=dev)
    mfma_ms = best(lambda: check(lib().moe_probe_mfma_bf16(iters, fsink.data_ptr(), mblocks, stream)))
    mfma_flops = mblocks * 4 * iters * 8 * 32768
    torch.cuda.synchronize()
    res = {"copy_GBs": 2 * (1 << 30) / (copy_ms / 1e3) / 1e9,
           "stream_read_GBs": (2 << 30) / (read_ms / 1e3) / 1e9,
           "mfma_bf16_TFLOPs": mfma_flops / (mfma_ms / 1e3) / 1e12,
           "how": "best of 5: 1 GiB torch device copy (read+write bytes); 2 GiB streaming read "
                  "(moe_probe_stream_read, 2048 workgroups); register-only 32x32x16 bf16 MFMA loop "
                  "(moe_probe_mfma_bf16, 2 workgroups of 4 waves per CU, pseudo-random operands)"}
    log(f"[bench] ceilings: copy {res['copy_GBs']:.0f} GB/s, stream read {res['stream_read_GBs']:.0f} GB/s, "
        f"MFMA bf16 {res['mfma_bf16_TFLOPs']:.0f} TFLOP/s")
    return res


# ----------------------------------------------------------------------------- one workload
def run_workload(name: str, args, dev) -> dict:
    import numpy as np
    import torch
    import mixture_experts_routed_route_amd as m
    from moe_synth import CONFIGS, make_inputs

    cfg = CONFIGS[name]
    log(f"[bench] {name}: generating inputs")
    d = make_inputs(cfg)
    layer = m.MoeLayer.from_arrays(d, dev, fold=args.fold, gate_up_fused=args.gate_up_lora == "fused",
                                   down_fused=args.down_lora == "fused")
    b = layer.plan(cfg.T, dev)
    wbytes = sum(expert_weight_bytes(cfg, op) for op in ("gate_up", "down")) * cfg.E
    rot = args.rotate or max(1, min(4, int(-(-(1 << 30) // wbytes))))
    layers = [layer] + [clone_layer(layer) for _ in range(rot - 1)]
    logits = torch.from_numpy(d["logits"]).to(dev)
    x = torch.from_numpy(d["x"]).view(torch.bfloat16).to(dev)
    torch.cuda.synchronize()
    has_fold = layer.lora is not None

    def step(i, ev=None):
        ly = layers[i % rot]
        ly.route_align(logits, b)
        if ev is not None:
            ev[0].record()
        ly.gate_up_stage(x, b)
        if ev is not None:
            ev[1].record()
        ly.down_stage(b)  # with the fused down fold: the LoRA shrink and the down GEMM that folds
        if ev is not None:
            ev[2].record()
        ly.lora_fold(b)
        if ev is not None:
            ev[3].record()
        ly.combine(b)

    # warmup: at least W steps and at least --warmup-seconds of GPU work, so that the timed steps run at
    # the steady state (clocks, caches and page tables settle after tens of milliseconds of work on
    # some workloads, not within a few steps)
    n_warm, t0 = 0, time.perf_counter()
    while n_warm < args.warmup or (time.perf_counter() - t0 < args.warmup_seconds and n_warm < 20000):
        step(n_warm)
        n_warm += 1
        if n_warm % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    log(f"[bench] {name}: warmup {n_warm} steps in {time.perf_counter() - t0:.2f} s")

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    # small batches are launch-bound: by default their steps replay from HIP graphs
    use_graph = args.graph or args.launch == "graph" or (args.launch == "auto" and cfg.T <= 64)
    if use_graph:
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
        log(f"[bench] {name}: timing {args.steps} graph replays")
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % rot].replay()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        log(f"[bench] {name}: per-kernel timing from an eager pass")
        for i in range(args.steps):
            step(i, events[i])
        torch.cuda.synchronize()
    else:
        log(f"[bench] {name}: timing {args.steps} steps")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i, events[i])
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
    ms = dt * 1e3 / args.steps
    gu_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    dn_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    fold_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in events])) if has_fold else None
    fused_fold = has_fold and layer.down_fold_fused(b)
    unfused = None
    if fused_fold:
        # the fused fold's cost: steps with the fold in the down GEMM's epilogue and steps with the
        # separate fold kernels after a plain down GEMM, alternating (so that clock and cache drift
        # fall on both alike); the fused fold's added time is its down stage over that plain GEMM
        def ab_step(i, fused, ev):
            for ly in layers:
                ly.down_fused = fused
            step(i, ev)
        for i in range(args.warmup):
            ab_step(i, False, None)
        torch.cuda.synchronize()
        ev_ab = {True: [], False: []}
        for i in range(2 * args.steps):
            fused = (i % 4) in (0, 3)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
            ev[4].record()
            ab_step(i // 2, fused, ev)
            ev[5].record()
            ev_ab[fused].append(ev)
        torch.cuda.synchronize()
        for ly in layers:
            ly.down_fused = True

        def mean(evs, a, c):
            return float(np.mean([e[a].elapsed_time(e[c]) for e in evs]))
        fused_down = mean(ev_ab[True], 1, 3)
        unfused = {"ms_per_step": mean(ev_ab[False], 4, 5), "down": mean(ev_ab[False], 1, 2),
                   "lora_fold": mean(ev_ab[False], 2, 3), "fused_ms_per_step": mean(ev_ab[True], 4, 5),
                   "fused_down_stage": fused_down,
                   "how": f"{args.steps} fused and {args.steps} unfused steps alternating, HIP events"}
        fold_ms = fused_down - unfused["down"]
        log(f"[bench] {name}: A/B of the down fold: fused step {unfused['fused_ms_per_step']:.3f} ms, unfused step "
            f"{unfused['ms_per_step']:.3f} ms; fused down stage {fused_down:.3f} ms against a plain down GEMM "
            f"{unfused['down']:.3f} ms + fold kernels {1e3 * unfused['lora_fold']:.1f} us")

    wt = {"bf16": "gemm_bf16_kernel", "fp8": "gemm_bf16_kernel (fp8 form)", "int4_gptq": "gemm_int4_kernel"}[cfg.weights]
    gu_what = ("gemm_bf16_kernel<gate_up> with the gate/up LoRA epilogue (+ 2 shrinks)"
               if layer.gate_up_lora and layer.gate_up_fused
               else "gate/up stage: 2 gathered GEMMs, 2 LoRA folds, SiLU*up" if layer.gate_up_lora
               else "gate/up stage: x quantisation + gemm_bf16_kernel<gate_up> (fp8 form)" if cfg.weights == "fp8"
               else f"{wt}<gate_up>")
    dn_what = ("down stage: Hs quantisation + gemm_bf16_kernel<down> (fp8 form)" if cfg.weights == "fp8"
               else "down stage: lora_shrink_kernel + gemm_bf16_kernel<down> with the LoRA epilogue" if fused_fold
               else f"{wt}<down>")
    peak_mfma = PEAK_FP8_TFLOPS if cfg.weights == "fp8" else PEAK_BF16_TFLOPS
    counts = b.routing.counts.cpu().numpy()
    active = int((counts > 0).sum())
    if has_fold:
        ff, fb, frows = fold_work(cfg, counts, d["lora_ids"], fused=fused_fold)
    dn_flops, dn_bytes = gemm_flops(cfg, "down"), gemm_bytes(cfg, "down", active)
    if fused_fold:   # the down stage also runs the shrink and the fold
        dn_flops, dn_bytes = dn_flops + ff, dn_bytes + fb
    roofs = {
        "gate_up": roofline(gemm_flops(cfg, "gate_up"), gemm_bytes(cfg, "gate_up", active), gu_ms, peak_mfma,
                            gu_what, measured_traffic(cfg.name, "gate_up")),
        "down": roofline(dn_flops, dn_bytes, dn_ms, peak_mfma, dn_what,
                         measured_traffic(cfg.name, "down_fused" if fused_fold else "down")),
    }
    if has_fold:
        mode = layer.fold_mode(b)
        what = ("the fold in the down GEMM's epilogue and lora_shrink_kernel: the fused down stage's time over "
                "the plain down GEMM's in the unfused steps of the same run" if fused_fold
                else "lora_shrink_kernel + lora_expand_fold_kernel" if mode == "grouped"
                else "gather_shrink_kernel + gather_expand_kernel")
        roofs["lora_fold"] = roofline(ff, fb, fold_ms, peak_mfma, what,
                                      None if fused_fold else measured_traffic(cfg.name, "lora_fold"))
        roofs["lora_fold"]["adapted_rows"] = frows
    gemm_tflops = (gemm_flops(cfg, "gate_up") + gemm_flops(cfg, "down")) / ((gu_ms + dn_ms) / 1e3) / 1e12
    log(f"[bench] {name}: step {ms:.3f} ms ({cfg.T / (ms / 1e3):.4g} tokens/s); gate/up {gu_ms:.3f} ms; "
        f"down {dn_ms:.3f} ms; grouped GEMMs {gemm_tflops:.1f} TFLOP/s"
        + (f"; LoRA fold ({'fused, added time' if fused_fold else layer.fold_mode(b)}) {1e3 * fold_ms:.1f} us"
           if fold_ms is not None else ""))
    for k, r in roofs.items():
        log(f"[bench] {name}: {k} roofline {r['bound']} {r['achieved']:.1f} {r['unit']} "
            f"({100 * r['frac']:.1f}% of peak), AI {r['algorithmic']['flop_per_byte']:.1f} flop/B")

    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.int16, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("[bench] copy calibration: 1 GiB device-to-device copy done")

    res = {
        "workload": cfg.name, "tokens": cfg.T, "hidden": cfg.H, "intermediate": cfg.I, "experts": cfg.E,
        "top_k": cfg.top_k, "block_size": cfg.block_size, "weights": cfg.weights, "lora_rank": cfg.lora_rank,
        **({"lora_fold": "fused" if fused_fold else layer.fold_mode(b)} if has_fold else {}),
        **({"lora_gate_up": "fused" if layer.gate_up_fused else "unfused"} if layer.gate_up_lora else {}),
        "launch": "hip_graph" if use_graph else "eager", "weight_copies_rotated": rot, "warmup_steps_run": n_warm,
        "active_experts": active,
        "tokens_per_s": cfg.T / (ms / 1e3), "ms_per_step": ms,
        "kernels_ms": {"gate_up": gu_ms, "down": dn_ms, **({"lora_fold": fold_ms} if has_fold else {})},
        **({"unfused_fold": unfused} if unfused else {}),
        "grouped_gemm_tflops": gemm_tflops,
        "roofline": roofs,
        "cpu_baseline": None,
    }
    del layers, layer, b, logits, x
    gc.collect()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        tok, secs = CPU_SAMPLE.get(name, (args.cpu_tokens or 1024, 4.0))
        if args.cpu_tokens:
            tok = args.cpu_tokens
        log(f"[bench] {name}: cpu oracle on {min(tok, cfg.T)} tokens")
        res["cpu_baseline"] = cpu_baseline(cfg, d, tok, secs)
        log(f"[bench] {name}: cpu oracle {res['cpu_baseline']['value']:.2f} tokens/s")
    del d
    gc.collect()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3, help="warmup steps per workload, at least")
    ap.add_argument("--warmup-seconds", type=float, default=0.3,
                    help="warmup per workload lasts at least this long (more steps than --warmup if needed)")
    ap.add_argument("--config", default="all", help="'all' (the five workloads, mixtral_prefill headline) or one name")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="token sample of the CPU oracle leg (0: per workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotate", type=int, default=0,
                    help="independent weight copies cycled through (0: enough for >= 1 GiB of weights, max 4)")
    ap.add_argument("--launch", default="auto", choices=["auto", "eager", "graph"],
                    help="time steps launched eagerly or replayed from HIP graphs (one captured step per weight "
                         "copy; the per-kernel figures then come from an eager pass of the same steps); auto: "
                         "graphs for batches of at most 64 tokens, whose steps are launch-bound")
    ap.add_argument("--graph", action="store_true", help="the same as --launch graph")
    ap.add_argument("--fold", default="auto", choices=["auto", "grouped", "gather"],
                    help="LoRA fold over the sorted rows or slot by slot (auto: by the padding share)")
    ap.add_argument("--down-lora", default="fused", choices=["fused", "unfused"],
                    help="down-projection LoRA fold in the down GEMM's epilogue where the fold runs over the sorted "
                         "rows (default), or the separate shrink and expand kernels")
    ap.add_argument("--gate-up-lora", default="fused", choices=["fused", "unfused"],
                    help="gate/up LoRA folded in the gate/up GEMM's epilogue, or the page's unfused order")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the copy / stream-read / MFMA-loop ceilings")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (reference for the FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures the single-GPU path only; --gpus {args.gpus} is not supported "
              "(multi-GPU expert/tensor parallel sharding is not part of this build)", file=sys.stderr)
        sys.exit(2)

    import torch
    from moe_synth import CONFIGS
    names = WORKLOADS if args.config == "all" else [args.config]
    for n in names:
        if n not in CONFIGS:
            sys.exit(f"unknown workload {n}; known: {', '.join(CONFIGS)}")
    dev = torch.device("cuda:0")
    ceilings = None if args.no_ceilings else measure_ceilings(dev)
    results = {}
    for n in names:
        results[n] = run_workload(n, args, dev)
    head = results[HEADLINE] if HEADLINE in results else results[names[0]]
    peak = PEAK_FP8_TFLOPS if head["weights"] == "fp8" else PEAK_BF16_TFLOPS
    gu = head["roofline"]["gate_up"]
    line = {
        "metric": "MoE layer tokens/s + grouped-GEMM TFLOP/s (% bf16 MFMA / HBM peak), 1 GPU",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_min_seconds": args.warmup_seconds,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8 e4m3 x fp8 e4m3, fp32 accumulate"}.get(
            head["weights"], "int4 weights x bf16, fp32 accumulate"),
        "data": "synthetic (seeded numpy PCG64; random-init expert weights)",
        "config": {k: head[k] for k in ("workload", "tokens", "hidden", "intermediate", "experts", "top_k",
                                         "block_size", "weights", "lora_rank", "launch")},
        "grouped_gemm_tflops": head["grouped_gemm_tflops"],
        "grouped_gemm_frac_mfma_peak": head["grouped_gemm_tflops"] / peak,
        "kernels_ms": head["kernels_ms"],
        "roofline": {k: gu[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic", "kernel",
                                        "algorithmic")},
        "cpu_baseline": head["cpu_baseline"],
        "ceilings": ceilings,
        "configs": results,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
