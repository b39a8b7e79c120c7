"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded inputs.

Bars: routing and alignment bit-exact; GEMM / fold / combine outputs within 2e-2
relative error per row (and over the whole tensor) against the fp64 oracle; sentinel
and padding rows never written.  Small workloads are checked on every row; the full
workloads are checked on every routing/alignment output and on sampled token rows.
"""
import sys

import numpy as np
import pytest

import oracle
from moe_synth import CONFIGS, MoeConfig, make_inputs, make_router_logits, f32_to_bf16_bits
from _util import (assert_close_rows, bf16_dev, bf16_host, bf16_ulp_diff, bits_host, close_rows_report, row_rel_err,
                   to_dev)

pytestmark = pytest.mark.gpu
TOL = 2e-2
CANARY = 0x7FC1  # a quiet-NaN bf16 pattern no kernel ever writes


def note(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import mixture_experts_routed_route_amd as m
    m.lib()  # raises if the library is missing: no fallback
    return torch.device("cuda:0")


def ops():
    import mixture_experts_routed_route_amd as m
    return m


# small workloads: several tiles, ragged K and N tails, skew, empty experts
SMALL = {
    "tiny": CONFIGS["tiny"],
    "mixtral_small": MoeConfig("mixtral_small", T=300, H=520, I=904, E=8, top_k=2, block_size=64, seed=1),
    "finegrained_small": MoeConfig("finegrained_small", T=700, H=256, I=192, E=128, top_k=8, block_size=64,
                                   logits="zipf", seed=2),
    "bs32_small": MoeConfig("bs32_small", T=257, H=384, I=136, E=16, top_k=4, block_size=32, seed=3),
    "bs128_small": MoeConfig("bs128_small", T=129, H=256, I=256, E=4, top_k=2, block_size=128, seed=4),
    "lora_small": MoeConfig("lora_small", T=200, H=512, I=256, E=16, top_k=6, block_size=64, lora_rank=16,
                            lora_max_rank=64, seed=5),
    "lora_all_small": MoeConfig("lora_all_small", T=200, H=512, I=256, E=16, top_k=6, block_size=64,
                                lora_rank=16, lora_max_rank=64, lora_gate_up=True, seed=8),
    "decode_int4": CONFIGS["decode_int4"],
    "decode_lora": CONFIGS["decode_lora"],
    "int4_prefill_small": MoeConfig("int4_prefill_small", T=100, H=512, I=256, E=8, top_k=2, block_size=32,
                                    weights="int4_gptq", group_size=128, seed=6),
    "int4_g64_small": MoeConfig("int4_g64_small", T=40, H=384, I=192, E=6, top_k=3, block_size=16,
                                weights="int4_gptq", group_size=64, seed=7),
}


# ----------------------------------------------------------------------------- A1 route
ROUTE_CASES = [(name, cfg) for name, cfg in CONFIGS.items()] + [
    ("E256_k8", MoeConfig("E256", T=1000, H=8, I=8, E=256, top_k=8, block_size=64, seed=11)),
    ("E200_k7", MoeConfig("E200", T=333, H=8, I=8, E=200, top_k=7, block_size=64, seed=12)),
    ("E1", MoeConfig("E1", T=17, H=8, I=8, E=1, top_k=1, block_size=16, seed=13)),
    ("k_eq_E", MoeConfig("kE", T=50, H=8, I=8, E=6, top_k=6, block_size=16, seed=14)),
    ("no_renorm", MoeConfig("nr", T=500, H=8, I=8, E=64, top_k=6, block_size=16, renormalize=False, seed=15)),
    # top_k above one wave's 64 lanes: selections 64.. live in the lanes' later slots
    ("E256_k96", MoeConfig("E256k96", T=70, H=8, I=8, E=256, top_k=96, block_size=64, seed=16)),
    ("E200_k130_no_renorm", MoeConfig("E200k130", T=33, H=8, I=8, E=200, top_k=130, block_size=16,
                                      renormalize=False, seed=17)),
    ("E256_k256", MoeConfig("E256k256", T=9, H=8, I=8, E=256, top_k=256, block_size=16, seed=18)),
    ("E128_k65", MoeConfig("E128k65", T=40, H=8, I=8, E=128, top_k=65, block_size=32, seed=19)),
    # at most 16 experts: one token per 16-lane row, a partial last block of rows
    ("E16_k4_ties", MoeConfig("E16", T=101, H=8, I=8, E=16, top_k=4, block_size=16, seed=41)),
    ("E13_k13_no_renorm", MoeConfig("E13", T=35, H=8, I=8, E=13, top_k=13, block_size=16, renormalize=False,
                                    seed=42)),
    ("E9_k3", MoeConfig("E9", T=18, H=8, I=8, E=9, top_k=3, block_size=16, seed=43)),
]


def _plant_ties(logits, E):
    """Exact ties, all-equal rows and -0.0 logits in the first rows."""
    logits[:20, min(7, E - 1)] = logits[:20, min(3, E - 1)]
    logits[20:30] = 0.0
    logits[30:35, : max(1, E // 2)] = -0.0


@pytest.mark.parametrize("name,cfg", ROUTE_CASES, ids=[c[0] for c in ROUTE_CASES])
def test_route_bit_exact(dev, name, cfg):
    note(f"route {name} T={cfg.T} E={cfg.E} k={cfg.top_k}")
    logits = make_router_logits(cfg)
    if name == "E256_k8":
        logits[:40, 7] = logits[:40, 3]           # exact ties
        logits[40:60] = 0.0                       # all equal
        logits[60:70, :128] = -0.0
    elif name.endswith("_ties"):
        _plant_ties(logits, cfg.E)
    ids_ref, w_ref = oracle.route(logits, cfg.top_k, cfg.renormalize)
    ids, w = ops().moe_route(to_dev(logits), cfg.top_k, cfg.renormalize)
    ids, w = ids.cpu().numpy(), w.cpu().numpy()
    assert np.array_equal(ids, ids_ref), f"{(ids != ids_ref).sum()} id mismatches"
    bad = np.flatnonzero(w.view(np.uint32) != w_ref.view(np.uint32))
    assert bad.size == 0, f"{bad.size} weight mismatches, first at {bad[:5]}: {w.ravel()[bad[:5]]} vs {w_ref.ravel()[bad[:5]]}"


# ----------------------------------------------------------------------------- A2 align
def _align_dev(ids_host, E, bs, max_pad=None):
    t = to_dev(np.ascontiguousarray(ids_host, dtype=np.int32))
    r = ops().moe_align(t, E, bs, max_pad)
    return {"counts": r.counts.cpu().numpy(), "offsets": r.offsets.cpu().numpy(),
            "sorted_ids": r.sorted_ids.cpu().numpy(), "expert_ids": r.expert_ids.cpu().numpy(),
            "total": int(r.total_padded.cpu().item()), "inv": r.inv_sorted.cpu().numpy()[: ids_host.size]}, r


def _assert_align_equal(got, ref):
    for key in ("counts", "offsets", "sorted_ids", "expert_ids", "inv"):
        a, b = got[key], ref[key]
        assert a.shape == b.shape and np.array_equal(a, b), f"{key}: {(a != b).sum()} mismatches"
    assert got["total"] == ref["total"]


@pytest.mark.parametrize("name", list(CONFIGS))
def test_align_bit_exact_configs(dev, name):
    cfg = CONFIGS[name]
    note(f"align {name} P={cfg.P} E={cfg.E} bs={cfg.block_size}")
    ids, _ = oracle.route(make_router_logits(cfg), cfg.top_k)
    got, _ = _align_dev(ids, cfg.E, cfg.block_size)
    _assert_align_equal(got, oracle.align(ids, cfg.E, cfg.block_size))


ALIGN_EDGE = [
    ("one_expert_all", lambda r: np.zeros((5000, 4), np.int32), 8, 64),
    ("chunk_plus_one", lambda r: r.integers(0, 3, (2049, 1)), 3, 16),
    ("many_chunks", lambda r: r.integers(0, 5, (50001, 4)), 5, 128),
    ("E256_bs128", lambda r: r.integers(0, 256, (3000, 8)), 256, 128),
    ("E256_sparse", lambda r: r.integers(0, 256, (7, 3)), 256, 16),
    ("invalid_ids", lambda r: r.integers(-3, 11, (999, 3)), 8, 32),
    ("single_pair", lambda r: np.array([[5]]), 6, 16),
]


@pytest.mark.parametrize("name,make,E,bs", ALIGN_EDGE, ids=[c[0] for c in ALIGN_EDGE])
def test_align_bit_exact_edges(dev, name, make, E, bs):
    ids = np.asarray(make(np.random.default_rng(sum(map(ord, name)))), dtype=np.int32)
    note(f"align edge {name} P={ids.size}")
    got, _ = _align_dev(ids, E, bs)
    _assert_align_equal(got, oracle.align(ids, E, bs))


def test_align_empty_and_oversized_capacity(dev):
    ids = np.zeros((0, 2), np.int32)
    got, _ = _align_dev(ids, 4, 16)
    ref = oracle.align(ids, 4, 16)
    _assert_align_equal(got, ref)
    ids = np.random.default_rng(0).integers(0, 8, (100, 2)).astype(np.int32)
    big = oracle.max_padded(200, 8, 16) + 5 * 16
    got, _ = _align_dev(ids, 8, 16, big)
    _assert_align_equal(got, oracle.align(ids, 8, 16, big))


# ----------------------------------------------------------------------------- shared stage setup
def _routing(cfg, d):
    ids, w = oracle.route(d["logits"], cfg.top_k, cfg.renormalize)
    al = oracle.align(ids, cfg.E, cfg.block_size)
    r = ops().moe_align(to_dev(ids.astype(np.int32)), cfg.E, cfg.block_size)  # bit-exact (tested above)
    return ids, w, al, r


def _weights_dev(d):
    return ops().MoeLayer.from_arrays(d, "cuda")


def _canary(rows, cols):
    import torch
    t = torch.full((rows, cols), CANARY, dtype=torch.int16, device="cuda")
    return t.view(torch.bfloat16)


def _real(al, P):
    return np.flatnonzero(al["sorted_ids"] < P)


# ----------------------------------------------------------------------------- A3 / A4 grouped GEMMs
@pytest.mark.parametrize("name", list(SMALL))
def test_grouped_gemms_small(dev, name):
    m = ops()
    cfg = SMALL[name]
    note(f"gemm {name}")
    d = make_inputs(cfg)
    ids, w, al, r = _routing(cfg, d)
    layer = _weights_dev(d)
    P = cfg.P
    real = _real(al, P)
    # gate/up + SiLU
    hs = _canary(r.max_pad, cfg.I)
    m.moe_grouped_gemm(m.MOE_OP_GATE_UP_SILU, bf16_dev(d["x"]), layer.gate, layer.up, r, out=hs)
    wg, wu, wd = oracle.moe_oracle._weights(d)
    h_ref = oracle.grouped_gate_up(d["x"], wg, wu, al, cfg.top_k)
    hs_b = bits_host(hs)
    assert (hs_b[np.setdiff1d(np.arange(r.max_pad), real)] == CANARY).all(), "padding rows of Hs written"
    assert_close_rows(bf16_host(hs)[real], h_ref[real], TOL, "gate/up")
    # down, fed with the oracle's own h rounded to bf16 (NaN in every padding row)
    h_in = np.full((r.max_pad, cfg.I), CANARY, np.uint16)
    h_in[real] = f32_to_bf16_bits(oracle.round_bf16(h_ref[real]).astype(np.float32))
    ys = _canary(r.max_pad, cfg.H)
    m.moe_grouped_gemm(m.MOE_OP_DOWN, bf16_dev(h_in), layer.down, None, r, out=ys)
    y_ref = oracle.grouped_down(oracle.bf16_bits_to_f64(h_in), wd, al)
    ys_b = bits_host(ys)
    assert (ys_b[np.setdiff1d(np.arange(r.max_pad), real)] == CANARY).all(), "padding rows of Ys written"
    assert_close_rows(bf16_host(ys)[real], y_ref[real], TOL, "down")


# Shapes whose tile counts make a workspace cut the last partial round of tiles along K (the
# split tail): on a 256-workgroup grid, T tiles leave T mod 256 tail tiles, split s ways when
# every XCD's share of them fits s times in its 32 workgroups and K holds s pieces of >= 8
# stages of 64.  Ragged K and N tails throughout.
SPLIT_K = {
    # 128-row tiles (85 rows per expert): gate/up 312 tiles (56 in the tail, 4 pieces), down 288
    # (32, 3 pieces)
    "rows128": MoeConfig("sk_128", T=1024, H=2824, I=1544, E=24, top_k=2, block_size=64, seed=31),
    # 256-row tiles: gate/up 272 tiles (16, 5 pieces); down 192 tiles, less than a round and
    # too many to split: whole tiles
    "rows256": MoeConfig("sk_256", T=1536, H=2824, I=2120, E=8, top_k=2, block_size=64, seed=33),
    # gate/up 144 tiles, not split; down 272 tiles (16 in the tail, 2 pieces of 8-9 stages)
    "rows256_min_pieces": MoeConfig("sk_256b", T=1536, H=4104, I=1032, E=8, top_k=2, block_size=64, seed=34),
    # less than a round: every tile is a tail tile, gate/up 128 tiles and down 80, in 2 pieces
    "all_tail": MoeConfig("sk_tail", T=1536, H=1032, I=1000, E=8, top_k=2, block_size=64, seed=35),
    # over 512 tiles on the 256-workgroup grid, so workgroups run several tiles and prepare the next
    # one inside the main loop, with segments of 3, 4 and 5 stages (the shortest that do):
    # gate/up 16 row tiles x 33 panels with K = 192 and 256; down 16 x 33 panels with K = 320
    "prefetch_k3": MoeConfig("pf_k3", T=1200, H=192, I=4104, E=8, top_k=2, block_size=64, seed=38),
    "prefetch_k4": MoeConfig("pf_k4", T=1200, H=256, I=4104, E=8, top_k=2, block_size=64, seed=39),
    "prefetch_down_k5": MoeConfig("pf_dn5", T=1200, H=8200, I=320, E=8, top_k=2, block_size=64, seed=40),
    # GPTQ int4 takes the workspace (size-checked) and does not use it: results as without it
    "int4_decode_g128": CONFIGS["decode_int4"],
    "int4_decode_g256": MoeConfig("sk_i4_256", T=16, H=2048, I=1536, E=64, top_k=6, block_size=16,
                                  weights="int4_gptq", group_size=256, seed=37),
}


@pytest.fixture(scope="module")
def shared_ws(dev):
    """One workspace for every split case, bf16 cases first: each call must leave the counters it
    used at zero, whatever kernel used the workspace before."""
    return ops().gemm_workspace("cuda")


@pytest.mark.parametrize("name", list(SPLIT_K))
def test_grouped_gemms_split_k_workspace(dev, shared_ws, name):
    """With and without the workspace, both GEMMs match the oracle on every real row; two calls
    that share the workspace give identical bits (the pieces of a split tile are summed in piece
    order, whatever their arrival order); the workspace counters are back at zero."""
    m = ops()
    cfg = SPLIT_K[name]
    note(f"gemm split-K {name} T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E}")
    d = make_inputs(cfg)
    ids, w, al, r = _routing(cfg, d)
    layer = _weights_dev(d)
    real = _real(al, cfg.P)
    pad = np.setdiff1d(np.arange(r.max_pad), real)
    ws = shared_ws
    wg, wu, wd = oracle.moe_oracle._weights(d)
    h_ref = oracle.grouped_gate_up(d["x"], wg, wu, al, cfg.top_k)
    h_in = np.full((r.max_pad, cfg.I), CANARY, np.uint16)
    h_in[real] = f32_to_bf16_bits(oracle.round_bf16(h_ref[real]).astype(np.float32))
    y_ref = oracle.grouped_down(oracle.bf16_bits_to_f64(h_in), wd, al)
    x_dev, h_dev = bf16_dev(d["x"]), bf16_dev(h_in)
    runs = []
    for use_ws in (False, True, True):
        hs = _canary(r.max_pad, cfg.I)
        m.moe_grouped_gemm(m.MOE_OP_GATE_UP_SILU, x_dev, layer.gate, layer.up, r, out=hs,
                           workspace=ws if use_ws else None)
        ys = _canary(r.max_pad, cfg.H)
        m.moe_grouped_gemm(m.MOE_OP_DOWN, h_dev, layer.down, None, r, out=ys, workspace=ws if use_ws else None)
        hs_b, ys_b = bits_host(hs), bits_host(ys)
        tag = "with workspace" if use_ws else "without workspace"
        assert (hs_b[pad] == CANARY).all() and (ys_b[pad] == CANARY).all(), f"padding rows written ({tag})"
        assert_close_rows(bf16_host(hs)[real], h_ref[real], TOL, f"gate/up {tag}")
        assert_close_rows(bf16_host(ys)[real], y_ref[real], TOL, f"down {tag}")
        runs.append((hs_b, ys_b))
    assert np.array_equal(runs[1][0], runs[2][0]) and np.array_equal(runs[1][1], runs[2][1])
    assert not ws[:4096].cpu().numpy().any(), "split counters not reset"


# ----------------------------------------------------------------------------- gathered projection + SiLU*up
GATHER_GEMM = {
    "bf16_128rows": SMALL["mixtral_small"],                                              # 4-wave tiles
    "bf16_256rows": MoeConfig("g256", T=1024, H=1032, I=776, E=8, top_k=2, block_size=64, seed=41),  # 8-wave
    "int4_decode": CONFIGS["decode_int4"],
    "int4_g64": SMALL["int4_g64_small"],
}


@pytest.mark.parametrize("name", list(GATHER_GEMM))
def test_gathered_projection_and_silu_mul(dev, shared_ws, name):
    """MOE_OP_GATHER: gate and up separately, no activation, x read by token; padding rows never
    written.  Then moe_silu_mul of those bf16 outputs against the oracle's bf16(silu(g) * u)."""
    m = ops()
    cfg = GATHER_GEMM[name]
    note(f"gathered projection {name}")
    d = make_inputs(cfg)
    ids, w, al, r = _routing(cfg, d)
    layer = _weights_dev(d)
    real = _real(al, cfg.P)
    pad = np.setdiff1d(np.arange(r.max_pad), real)
    wg, wu, wd = oracle.moe_oracle._weights(d)
    X = oracle.bf16_bits_to_f64(d["x"])
    outs = []
    for wdev, whost, what in ((layer.gate, wg, "gate"), (layer.up, wu, "up")):
        ref = np.full((r.max_pad, cfg.I), np.nan)
        for e, rr in oracle.moe_oracle._rows_by_expert(al).items():
            ref[rr] = X[al["sorted_ids"][rr] // cfg.top_k] @ oracle.expert_matrix(whost, e).T
        for ws in (None, shared_ws):
            c = _canary(r.max_pad, cfg.I)
            m.moe_grouped_gemm(m.MOE_OP_GATHER, bf16_dev(d["x"]), wdev, None, r, out=c, workspace=ws)
            cb = bits_host(c)
            assert (cb[pad] == CANARY).all(), f"padding rows of {what} written"
            assert_close_rows(bf16_host(c)[real], ref[real], TOL, f"{what} (workspace {ws is not None})")
        outs.append(c)
    g, u = outs
    h = _canary(r.max_pad, cfg.I)
    m.moe_silu_mul(g, u, h, r)
    hb = bits_host(h)
    assert (hb[pad] == CANARY).all(), "padding rows of Hs written"
    gf, uf = bf16_host(g)[real], bf16_host(u)[real]
    want = f32_to_bf16_bits(oracle.round_bf16(oracle.silu(gf) * uf).astype(np.float32))
    ulp = bf16_ulp_diff(hb[real], want)
    note(f"  silu_mul: exact {(ulp == 0).mean():.5f}, max ulp {ulp.max()}")
    assert ulp.max() <= 1 and (ulp == 0).mean() >= 0.999


def test_silu_mul_every_row(dev):
    """Without sorted ids every row is written (the slot-major layout), including large |gate|."""
    import torch
    m = ops()
    rng = np.random.default_rng(9)
    g = f32_to_bf16_bits((rng.standard_normal((37, 264)) * 6).astype(np.float32))
    g[0, :8] = f32_to_bf16_bits(np.float32([-100, -60, -20, 0, 20, 60, 100, -0.0]))
    u = f32_to_bf16_bits(rng.standard_normal((37, 264)).astype(np.float32))
    out = torch.empty((37, 264), dtype=torch.bfloat16, device="cuda")
    m.moe_silu_mul(bf16_dev(g), bf16_dev(u), out)
    gf, uf = oracle.bf16_bits_to_f64(g), oracle.bf16_bits_to_f64(u)
    want = f32_to_bf16_bits(oracle.round_bf16(oracle.silu(gf) * uf).astype(np.float32))
    ulp = bf16_ulp_diff(bits_host(out), want)
    assert ulp.max() <= 1 and (ulp == 0).mean() >= 0.999


@pytest.mark.parametrize("scale_mult", [1.0, 100.0])
def test_lora_fold_gate_up_form(dev, scale_mult):
    """The grouped fold with x_gather: token-major x, base = a sorted gate output."""
    m = ops()
    cfg = SMALL["lora_all_small"]
    d = make_inputs(cfg)
    d["lora_gate_scale"] = (d["lora_gate_scale"] * scale_mult).astype(np.float32)
    ids, w, al, r = _routing(cfg, d)
    real = _real(al, cfg.P)
    layer = m.MoeLayer.from_arrays(d, "cuda")
    rng = np.random.default_rng(23)
    base = np.full((r.max_pad, cfg.I), CANARY, np.uint16)
    base[real] = f32_to_bf16_bits(rng.standard_normal((real.size, cfg.I)).astype(np.float32))
    tabs = oracle.moe_oracle._lora_tables(d, "gate")
    X = oracle.bf16_bits_to_f64(d["x"])
    ref = oracle.lora_fold(oracle.bf16_bits_to_f64(base), X, tabs, al, cfg.top_k, x_gather=True)
    sd = oracle.lora_fold(np.zeros(base.shape), X, tabs, al, cfg.top_k, x_gather=True)
    got = bf16_dev(base)
    m.moe_lora_fold(bf16_dev(d["x"]), got, layer.lora_gate, r, x_gather=True)
    gb = bits_host(got)
    pad = np.setdiff1d(np.arange(r.max_pad), real)
    assert (gb[pad] == CANARY).all()
    adapted = np.array([rr for rr in real if (np.searchsorted(al["offsets"], rr, side="right") - 1) % 2 == 0])
    _gather_check(gb, ref, sd, base, adapted, f"gate/up form x{scale_mult}")
    others = np.setdiff1d(real, adapted)
    assert np.array_equal(gb[others], base[others])


@pytest.mark.parametrize("case", ["lora_all_small", "lora_all_256rows", "x100", "adapter",
                                  "max_rank_32_256rows", "max_rank_128_256rows", "max_rank_96",
                                  "prefetch_256rows"])
def test_gate_up_lora_fused_epilogue(dev, shared_ws, case):
    """The gate/up LoRA folded in the GEMM's epilogue against the oracle and against the
    unfused GPU path (gathered gate and up, folds, SiLU * up) on the same inputs, with max_rank
    32, 64, 96 and 128 (the epilogue's loop over the rank) on the 128- and 256-row kernels."""
    import torch
    m = ops()
    cfg = SMALL["lora_all_small"]
    if case in ("lora_all_256rows", "max_rank_32_256rows", "max_rank_128_256rows"):
        cfg = cfg.with_(T=1100, E=8, top_k=2, seed=9)   # >= 128 rows per expert: 256-row tiles
    elif case == "prefetch_256rows":   # 16 row tiles x 33 panels, K = 256: 4-stage segments, several
        cfg = cfg.with_(T=1100, E=8, top_k=2, H=256, I=4104, seed=10)   # tiles per workgroup
    if case == "max_rank_32_256rows":
        cfg = cfg.with_(lora_rank=24, lora_max_rank=32)
    elif case == "max_rank_128_256rows":
        cfg = cfg.with_(lora_rank=100, lora_max_rank=128)
    elif case == "max_rank_96":
        cfg = cfg.with_(lora_rank=80, lora_max_rank=96)
    note(f"gate/up lora fused {case}")
    d = make_inputs(cfg)
    if case == "x100":
        for proj in ("gate", "up"):
            d[f"lora_{proj}_scale"] = (d[f"lora_{proj}_scale"] * 100).astype(np.float32)
    ra = np.where(np.arange(cfg.T) % 4 == 1, -1, 0).astype(np.int32) if case == "adapter" else None
    ids, w, al, r = _routing(cfg, d)
    real = _real(al, cfg.P)
    layer = m.MoeLayer.from_arrays(d, "cuda")
    unf = m.MoeLayer.from_arrays(d, "cuda", gate_up_fused=False)
    outs = {}
    for name, lay in (("fused", layer), ("unfused", unf)):
        b = lay.plan(cfg.T, "cuda")
        lay.route_align(to_dev(d["logits"]), b)
        b.hs.view(torch.int16).fill_(CANARY)
        lay.gate_up_stage(bf16_dev(d["x"]), b, to_dev(ra) if ra is not None else None)
        torch.cuda.synchronize()
        outs[name] = bits_host(b.hs)
    pad = np.setdiff1d(np.arange(r.max_pad), real)
    assert (outs["fused"][pad] == CANARY).all(), "padding rows of Hs written"
    tg, tu = oracle.moe_oracle._lora_tables(d, "gate"), oracle.moe_oracle._lora_tables(d, "up")
    wg, wu, wd = oracle.moe_oracle._weights(d)
    fused = oracle.bf16_bits_to_f64(outs["fused"][real])
    unfused = oracle.bf16_bits_to_f64(outs["unfused"][real])
    assert_close_rows(fused, unfused, 1e-2, f"fused vs unfused ({case})", ulps=4)
    exact = (outs["fused"][real] == outs["unfused"][real]).mean()
    note(f"  fused == unfused bits on {exact:.4f} of the values")
    if ra is None:
        h = oracle.grouped_gate_up_lora(d["x"], wg, wu, al, cfg.top_k, tg, tu)
        assert_close_rows(fused, h[real], TOL, f"fused vs oracle ({case})", ulps=4)
    else:
        # tokens whose adapter entry is < 0 get the unfolded (bf16 gate and up) result
        h0 = oracle.grouped_gate_up_lora(d["x"], wg, wu, al, cfg.top_k, None, None)
        h1 = oracle.grouped_gate_up_lora(d["x"], wg, wu, al, cfg.top_k, tg, tu)
        skip = np.array([ra[al["sorted_ids"][rr] // cfg.top_k] < 0 for rr in real])
        want = np.where(skip[:, None], h0[real], h1[real])
        assert_close_rows(fused, want, TOL, f"fused vs oracle ({case})", ulps=4)


@pytest.mark.parametrize("fold", ["grouped", "gather"])
def test_layer_gate_up_lora(dev, fold):
    """The gate/up LoRA path in the layer: Hs from the GPU's own gate and up outputs folded and
    multiplied, stage by stage against the oracle; then the whole output."""
    import torch
    m = ops()
    cfg = SMALL["lora_all_small"]
    note(f"layer gate/up lora {fold}")
    d = make_inputs(cfg)
    layer = m.MoeLayer.from_arrays(d, "cuda", fold=fold, gate_up_fused=False)
    b = layer.plan(cfg.T, "cuda")
    layer.route_align(to_dev(d["logits"]), b)
    x = bf16_dev(d["x"])
    m.moe_grouped_gemm(m.MOE_OP_GATHER, x, layer.gate, None, b.routing, out=b.g)
    m.moe_grouped_gemm(m.MOE_OP_GATHER, x, layer.up, None, b.routing, out=b.u)
    torch.cuda.synchronize()
    g0, u0 = bits_host(b.g), bits_host(b.u)
    layer.gate_up_stage(x, b)          # the same GEMMs again, then the folds and SiLU * up
    ref = oracle.moe_layer(d)
    al = ref["align"]
    real = _real(al, cfg.P)
    X = oracle.bf16_bits_to_f64(d["x"])
    adapted = np.array([rr for rr in real if (np.searchsorted(al["offsets"], rr, side="right") - 1) % 2 == 0])
    for base0, got, proj in ((g0, b.g, "gate"), (u0, b.u, "up")):
        tabs = oracle.moe_oracle._lora_tables(d, proj)
        want = oracle.lora_fold(oracle.bf16_bits_to_f64(base0), X, tabs, al, cfg.top_k, x_gather=True)
        sd = oracle.lora_fold(np.zeros(base0.shape), X, tabs, al, cfg.top_k, x_gather=True)
        _gather_check(bits_host(got), want, sd, base0, adapted, f"{proj} fold ({fold})")
    gf, uf = bf16_host(b.g)[real], bf16_host(b.u)[real]
    want_h = f32_to_bf16_bits(oracle.round_bf16(oracle.silu(gf) * uf).astype(np.float32))
    assert bf16_ulp_diff(bits_host(b.hs)[real], want_h).max() <= 1
    assert_close_rows(bf16_host(b.hs)[real], ref["h"][real], TOL, "Hs against the oracle's", ulps=4)
    layer.down_stage(b)
    layer.lora_fold(b)
    out = layer.combine(b)
    assert_close_rows(bf16_host(out), ref["out"], TOL, f"layer gate/up lora {fold}")


# ----------------------------------------------------------------------------- fp8 prefill
FP8_SMALL = {
    # ragged K and N against the 128-wide tiles, one expert over several row tiles, empty experts
    "fp8_small": MoeConfig("fp8_small", T=300, H=528, I=912, E=8, top_k=2, block_size=64, weights="fp8", seed=51),
    "fp8_skewed": MoeConfig("fp8_skewed", T=500, H=256, I=384, E=32, top_k=4, block_size=32, weights="fp8",
                            logits="zipf", seed=52),
    # >= 128 rows per expert on average: 256-row tiles with 8 waves
    "fp8_big": MoeConfig("fp8_big", T=1024, H=528, I=912, E=4, top_k=2, block_size=64, weights="fp8", seed=53),
    # less than a round of tiles, K of 17 stages of 128: with the workspace every tile is a tail
    # tile cut in 2 pieces (gate/up here: 9 column panels, K = 2176)
    "fp8_split_gate_up": MoeConfig("fp8_split_gu", T=1024, H=2176, I=1040, E=4, top_k=2, block_size=64,
                                   weights="fp8", seed=54),
    # several tiles per workgroup, the next prepared inside the main loop: gate/up 16 row tiles x
    # 33 panels with K = 384 (3 stages of 128), down 16 x 33 panels with K = 384
    "fp8_prefetch_gate_up": MoeConfig("fp8_pf_gu", T=1200, H=384, I=4112, E=8, top_k=2, block_size=64,
                                      weights="fp8", seed=57),
    "fp8_prefetch_down": MoeConfig("fp8_pf_dn", T=1200, H=8208, I=384, E=8, top_k=2, block_size=64,
                                   weights="fp8", seed=58),
    # ... and down here (5 column panels of 256, K = 2176)
    "fp8_split_down": MoeConfig("fp8_split_dn", T=1024, H=1040, I=2176, E=4, top_k=2, block_size=64,
                                weights="fp8", seed=55),
}


@pytest.mark.parametrize("k", [1040, 3088, 6160, 14336, 16400])
def test_quantize_fp8_bit_exact(dev, k):
    """Codes and scales equal the oracle's bit for bit (every code is decided from the same fp32
    product); with sorted ids only real rows are written.  The widths select each form of the
    kernel: 1, 2, 4 and 8 chunks of 16 bytes held per thread (partly filled at 3088, 6160 and
    14336), and the two-pass form past 16384."""
    import torch
    m = ops()
    rng = np.random.default_rng(61)
    rows = 77
    x = f32_to_bf16_bits((rng.standard_normal((rows, k)) * np.exp(rng.uniform(-8, 8, (rows, 1)))).astype(np.float32))
    x[3] = 0                                        # all-zero row
    x[5, :] = f32_to_bf16_bits(np.float32(1.5))     # constant row: every code is +448
    x[6, ::7] = f32_to_bf16_bits(np.float32(-2.0 ** -120))
    q = torch.empty((rows, k), dtype=torch.uint8, device="cuda")
    sc = torch.empty(rows, dtype=torch.float32, device="cuda")
    m.moe_quantize_fp8(bf16_dev(x), q, sc)
    want_q, want_s = oracle.quantize_rows_fp8(oracle.bf16_bits_to_f64(x))
    got_q = q.cpu().numpy()
    note(f"quantize: {(got_q != want_q).sum()} codes differ")
    assert np.array_equal(got_q, want_q)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    # sorted rows: sentinel rows keep their canary bytes and scales
    cfg = FP8_SMALL["fp8_skewed"]
    d = make_inputs(cfg)
    ids, w, al, r = _routing(cfg, d)
    real = _real(al, cfg.P)
    hs = f32_to_bf16_bits(rng.standard_normal((r.max_pad, 96)).astype(np.float32))
    q2 = torch.full((r.max_pad, 96), 0xA5, dtype=torch.uint8, device="cuda")
    s2 = torch.full((r.max_pad,), -7.0, dtype=torch.float32, device="cuda")
    m.moe_quantize_fp8(bf16_dev(hs), q2, s2, r)
    wq, ws = oracle.quantize_rows_fp8(oracle.bf16_bits_to_f64(hs[real]))
    gq, gs = q2.cpu().numpy(), s2.cpu().numpy()
    assert np.array_equal(gq[real], wq) and np.array_equal(gs[real], ws)
    pad = np.setdiff1d(np.arange(r.max_pad), real)
    assert (gq[pad] == 0xA5).all() and (gs[pad] == -7.0).all()


@pytest.mark.parametrize("name", list(FP8_SMALL))
def test_grouped_gemm_fp8(dev, shared_ws, name):
    """Both fp8 GEMMs against the oracle on the oracle's own codes and scales (so only the GEMM
    is compared), without and with the split-tail workspace; sentinel and padding rows are never
    written; two calls with the workspace give the same bits; its counters end at zero."""
    import torch
    m = ops()
    cfg = FP8_SMALL[name]
    note(f"gemm fp8 {name}")
    d = make_inputs(cfg)
    ids, w, al, r = _routing(cfg, d)
    layer = _weights_dev(d)
    real = _real(al, cfg.P)
    pad = np.setdiff1d(np.arange(r.max_pad), real)
    ref = oracle.moe_layer(d)
    xq, sx = ref["xq"], ref["sx"]
    hq = np.zeros((r.max_pad, cfg.I), np.uint8)
    sh = np.ones(r.max_pad, np.float32)
    hq[real], sh[real] = ref["hq"][real], ref["sh"][real]
    runs = []
    for ws in (None, shared_ws, shared_ws):
        tag = "with workspace" if ws is not None else "without workspace"
        hs = _canary(r.max_pad, cfg.I)
        m.moe_grouped_gemm_fp8(m.MOE_OP_GATE_UP_SILU, to_dev(xq), to_dev(sx), layer.gate, layer.up, r, out=hs,
                               workspace=ws)
        hb = bits_host(hs)
        assert (hb[pad] == CANARY).all(), f"padding rows of Hs written ({tag})"
        e1, e2 = assert_close_rows(bf16_host(hs)[real], ref["h"][real], TOL, f"fp8 gate/up ({tag})")
        note(f"  gate/up worst row {e1:.2e} ({tag})")
        ys = _canary(r.max_pad, cfg.H)
        m.moe_grouped_gemm_fp8(m.MOE_OP_DOWN, to_dev(hq), to_dev(sh), layer.down, None, r, out=ys, workspace=ws)
        yb = bits_host(ys)
        assert (yb[pad] == CANARY).all(), f"padding rows of Ys written ({tag})"
        e1, e2 = assert_close_rows(bf16_host(ys)[real], ref["y"][real], TOL, f"fp8 down ({tag})")
        note(f"  down worst row {e1:.2e} ({tag})")
        runs.append((hb, yb))
    assert np.array_equal(runs[1][0], runs[2][0]) and np.array_equal(runs[1][1], runs[2][1])
    assert not shared_ws[:4096].cpu().numpy().any(), "split counters not reset"


@pytest.mark.parametrize("name", list(FP8_SMALL))
def test_layer_fp8_end_to_end(dev, name):
    """The fp8 layer stage by stage on the GPU's own intermediates, each stage to the usual bar
    (codes bit-exact; GEMMs and combine within 2e-2 per row and per element of the row's rms):
    those are the gate.  Against the fully independent oracle the figures are only reported: where
    the GPU's bf16 Hs differs from the oracle's in the last bit, an e4m3 code of the down GEMM's
    input can round the other way, so the two chains see different fp8 inputs."""
    cfg = FP8_SMALL[name]
    d = make_inputs(cfg)
    layer, b, out = _layer_run(cfg, d)
    ref = oracle.moe_layer(d)
    al = ref["align"]
    real = _real(al, cfg.P)
    assert np.array_equal(b.ids.cpu().numpy(), ref["ids"])
    assert np.array_equal(b.xq.cpu().numpy(), ref["xq"]) and np.array_equal(b.sx.cpu().numpy(), ref["sx"])
    assert_close_rows(bf16_host(b.hs)[real], ref["h"][real], TOL, f"{name} Hs")
    hs_gpu = bf16_host(b.hs)
    hq, sh = oracle.quantize_rows_fp8(hs_gpu[real])
    assert np.array_equal(b.hq.cpu().numpy()[real], hq) and np.array_equal(b.sh.cpu().numpy()[real], sh)
    hq_full = np.zeros((len(al["sorted_ids"]), cfg.I), np.uint8)
    sh_full = np.ones(len(al["sorted_ids"]), np.float32)
    hq_full[real], sh_full[real] = hq, sh
    y_chain = oracle.grouped_down_fp8(hq_full, sh_full, d["fp8_down"], al)
    assert_close_rows(bf16_host(b.ys)[real], y_chain[real], TOL, f"{name} Ys on the GPU's codes")
    out_chain = oracle.combine(bf16_host(b.ys), al["inv"], ref["w"], cfg.T, cfg.top_k)
    assert_close_rows(bf16_host(out), out_chain, TOL, f"{name} combine")
    e1, e2, e3 = close_rows_report(bf16_host(out), ref["out"])
    note(f"layer fp8 {name}: against the independent oracle (report) worst row {e1:.2e}, tensor {e2:.2e}, "
         f"worst |diff|/rms(row) {e3:.2e}")


def test_layer_fp8_with_down_lora(dev):
    """fp8 experts with a down-projection LoRA (the fold reads the bf16 Hs the fp8 gate/up wrote):
    the folded Ys rows against the oracle fold of the GPU's own Hs and unfolded Ys (the gate), and
    the output against the independent oracle (reported)."""
    import torch
    m = ops()
    cfg = MoeConfig("fp8_lora", T=200, H=512, I=256, E=16, top_k=6, block_size=64, weights="fp8", lora_rank=16,
                    lora_max_rank=64, seed=56)
    d = make_inputs(cfg)
    d["lora_scale"] = (d["lora_scale"] * 20).astype(np.float32)   # a fold well above the fp8 noise
    layer = m.MoeLayer.from_arrays(d, "cuda")
    b = layer.plan(cfg.T, "cuda")
    layer.route_align(to_dev(d["logits"]), b)
    lora, layer.lora = layer.lora, None
    layer.experts(bf16_dev(d["x"]), b)
    layer.lora = lora
    torch.cuda.synchronize()
    hs, ys0 = bits_host(b.hs), bits_host(b.ys)
    layer.lora_fold(b)
    out = layer.combine(b)
    ref = oracle.moe_layer(d)
    al = ref["align"]
    real = _real(al, cfg.P)
    tabs = oracle.moe_oracle._lora_tables(d)
    hs_f = np.where(np.isin(np.arange(hs.shape[0]), real)[:, None], oracle.bf16_bits_to_f64(hs), 0.0)
    want = oracle.lora_fold(oracle.bf16_bits_to_f64(ys0), hs_f, tabs, al, cfg.top_k)
    sd = oracle.lora_fold(np.zeros(ys0.shape), hs_f, tabs, al, cfg.top_k)
    adapted = np.array([rr for rr in real if (np.searchsorted(al["offsets"], rr, side="right") - 1) % 2 == 0])
    _gather_check(bits_host(b.ys), want, sd, ys0, adapted, "fp8 layer down fold")
    out_chain = oracle.combine(bf16_host(b.ys), al["inv"], ref["w"], cfg.T, cfg.top_k)
    assert_close_rows(bf16_host(out), out_chain, TOL, "fp8 + LoRA combine of the GPU's Ys")
    e1, e2, e3 = close_rows_report(bf16_host(out), ref["out"])
    note(f"fp8 + LoRA layer against the independent oracle (report): worst row {e1:.2e}, elementwise {e3:.2e}")


# ----------------------------------------------------------------------------- A6 combine
@pytest.mark.parametrize("name", ["tiny", "finegrained_small", "mixtral_small"])
def test_combine(dev, name):
    m = ops()
    cfg = SMALL[name]
    d = make_inputs(cfg)
    ids, w, al, r = _routing(cfg, d)
    rng = np.random.default_rng(9)
    y = rng.standard_normal((r.max_pad, cfg.H)).astype(np.float32)
    y_bits = f32_to_bf16_bits(y)
    out = m.moe_combine(bf16_dev(y_bits), r.inv_sorted[: cfg.P], to_dev(w))
    ref = oracle.combine(oracle.bf16_bits_to_f64(y_bits), al["inv"], w, cfg.T, cfg.top_k)
    assert_close_rows(bf16_host(out), ref, TOL, "combine")
    ulp = bf16_ulp_diff(bits_host(out), f32_to_bf16_bits(oracle.round_bf16(ref).astype(np.float32)))
    assert ulp.max() <= 1 and (ulp == 0).mean() > 0.99
    # slot-major (no inverse map)
    out2 = m.moe_combine(bf16_dev(y_bits[: cfg.P]), None, to_dev(w))
    ref2 = oracle.combine(oracle.bf16_bits_to_f64(y_bits[: cfg.P]), None, w, cfg.T, cfg.top_k)
    assert_close_rows(bf16_host(out2), ref2, TOL, "combine slot-major")
    # a dropped pair contributes nothing
    inv = al["inv"].copy()
    inv[::3] = -1
    out3 = m.moe_combine(bf16_dev(y_bits), to_dev(inv), to_dev(w))
    ref3 = oracle.combine(oracle.bf16_bits_to_f64(y_bits), inv, w, cfg.T, cfg.top_k)
    assert_close_rows(bf16_host(out3), ref3, TOL, "combine dropped")


# ----------------------------------------------------------------------------- A5 LoRA fold
def _fold_setup(cfg, scale_mult=1.0):
    d = make_inputs(cfg)
    if scale_mult != 1.0:
        d["lora_scale"] = (d["lora_scale"] * scale_mult).astype(np.float32)
    ids, w, al, r = _routing(cfg, d)
    P = cfg.P
    real = _real(al, P)
    rng = np.random.default_rng(21)
    x = np.full((r.max_pad, cfg.I), CANARY, np.uint16)
    x[real] = f32_to_bf16_bits(rng.standard_normal((real.size, cfg.I)).astype(np.float32))
    base = np.full((r.max_pad, cfg.H), CANARY, np.uint16)
    base[real] = f32_to_bf16_bits((rng.standard_normal((real.size, cfg.H)) * 0.05).astype(np.float32))
    return d, al, r, real, x, base


@pytest.mark.parametrize("scale_mult", [1.0, 100.0])
def test_lora_fold_stage(dev, scale_mult):
    m = ops()
    cfg = SMALL["lora_small"]
    d, al, r, real, x, base = _fold_setup(cfg, scale_mult)
    layer = _weights_dev(d)
    tabs = oracle.moe_oracle._lora_tables(d)
    ref = oracle.lora_fold(oracle.bf16_bits_to_f64(base), oracle.bf16_bits_to_f64(x), tabs, al, cfg.top_k)
    ref_bits = np.full_like(base, CANARY)
    ref_bits[real] = f32_to_bf16_bits(ref[real].astype(np.float32))
    got = bf16_dev(base)
    m.moe_lora_fold(bf16_dev(x), got, layer.lora, r)
    gb = bits_host(got)
    pad = np.setdiff1d(np.arange(r.max_pad), real)
    assert (gb[pad] == CANARY).all(), "padding rows of the base written"
    ulp = bf16_ulp_diff(gb[real], ref_bits[real])
    note(f"fold x{scale_mult}: exact {(ulp == 0).mean():.5f}, max ulp {ulp.max()}")
    assert ulp.max() <= 1 and (ulp == 0).mean() >= 0.999
    # unadapted experts (odd ids) are bit-identical to the base
    changed = np.any(gb != base, axis=1)
    for rr in np.flatnonzero(changed):
        e = np.searchsorted(al["offsets"], rr, side="right") - 1
        assert e % 2 == 0, f"row {rr} of unadapted expert {e} changed"
    assert changed.sum() > 0


def test_lora_fold_windows_bit_identical(dev):
    m = ops()
    cfg = SMALL["lora_small"]
    d, al, r, real, x, base = _fold_setup(cfg)
    layer = _weights_dev(d)
    one = bf16_dev(base)
    m.moe_lora_fold(bf16_dev(x), one, layer.lora, r)
    for cap in (100, 64, 1000, 17):
        chunked = bf16_dev(base)
        import torch
        xa = torch.empty((cap, layer.lora.max_rank), dtype=torch.bfloat16, device="cuda")
        for s, e in m.lora_windows(r.max_pad, cap):
            m.moe_lora_fold(bf16_dev(x), chunked, layer.lora, r, xa=xa, row_offset=s, row_end=e)
        assert np.array_equal(bits_host(chunked), bits_host(one)), f"cap {cap}"


def test_lora_fold_row_adapter(dev):
    m = ops()
    cfg = SMALL["lora_small"]
    d, al, r, real, x, base = _fold_setup(cfg)
    layer = _weights_dev(d)
    ra = np.where(np.arange(cfg.T) % 3 == 0, -1, 0).astype(np.int32)
    tabs = oracle.moe_oracle._lora_tables(d)
    ref = oracle.lora_fold(oracle.bf16_bits_to_f64(base), oracle.bf16_bits_to_f64(x), tabs, al, cfg.top_k,
                           row_adapter=ra)
    got = bf16_dev(base)
    m.moe_lora_fold(bf16_dev(x), got, layer.lora, r, row_adapter=to_dev(ra))
    gb = bits_host(got)
    ulp = bf16_ulp_diff(gb[real], f32_to_bf16_bits(ref[real].astype(np.float32)))
    assert ulp.max() <= 1 and (ulp == 0).mean() >= 0.999
    skipped = [rr for rr in real if ra[al["sorted_ids"][rr] // cfg.top_k] < 0]
    assert np.array_equal(gb[skipped], base[skipped])


# ----------------------------------------------------------------------------- A5 gather fold (decode form)
# (name, tokens, top_k, experts, k_in, n_out, max_rank, real rank, x_gather, scale multiplier, adapter map)
GATHER_CASES = [
    ("decode_down", 16, 6, 64, 1408, 2048, 64, 16, 0, 1.0, False),
    ("decode_gate_up", 16, 6, 64, 2048, 1408, 64, 16, 1, 1.0, False),
    ("decode_down_x100", 16, 6, 64, 1408, 2048, 64, 16, 0, 100.0, False),
    ("ragged_r32_adapter", 7, 3, 10, 72, 264, 32, 32, 0, 1.0, True),
    ("ragged_r96_gather", 9, 2, 5, 200, 520, 96, 80, 1, 1.0, True),
    ("r128_k4", 33, 4, 12, 640, 136, 128, 128, 0, 1.0, False),
    ("one_slot", 1, 1, 1, 40, 8, 32, 8, 1, 1.0, False),
]


def _gather_setup(T, k, E, k_in, n_out, R, r, scale_mult, seed):
    """Router ids (with a dropped and an out-of-table id), tables for the even experts, bf16 x and base."""
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, _ = oracle.route(logits, k)
    ids = ids.reshape(-1).copy()
    if ids.size > 5:
        ids[1], ids[4] = -1, E + 2
    adapted = list(range(0, E, 2))
    a_l, b_l, s_l = [], [], []
    for _ in adapted:
        a = np.zeros((R, k_in), np.uint16)
        a[:r] = f32_to_bf16_bits((rng.standard_normal((r, k_in)) * 0.01).astype(np.float32))
        b = np.zeros((n_out, R), np.uint16)
        b[:, :r] = f32_to_bf16_bits((rng.standard_normal((n_out, r)) * 0.01).astype(np.float32))
        a_l.append(a), b_l.append(b), s_l.append(float(np.float32(rng.uniform(0.5, 2.0) * scale_mult)))
    return rng, ids.astype(np.int32), adapted, a_l, b_l, s_l


def _gather_dev_tables(adapted, a_l, b_l, s_l):
    m = ops()
    return m.pack_lora_tables(adapted, [bf16_dev(a) for a in a_l], [bf16_dev(b) for b in b_l], s_l, "cuda")


def _gather_check(got_bits, ref, scaled_delta, base_bits, rows, what):
    """At least 99.9% of the folded values bit-exact; every one within 3 bf16 ulps of the largest
    of |base|, |result| and |scale * delta|.  The kernel sums in fp32 in another order than the
    oracle, so an xa or delta value next to a rounding boundary may round the other way: a delta
    one ulp off moves scale * delta by under 2 ulps of itself, and the result rounds once more.
    Where base and scale * delta cancel, this is many ulps of the small result."""
    g = oracle.bf16_bits_to_f64(got_bits[rows])
    r = ref[rows]
    m = np.maximum(np.maximum(np.abs(oracle.bf16_bits_to_f64(base_bits[rows])), np.abs(r)),
                   np.abs(scaled_delta[rows]))
    _, ex = np.frexp(m)
    ulp_m = np.ldexp(1.0, np.maximum(ex - 8, -133))
    worst = (np.abs(g - r) / ulp_m).max()
    exact = (g == r).mean()
    note(f"{what}: exact {exact:.5f}, max |diff| {worst:.2f} ulp of the largest term")
    assert worst <= 3 and exact >= 0.999, what


@pytest.mark.parametrize("case", GATHER_CASES, ids=[c[0] for c in GATHER_CASES])
def test_lora_gather_fold_slot_major(dev, case):
    m = ops()
    name, T, k, E, k_in, n_out, R, r, xg, smult, use_ra = case
    note(f"gather fold {name}")
    rng, ids, adapted, a_l, b_l, s_l = _gather_setup(T, k, E, k_in, n_out, R, r, smult, seed=31 + len(name))
    n = T * k
    x = f32_to_bf16_bits(rng.standard_normal((T if xg else n, k_in)).astype(np.float32))
    base = f32_to_bf16_bits((rng.standard_normal((n, n_out)) * 0.05).astype(np.float32))
    ra = np.where(np.arange(T) % 3 == 1, -1, 0).astype(np.int32) if use_ra else None
    tabs = oracle.pack_expert_tables([(e, a, b, sc) for e, a, b, sc in zip(adapted, a_l, b_l, s_l)])
    ref = oracle.lora_gather_fold(oracle.bf16_bits_to_f64(base), oracle.bf16_bits_to_f64(x), tabs, ids, k,
                                  x_gather=bool(xg), row_adapter=ra)
    sd = oracle.lora_gather_fold(np.zeros(base.shape), oracle.bf16_bits_to_f64(x), tabs, ids, k,
                                 x_gather=bool(xg), row_adapter=ra)
    got = bf16_dev(base)
    m.moe_lora_gather_fold(bf16_dev(x), got, _gather_dev_tables(adapted, a_l, b_l, s_l), to_dev(ids), k,
                           x_gather=bool(xg), row_adapter=to_dev(ra) if ra is not None else None)
    gb = bits_host(got)
    folded = np.array([0 <= e < tabs[3] and e % 2 == 0 and (ra is None or ra[s // k] >= 0)
                       for s, e in enumerate(ids)])
    assert folded.any()
    assert np.array_equal(gb[~folded], base[~folded]), "a skipped slot changed"
    _gather_check(gb, ref, sd, base, np.flatnonzero(folded), name)


def test_lora_gather_fold_row_map_on_sorted_buffers(dev):
    """Through the inverse map the gather fold updates the sorted buffers of the grouped path:
    padding rows and the rows of dropped pairs stay untouched."""
    m = ops()
    T, k, E, k_in, n_out, R, r = 24, 6, 16, 256, 512, 64, 16
    rng, ids, adapted, a_l, b_l, s_l = _gather_setup(T, k, E, k_in, n_out, R, r, 1.0, seed=77)
    al = oracle.align(ids, E, 16)
    rows = len(al["sorted_ids"])
    x = np.full((rows, k_in), CANARY, np.uint16)
    base = np.full((rows, n_out), CANARY, np.uint16)
    real = np.flatnonzero(al["sorted_ids"] < ids.size)
    x[real] = f32_to_bf16_bits(rng.standard_normal((real.size, k_in)).astype(np.float32))
    base[real] = f32_to_bf16_bits((rng.standard_normal((real.size, n_out)) * 0.05).astype(np.float32))
    tabs = oracle.pack_expert_tables([(e, a, b, sc) for e, a, b, sc in zip(adapted, a_l, b_l, s_l)])
    ref = oracle.lora_gather_fold(oracle.bf16_bits_to_f64(base), oracle.bf16_bits_to_f64(x), tabs, ids, k,
                                  row_map=al["inv"])
    sd = oracle.lora_gather_fold(np.zeros(base.shape), oracle.bf16_bits_to_f64(x), tabs, ids, k,
                                 row_map=al["inv"])
    got = bf16_dev(base)
    m.moe_lora_gather_fold(bf16_dev(x), got, _gather_dev_tables(adapted, a_l, b_l, s_l), to_dev(ids), k,
                           row_map=to_dev(al["inv"]))
    gb = bits_host(got)
    mapped = np.array([int(al["inv"][s]) for s, e in enumerate(ids) if 0 <= e < tabs[3] and e % 2 == 0])
    untouched = np.setdiff1d(np.arange(rows), mapped)
    assert np.array_equal(gb[untouched], base[untouched])
    _gather_check(gb, ref, sd, base, mapped, "row_map")
    # the grouped fold on the same buffers gives the oracle's result too
    import torch
    routing = m.Routing.allocate(ids.size, k, E, 16, "cuda")
    m.moe_align(to_dev(ids.reshape(T, k)), E, 16, out=routing)
    grouped = bf16_dev(base)
    m.moe_lora_fold(bf16_dev(x), grouped, _gather_dev_tables(adapted, a_l, b_l, s_l), routing)
    _gather_check(bits_host(grouped), ref, sd, base, mapped, "grouped fold, same rows")


def test_lora_gather_fold_no_slots(dev):
    import torch
    m = ops()
    rng, ids, adapted, a_l, b_l, s_l = _gather_setup(2, 2, 4, 64, 64, 32, 8, 1.0, seed=3)
    base = bf16_dev(f32_to_bf16_bits(np.ones((4, 64), np.float32)))
    m.moe_lora_gather_fold(bf16_dev(np.zeros((4, 64), np.uint16)), base,
                           _gather_dev_tables(adapted, a_l, b_l, s_l), torch.empty(0, dtype=torch.int32,
                                                                                   device="cuda"), 2)
    torch.cuda.synchronize()
    assert (bits_host(base) == f32_to_bf16_bits(np.float32(1.0))).all()


# ----------------------------------------------------------------------------- whole layer
def _layer_run(cfg, d):
    m = ops()
    layer = m.MoeLayer.from_arrays(d, "cuda")
    b = layer.plan(cfg.T, "cuda")
    out = layer.forward(to_dev(d["logits"]), bf16_dev(d["x"]), b)
    return layer, b, out


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_end_to_end_small(dev, name):
    cfg = SMALL[name]
    note(f"layer {name}")
    d = make_inputs(cfg)
    layer, b, out = _layer_run(cfg, d)
    ref = oracle.moe_layer(d)
    assert np.array_equal(b.ids.cpu().numpy(), ref["ids"])
    assert_close_rows(bf16_host(out), ref["out"], TOL, f"layer {name}")


@pytest.mark.slow
@pytest.mark.parametrize("name", list(CONFIGS))
def test_layer_full_size_sampled(dev, name):
    cfg = CONFIGS[name]
    note(f"layer full {name}")
    d = make_inputs(cfg)
    layer, b, out = _layer_run(cfg, d)
    ids, w = oracle.route(d["logits"], cfg.top_k, cfg.renormalize)
    assert np.array_equal(b.ids.cpu().numpy(), ids)
    assert np.array_equal(b.w.cpu().numpy().view(np.uint32), w.view(np.uint32))
    al = oracle.align(ids, cfg.E, cfg.block_size)
    assert np.array_equal(b.routing.sorted_ids.cpu().numpy(), al["sorted_ids"])
    # sampled tokens: first, last, and a spread in between (and the busiest expert's rows)
    rng = np.random.default_rng(0)
    n = min(cfg.T, 24)
    toks = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, n, replace=False)]))
    ref = oracle.moe_tokens(d, toks, (ids, w))
    got = bf16_host(out)[toks]
    if cfg.weights == "fp8":
        # the fp8 chain is gated stage by stage (test_grouped_gemms_full_size_rows); end to end it is
        # reported (the two chains may quantise a last-bit-different Hs element differently)
        out_chain = oracle.combine(bf16_host(b.ys), al["inv"], w, cfg.T, cfg.top_k)
        assert_close_rows(got, out_chain[toks], TOL, f"layer full {name}: combine of the GPU's Ys")
        e1, e2, e3 = close_rows_report(got, ref)
        note(f"  against the independent oracle (report): worst row {e1:.2e}, tensor {e2:.2e}, elementwise {e3:.2e}")
    else:
        e1, e2 = assert_close_rows(got, ref, TOL, f"layer full {name}")
        note(f"  worst row rel err {e1:.2e}, tensor {e2:.2e}")


def _selected_rows(al, P, BM, N, K, gate_up, grid, split):
    """Sorted rows a full-size stage check evaluates: the first and last real row of every active
    expert and the first row of its last tile, up to 16 rows (both ends included) of the busiest
    expert's last tile, and first / middle / last real rows of every row tile that holds a piece of
    the split tail (the restated schedule of test_gemm_addressing)."""
    from test_gemm_addressing import _decode_tile, _split_tail_segments
    off, cnt = al["offsets"], al["counts"]
    E = len(cnt)
    rows = set()
    spans = []
    for e in range(E):
        nt = -(-(int(off[e + 1]) - int(off[e])) // BM)
        spans.append((e, nt))
        if cnt[e] == 0:
            continue
        lo, last = int(off[e]), int(off[e]) + int(cnt[e]) - 1
        rows |= {lo, last, lo + (nt - 1) * BM}
    busy = int(np.argmax(cnt))
    t0 = int(off[busy]) + (spans[busy][1] - 1) * BM
    last = int(off[busy]) + int(cnt[busy]) - 1
    rows |= set(np.unique(np.linspace(t0, last, 16).astype(int)).tolist())
    n_tail_tiles = 0
    if split:
        tile_r0 = [int(off[e]) + t * BM for e, nt in spans for t in range(nt)]
        tile_last = [min(r0 + BM, int(off[e]) + int(cnt[e])) - 1 for (e, nt) in spans for r0 in
                     [int(off[e]) + t * BM for t in range(nt)]]
        m_real = len(tile_r0)
        n_tiles = -(-N // (128 if gate_up else 256))
        segs, Tw = _split_tail_segments(m_real * n_tiles, -(-K // 64), grid)
        for L in sorted({sg[0] for sg in segs if sg[0] >= Tw}):
            m_t, _ = _decode_tile(L, 2048 // BM, m_real, n_tiles)
            a, b = tile_r0[m_t], tile_last[m_t]
            if b >= a:
                rows |= {a, (a + b) // 2, b}
                n_tail_tiles += 1
    real = [r for r in sorted(rows) if 0 <= r < len(al["sorted_ids"]) and al["sorted_ids"][r] < P]
    return np.array(real, dtype=np.int64), n_tail_tiles


@pytest.mark.parametrize("name", ["mixtral_prefill", "finegrained_skewed", "lora_prefill", "fp8_prefill"])
def test_grouped_gemms_full_size_rows(dev, name):
    """Both grouped GEMMs at full size, in the bench's launch configuration (split tail workspace),
    stage by stage on the GPU's own inputs: selected sorted rows (expert boundaries, the busiest
    expert's last tile, every row tile holding a split-tail piece) against the oracle, each row to
    2e-2 relative error and every element to 2e-2 of its row's rms."""
    import torch
    cfg = CONFIGS[name]
    note(f"full-size GEMM rows {name}")
    d = make_inputs(cfg)
    m = ops()
    layer = m.MoeLayer.from_arrays(d, "cuda", down_fused=False)   # the plain down GEMM first
    b = layer.plan(cfg.T, "cuda")
    x = bf16_dev(d["x"])
    layer.route_align(to_dev(d["logits"]), b)
    layer.gate_up_stage(x, b)
    layer.down_stage(b)
    torch.cuda.synchronize()
    ids, w = oracle.route(d["logits"], cfg.top_k, cfg.renormalize)
    al = oracle.align(ids, cfg.E, cfg.block_size)
    assert np.array_equal(b.routing.sorted_ids.cpu().numpy(), al["sorted_ids"])
    BM = 256 if cfg.P >= 128 * cfg.E else 128
    grid = min(torch.cuda.get_device_properties(0).multi_processor_count // 8 * 8, 256)
    fp8 = cfg.weights == "fp8"
    hs_gpu = bf16_host(b.hs)
    ys_gpu = bf16_host(b.ys)
    rows_gu, tail_gu = _selected_rows(al, cfg.P, BM, cfg.I, cfg.H, True, grid, not fp8)
    rows_dn, tail_dn = _selected_rows(al, cfg.P, BM, cfg.H, cfg.I, False, grid, not fp8)
    note(f"  BM={BM}: gate/up {rows_gu.size} rows ({tail_gu} split-tail row tiles), "
         f"down {rows_dn.size} rows ({tail_dn} split-tail row tiles)")
    if fp8:
        xq, sx = oracle.quantize_rows_fp8(oracle.bf16_bits_to_f64(d["x"]))
        h = oracle.grouped_gate_up_fp8(xq, sx, d["fp8_gate"], d["fp8_up"], al, cfg.top_k, rows=rows_gu)
        hq = np.zeros((len(al["sorted_ids"]), cfg.I), np.uint8)
        sh = np.ones(len(al["sorted_ids"]), np.float32)
        hq[rows_dn], sh[rows_dn] = oracle.quantize_rows_fp8(hs_gpu[rows_dn])
        assert np.array_equal(b.hq.cpu().numpy()[rows_dn], hq[rows_dn])
        y = oracle.grouped_down_fp8(hq, sh, d["fp8_down"], al, rows=rows_dn)
    else:
        wg, wu, wd = oracle.moe_oracle._weights(d)
        h = oracle.grouped_gate_up(d["x"], wg, wu, al, cfg.top_k, rows=rows_gu)
        y = oracle.grouped_down(hs_gpu, wd, al, rows=rows_dn)
    assert_close_rows(hs_gpu[rows_gu], h[rows_gu], TOL, f"{name} gate/up rows")
    assert_close_rows(ys_gpu[rows_dn], y[rows_dn], TOL, f"{name} down rows")
    if layer.lora is not None and not fp8:
        # the down-projection fold in the down GEMM's epilogue, as the bench runs it: on the selected
        # rows against the oracle's fold of this plain down output; rows it does not fold unchanged
        plain = bits_host(b.ys)
        layer.down_fused = True
        assert layer.down_fold_fused(b)
        layer.down_stage(b)
        torch.cuda.synchronize()
        fb = bits_host(b.ys)
        tabs = oracle.moe_oracle._lora_tables(d)
        H = oracle.bf16_bits_to_f64(bits_host(b.hs))
        ref = oracle.lora_fold(oracle.bf16_bits_to_f64(plain), H, tabs, al, cfg.top_k)
        sd = oracle.lora_fold(np.zeros(ref.shape), H, tabs, al, cfg.top_k, bf16_base=False)
        ref_bits = f32_to_bf16_bits(ref[rows_dn].astype(np.float32))
        same = np.all(ref_bits == plain[rows_dn], axis=1)
        assert np.array_equal(fb[rows_dn][same], plain[rows_dn][same])
        folded = rows_dn[~same]
        assert folded.size > 0
        _gather_check(fb, ref, sd, plain, folded, f"{name} fused down fold, {folded.size} selected rows")


@pytest.mark.parametrize("name,fold", [("lora_small", "grouped"), ("lora_small", "gather"),
                                       ("decode_lora", "grouped"), ("decode_lora", "gather")])
def test_layer_lora_fold_modes(dev, name, fold):
    """Both folds inside the layer: the folded Ys rows against the oracle fold of the GPU's own
    Hs and unfolded Ys (a missing fold is below the end-to-end tolerance), then the output."""
    import torch
    m = ops()
    cfg = SMALL[name]
    note(f"layer fold {name} {fold}")
    d = make_inputs(cfg)
    layer = m.MoeLayer.from_arrays(d, "cuda", fold=fold, down_fused=False)   # the fold kernels after the GEMMs
    b = layer.plan(cfg.T, "cuda")
    assert layer.fold_mode(b) == fold
    layer.route_align(to_dev(d["logits"]), b)
    lora, layer.lora = layer.lora, None
    layer.experts(bf16_dev(d["x"]), b)          # the GEMMs only
    layer.lora = lora
    torch.cuda.synchronize()
    hs, ys0 = bits_host(b.hs), bits_host(b.ys)
    layer.lora_fold(b)
    out = layer.combine(b)
    ref = oracle.moe_layer(d)
    al = ref["align"]
    real = _real(al, cfg.P)
    tabs = oracle.moe_oracle._lora_tables(d)
    hs_f = np.where(np.isin(np.arange(hs.shape[0]), real)[:, None], oracle.bf16_bits_to_f64(hs), 0.0)
    ys0_f = oracle.bf16_bits_to_f64(ys0)
    want = oracle.lora_fold(ys0_f, hs_f, tabs, al, cfg.top_k)
    sd = oracle.lora_fold(np.zeros(ys0.shape), hs_f, tabs, al, cfg.top_k)
    adapted_rows = np.array([rr for rr in real
                             if (np.searchsorted(al["offsets"], rr, side="right") - 1) % 2 == 0])
    _gather_check(bits_host(b.ys), want, sd, ys0, adapted_rows, f"layer fold {name} {fold}")
    others = np.setdiff1d(real, adapted_rows)
    assert np.array_equal(bits_host(b.ys)[others], ys0[others])
    assert_close_rows(bf16_host(out), ref["out"], TOL, f"layer {name} {fold}")


def test_layer_graph_replay_matches_eager(dev):
    import torch
    m = ops()
    cfg = SMALL["lora_small"]
    d = make_inputs(cfg)
    layer = m.MoeLayer.from_arrays(d, "cuda")
    b = layer.plan(cfg.T, "cuda")
    logits, x = to_dev(d["logits"]), bf16_dev(d["x"])
    eager = bits_host(layer.forward(logits, x, b)).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        layer.forward(logits, x, b)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            layer.forward(logits, x, b)
    torch.cuda.synchronize()
    for i in range(3):
        b.out.zero_()
        b.ys.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_host(b.out), eager), f"replay {i} differs from eager"
        layer.forward(logits, x, b)  # eager work between replays
        torch.cuda.synchronize()


def test_layer_graph_replay_split_tail(dev, shared_ws):
    """A layer whose GEMMs split their tail tiles (counters and partials in the workspace, reset by
    the kernels themselves, no memset) replays from a HIP graph bit-identically to eager runs."""
    import torch
    m = ops()
    cfg = SPLIT_K["rows256"]
    d = make_inputs(cfg)
    layer = m.MoeLayer.from_arrays(d, "cuda")
    b = layer.plan(cfg.T, "cuda")
    b.ws = shared_ws
    logits, x = to_dev(d["logits"]), bf16_dev(d["x"])
    eager = bits_host(layer.forward(logits, x, b)).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        layer.forward(logits, x, b)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            layer.forward(logits, x, b)
    torch.cuda.synchronize()
    for i in range(3):
        b.out.zero_()
        b.hs.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_host(b.out), eager), f"replay {i} differs from eager"
        layer.forward(logits, x, b)  # eager work between replays
        torch.cuda.synchronize()
    assert not shared_ws[:4096].cpu().numpy().any(), "split counters not reset"


def test_layer_deterministic(dev):
    cfg = SMALL["finegrained_small"]
    d = make_inputs(cfg)
    _, _, o1 = _layer_run(cfg, d)
    _, _, o2 = _layer_run(cfg, d)
    assert np.array_equal(bits_host(o1), bits_host(o2))


def test_grouped_gemms_padded_total_at_capacity(dev):
    """Regression: every expert holds a multiple of block_size plus one pair, so the padded total
    equals the sorted capacity and the last 256-row tile of the last expert extends past the
    end of the buffers; such rows must neither be read out of bounds nor stored."""
    m = ops()
    E, bs, per = 2, 64, 8 * 64 + 1
    cfg = MoeConfig("tight", T=E * per, H=256, I=256, E=E, top_k=1, block_size=bs, seed=21)
    d = make_inputs(cfg)
    ids = np.repeat(np.arange(E, dtype=np.int32), per).reshape(-1, 1)
    al = oracle.align(ids, E, bs)
    assert al["total"] == len(al["sorted_ids"])  # the padded total reaches the capacity
    r = m.moe_align(to_dev(ids), E, bs)
    layer = _weights_dev(d)
    real = _real(al, cfg.P)
    hs = _canary(r.max_pad, cfg.I)
    m.moe_grouped_gemm(m.MOE_OP_GATE_UP_SILU, bf16_dev(d["x"]), layer.gate, layer.up, r, out=hs)
    h_ref = oracle.grouped_gate_up(d["x"], d["wg"], d["wu"], al, 1)
    assert_close_rows(bf16_host(hs)[real], h_ref[real], TOL, "gate/up at capacity")
    # down, fed with the oracle's own h rounded to bf16 (NaN in every padding row)
    h_in = np.full((r.max_pad, cfg.I), CANARY, np.uint16)
    h_in[real] = f32_to_bf16_bits(oracle.round_bf16(h_ref[real]).astype(np.float32))
    ys = _canary(r.max_pad, cfg.H)
    m.moe_grouped_gemm(m.MOE_OP_DOWN, bf16_dev(h_in), layer.down, None, r, out=ys)
    y_ref = oracle.grouped_down(oracle.bf16_bits_to_f64(h_in), d["wd"], al)
    assert_close_rows(bf16_host(ys)[real], y_ref[real], TOL, "down at capacity")
    pad = np.setdiff1d(np.arange(r.max_pad), real)
    assert (bits_host(ys)[pad] == CANARY).all()


# ----------------------------------------------------------------------------- A1+A2 fused entry point
ROUTE_ALIGN_CASES = [
    ("decode_int4", CONFIGS["decode_int4"]),                        # one launch (96 pairs)
    ("tiny", CONFIGS["tiny"]),                                      # one launch (128 pairs)
    ("mixtral_prefill", CONFIGS["mixtral_prefill"]),                # route + two align launches
    ("E256_k8", MoeConfig("E256", T=200, H=8, I=8, E=256, top_k=8, block_size=64, seed=21)),
    ("E200_k7_chunk_edge", MoeConfig("E200", T=292, H=8, I=8, E=200, top_k=7, block_size=32, seed=22)),
    ("E1", MoeConfig("E1", T=17, H=8, I=8, E=1, top_k=1, block_size=16, seed=23)),
    ("k_eq_E_no_renorm", MoeConfig("kE", T=50, H=8, I=8, E=6, top_k=6, block_size=16, renormalize=False, seed=24)),
    ("one_chunk_max", MoeConfig("c1", T=256, H=8, I=8, E=64, top_k=8, block_size=128, seed=25)),
    ("one_over_chunk", MoeConfig("c2", T=2049, H=8, I=8, E=3, top_k=1, block_size=16, seed=26)),
    ("T40_four_per_wave", MoeConfig("t40", T=40, H=8, I=8, E=128, top_k=8, block_size=32, seed=27)),
    ("T64_E256", MoeConfig("t64", T=64, H=8, I=8, E=256, top_k=4, block_size=16, seed=28)),
    ("T65_two_calls", MoeConfig("t65", T=65, H=8, I=8, E=32, top_k=2, block_size=16, seed=29)),
    ("E256_k96_one_launch", MoeConfig("k96", T=20, H=8, I=8, E=256, top_k=96, block_size=16, seed=30)),
    ("E192_k100_two_calls", MoeConfig("k100", T=30, H=8, I=8, E=192, top_k=100, block_size=16, seed=31)),
    # at most 16 experts and more than 16 tokens: one token per 16-lane row
    ("T64_E16_ties", MoeConfig("t64e16", T=64, H=8, I=8, E=16, top_k=4, block_size=16, seed=32)),
    ("T17_E16", MoeConfig("t17e16", T=17, H=8, I=8, E=16, top_k=2, block_size=16, seed=33)),
    ("T50_E9_k9_no_renorm", MoeConfig("t50e9", T=50, H=8, I=8, E=9, top_k=9, block_size=32, renormalize=False,
                                      seed=34)),
]


@pytest.mark.parametrize("name,cfg", ROUTE_ALIGN_CASES, ids=[c[0] for c in ROUTE_ALIGN_CASES])
def test_route_align_matches_oracle(dev, name, cfg):
    """moe_route_align equals the oracle's route followed by its align, bit for bit (single-launch
    path for batches of at most 2048 pairs, the two-call path above)."""
    import torch
    note(f"route_align {name} T={cfg.T} E={cfg.E} k={cfg.top_k} P={cfg.P}")
    m = ops()
    logits = make_router_logits(cfg)
    if name.endswith("_ties"):
        _plant_ties(logits, cfg.E)
    ids_ref, w_ref = oracle.route(logits, cfg.top_k, cfg.renormalize)
    ref = oracle.align(ids_ref, cfg.E, cfg.block_size)
    ids = torch.empty((cfg.T, cfg.top_k), dtype=torch.int32, device=dev)
    w = torch.empty((cfg.T, cfg.top_k), dtype=torch.float32, device=dev)
    r = m.Routing.allocate(cfg.P, cfg.top_k, cfg.E, cfg.block_size, dev)
    r.sorted_ids.fill_(-7)   # every row must be written
    r.expert_ids.fill_(-7)
    m.moe_route_align(to_dev(logits), cfg.top_k, cfg.renormalize, cfg.block_size, ids, w, r)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), w_ref.view(np.uint32))
    got = {"counts": r.counts.cpu().numpy(), "offsets": r.offsets.cpu().numpy(),
           "sorted_ids": r.sorted_ids.cpu().numpy(), "expert_ids": r.expert_ids.cpu().numpy(),
           "total": int(r.total_padded.cpu().item()), "inv": r.inv_sorted.cpu().numpy()[: cfg.P]}
    _assert_align_equal(got, ref)


def test_route_align_zero_tokens(dev):
    import torch
    m = ops()
    r = m.Routing.allocate(0, 2, 4, 16, dev)
    r.sorted_ids.fill_(-7)
    ids = torch.empty((0, 2), dtype=torch.int32, device=dev)
    w = torch.empty((0, 2), dtype=torch.float32, device=dev)
    m.moe_route_align(torch.empty((0, 4), dtype=torch.float32, device=dev), 2, True, 16, ids, w, r)
    ref = oracle.align(np.zeros((0, 2), np.int32), 4, 16)
    assert np.array_equal(r.sorted_ids.cpu().numpy(), ref["sorted_ids"])
    assert np.array_equal(r.offsets.cpu().numpy(), ref["offsets"])
