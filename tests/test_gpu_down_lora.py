"""GPU parity of the down-projection LoRA fold run in the down GEMM's epilogue
(moe_grouped_gemm_down_lora; atlas moe_lora_grouped.rs, moe_lora_grouped_down: shrink, then expand
and fold in place into the sorted BF16 expert_down_out).

On the same sorted Hs (random bf16 on the real rows, a canary elsewhere) each case checks:
  * padding and sentinel rows of Ys are never written;
  * rows that are not folded (unadapted experts, tokens of adapter < 0) are bit-identical to the
    plain down GEMM's;
  * the folded rows against the oracle's fold applied to the GPU's own plain down output, to the
    fold's bar (>= 99.9% bit-exact, each value within 3 bf16 ulps of the largest of |base|,
    |result| and |scale * delta|), and against the unfused GPU path (down GEMM, then
    moe_lora_fold) to the same bar;
  * the whole Ys against the fully independent oracle (down GEMM and fold in fp64) at 2e-2 per row
    and per element of the row's rms.
Cases cover both tile heights (128-row tiles below 128 rows per expert, 256-row tiles above), one
and three adapters, a per-token adapter map, scales x100, max_rank 32 to 128, several tiles per
workgroup with the next tile prepared inside the main loop, and split tails through the workspace.
"""
import numpy as np
import pytest

import oracle
from moe_synth import MoeConfig, make_inputs, f32_to_bf16_bits
from _util import assert_close_rows, bf16_dev, bits_host, to_dev

pytestmark = pytest.mark.gpu
TOL = 2e-2
CANARY = 0x7FC1

_BASE = MoeConfig("dl_small", T=200, H=512, I=256, E=16, top_k=6, block_size=64, lora_rank=16, lora_max_rank=64,
                  seed=61)
_256 = dict(T=1100, E=8, top_k=2)   # 275 rows per expert: 256-row tiles
CASES = {
    # (config, scale multiplier, per-token adapter map with -1 entries, use the split-tail workspace)
    "rows128": (_BASE, 1.0, False, False),
    "rows256": (_BASE.with_(name="dl_256", seed=62, **_256), 1.0, False, False),
    "rows256_x100": (_BASE.with_(name="dl_256x", seed=63, **_256), 100.0, False, False),
    "rows128_adapter_map": (_BASE.with_(name="dl_map", seed=64), 1.0, True, False),
    "rows256_adapter_map": (_BASE.with_(name="dl_256map", seed=65, **_256), 1.0, True, False),
    "mixed3_rows128": (_BASE.with_(name="dl_mix", T=300, lora_adapters=3, seed=66), 1.0, False, False),
    "mixed3_rows256": (_BASE.with_(name="dl_mix256", lora_adapters=3, seed=67, **_256), 1.0, False, False),
    "max_rank_32_rows256": (_BASE.with_(name="dl_r32", lora_rank=24, lora_max_rank=32, seed=68, **_256), 1.0,
                            False, False),
    "max_rank_128_rows256": (_BASE.with_(name="dl_r128", lora_rank=100, lora_max_rank=128, seed=69, **_256), 1.0,
                             False, False),
    "max_rank_96_rows128": (_BASE.with_(name="dl_r96", lora_rank=80, lora_max_rank=96, seed=70), 1.0, False, False),
    # 16 row tiles x 33 panels (N = 8200, a ragged last panel), K = 320: 5-stage segments, several tiles
    # per workgroup, the next one prepared inside the main loop
    "prefetch_k5_rows256": (MoeConfig("dl_pf", T=1200, H=8200, I=320, E=8, top_k=2, block_size=64, lora_rank=16,
                                      lora_max_rank=64, seed=71), 1.0, True, False),
    # split tails: 256-row tiles, 272 down tiles (16 in the tail, 2 pieces); 128-row tiles, 288 down
    # tiles (32 in the tail, 3 pieces)
    "split_rows256": (MoeConfig("dl_sk256", T=1536, H=4104, I=1032, E=8, top_k=2, block_size=64, lora_rank=16,
                                lora_max_rank=64, seed=72), 1.0, True, True),
    "split_rows128": (MoeConfig("dl_sk128", T=1024, H=2824, I=1544, E=24, top_k=2, block_size=64, lora_rank=16,
                                lora_max_rank=64, seed=73), 1.0, False, True),
}


def note(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import mixture_experts_routed_route_amd as m
    m.lib()  # raises if the library is missing: no fallback
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def ws(dev):
    import mixture_experts_routed_route_amd as m
    return m.gemm_workspace("cuda")


def _canary(rows, cols):
    import torch
    return torch.full((rows, cols), CANARY, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def _fold_bar(got_bits, ref, scaled_delta, base_bits, what):
    """>= 99.9% of the values bit-exact, each within 3 bf16 ulps of the largest of |base|, |result|
    and |scale * delta| (the two sides sum xa and delta in different fp32 orders)."""
    g = oracle.bf16_bits_to_f64(got_bits)
    mag = np.maximum(np.maximum(np.abs(oracle.bf16_bits_to_f64(base_bits)), np.abs(ref)), np.abs(scaled_delta))
    _, ex = np.frexp(mag)
    ulp_m = np.ldexp(1.0, np.maximum(ex - 8, -133))
    worst = float((np.abs(g - ref) / ulp_m).max()) if g.size else 0.0
    exact = float((g == ref).mean()) if g.size else 1.0
    note(f"  [{what}] exact {exact:.5f}, max |diff| {worst:.2f} ulp of the largest term")
    assert worst <= 3 and exact >= 0.999, what


@pytest.mark.parametrize("case", list(CASES))
def test_down_lora_fused_epilogue(dev, ws, case):
    import torch
    import mixture_experts_routed_route_amd as m
    cfg, smult, use_map, use_ws = CASES[case]
    note(f"down lora fused {case}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} top_k={cfg.top_k} "
         f"rank {cfg.lora_rank}/{cfg.lora_max_rank} adapters {cfg.lora_adapters} ws={use_ws}")
    d = make_inputs(cfg)
    if smult != 1.0:
        d["lora_scale"] = (d["lora_scale"] * smult).astype(np.float32)
    ra = d.get("row_adapter")
    if use_map and ra is None:
        ra = np.where(np.arange(cfg.T) % 4 == 1, -1, 0).astype(np.int32)
    ids, w = oracle.route(d["logits"], cfg.top_k, cfg.renormalize)
    al = oracle.align(ids, cfg.E, cfg.block_size)
    r = m.moe_align(to_dev(ids.astype(np.int32)), cfg.E, cfg.block_size)
    real = np.flatnonzero(al["sorted_ids"] < cfg.P)
    pad = np.setdiff1d(np.arange(r.max_pad), real)
    rng = np.random.default_rng(cfg.seed + 100)
    hs = np.full((r.max_pad, cfg.I), CANARY, np.uint16)
    hs[real] = f32_to_bf16_bits(rng.standard_normal((real.size, cfg.I)).astype(np.float32))
    layer = m.MoeLayer.from_arrays(d, "cuda")
    tables = layer.lora
    hs_dev = bf16_dev(hs)
    ra_dev = to_dev(ra) if ra is not None else None
    wsp = ws if use_ws else None

    plain = _canary(r.max_pad, cfg.H)
    m.moe_grouped_gemm(m.MOE_OP_DOWN, hs_dev, layer.down, None, r, out=plain, workspace=wsp)
    unf = plain.clone()
    m.moe_lora_fold(hs_dev, unf, tables, r, row_adapter=ra_dev)
    xa = torch.empty((r.max_pad, tables.max_rank), dtype=torch.bfloat16, device="cuda")
    fused = _canary(r.max_pad, cfg.H)
    m.moe_grouped_gemm_down_lora(hs_dev, layer.down, r, tables, xa, out=fused, row_adapter=ra_dev, workspace=wsp)
    torch.cuda.synchronize()
    pb, ub, fb = bits_host(plain), bits_host(unf), bits_host(fused)

    assert (fb[pad] == CANARY).all(), "padding or sentinel rows of Ys written"
    # the fold on the GPU's own plain down output: rows the oracle leaves alone are the plain rows
    tabs = oracle.moe_oracle._lora_tables(d)
    H = oracle.bf16_bits_to_f64(hs)
    base = oracle.bf16_bits_to_f64(pb)
    ref = oracle.lora_fold(base, H, tabs, al, cfg.top_k, row_adapter=ra)
    sd = oracle.lora_fold(np.zeros(base.shape), H, tabs, al, cfg.top_k, row_adapter=ra, bf16_base=False)
    ref_bits = f32_to_bf16_bits(ref[real].astype(np.float32))
    same = np.all(ref_bits == pb[real], axis=1)
    assert np.array_equal(fb[real][same], pb[real][same]), "a row that is not folded differs from the plain GEMM"
    folded = real[~same]
    assert folded.size > 0
    note(f"  {folded.size} of {real.size} real rows folded")
    _fold_bar(fb[folded], ref[folded], sd[folded], pb[folded], f"fused vs oracle fold of the GPU base ({case})")
    _fold_bar(fb[folded], oracle.bf16_bits_to_f64(ub[folded]), sd[folded], pb[folded],
              f"fused vs unfused GPU path ({case})")
    note(f"  fused == unfused bits on {(fb[real] == ub[real]).mean():.5f} of the values")
    # the whole Ys against the independent oracle: the down GEMM in fp64, rounded, then the fold
    wd = oracle.moe_oracle._weights(d)[2]
    y0 = oracle.round_bf16(oracle.grouped_down(H, wd, al))
    want = oracle.lora_fold(y0, H, tabs, al, cfg.top_k, row_adapter=ra)
    assert_close_rows(oracle.bf16_bits_to_f64(fb[real]), want[real], TOL, f"fused vs oracle ({case})", ulps=2)
    if ra is not None and (ra < 0).any():
        skipped = [rr for rr in real if ra[al["sorted_ids"][rr] // cfg.top_k] < 0]
        assert np.array_equal(fb[skipped], pb[skipped]), "rows of tokens with adapter < 0 were folded"
    if cfg.lora_adapters > 1:
        by = np.array([ra[al["sorted_ids"][rr] // cfg.top_k] for rr in folded])
        assert set(np.unique(by)) == set(range(cfg.lora_adapters)), np.unique(by)


def test_down_lora_layer_matches_unfused(dev):
    """The layer with the fused down fold against the layer with the separate fold kernels and
    against the oracle's whole layer, on lora_small-shaped inputs with a per-token adapter map."""
    import torch
    import mixture_experts_routed_route_amd as m
    cfg = _BASE.with_(name="dl_layer", lora_adapters=2, seed=74)
    note(f"down lora layer {cfg.name}")
    d = make_inputs(cfg)
    ra = to_dev(d["row_adapter"])
    outs = {}
    for name, fused in (("fused", True), ("unfused", False)):
        layer = m.MoeLayer.from_arrays(d, "cuda", fold="grouped", down_fused=fused)
        b = layer.plan(cfg.T, "cuda")
        assert layer.down_fold_fused(b) == fused
        out = layer.forward(to_dev(d["logits"]), bf16_dev(d["x"]), b, row_adapter=ra)
        torch.cuda.synchronize()
        outs[name] = oracle.bf16_bits_to_f64(bits_host(out))
    ref = oracle.moe_layer(d)["out"]
    assert_close_rows(outs["fused"], outs["unfused"], TOL, "layer fused vs unfused", ulps=2)
    assert_close_rows(outs["fused"], ref, TOL, "layer fused vs oracle", ulps=4)
