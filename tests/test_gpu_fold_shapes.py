"""Grouped LoRA fold (moe_lora_fold) across shapes, against the oracle (atlas moe_lora_grouped.rs,
moe_lora_grouped_down; adapters per atlas MoeExpertRoute).

The kernels take different paths by shape, and each case here drives some of them:
  * block sizes 16 and 32 put several experts in one 64-row tile (the expand's general path, several
    (expert, adapter) passes in the shrink); 64 and 128 keep a tile on one expert (the one-pair path);
  * max_rank 32, 64, 96 and 128 select the shrink's and the expand's per-rank instantiations;
  * k_in not a multiple of 128 ends a wave's k range inside a k-step; n_out not a multiple of 256
    (and above 1024: a second column group) ends slabs inside a wave's columns;
  * several adapters through a map (with ids past the installed adapters and -1), dropped router
    ids, and windows that start off the 16-row grid.
Rows that must not change (padding, skipped tokens, unadapted experts) are compared bit for bit;
folded values meet the fold's bar (>= 99.9% bit-exact, every one within 3 bf16 ulps of the largest
of |base|, |result| and |scale * delta|: the kernels sum in fp32 in another order than the oracle).
"""
import sys

import numpy as np
import pytest

from _util import bf16_dev, bits_host, to_dev
from moe_synth import f32_to_bf16_bits
import oracle

pytestmark = pytest.mark.gpu
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


# (name, T, top_k, E, block, k_in, n_out, max_rank, real rank, x_gather, adapters, map, window cap)
CASES = [
    ("bs16_r32_ragged", 96, 4, 16, 16, 200, 264, 32, 32, 0, 1, False, None),
    ("bs32_r96_gather_map", 150, 3, 12, 32, 520, 1096, 96, 80, 1, 1, True, None),
    ("bs64_r128_two_adapters", 200, 6, 16, 64, 384, 1560, 128, 100, 0, 2, True, None),
    ("bs16_r64_three_adapters_windows", 120, 6, 32, 16, 256, 520, 64, 16, 1, 3, True, 40),
    ("bs128_r64_wide", 129, 2, 4, 128, 136, 2056, 64, 64, 0, 1, False, None),
    ("bs64_r32_windows_map", 90, 6, 8, 64, 1408, 776, 32, 16, 0, 1, True, 100),
]


def _adapter_tables(rng, E, k_in, n_out, R, r, j):
    """Adapter j adapts the experts e with (e + j) % 3 != 1; A_e, B_e hold `r` real ranks of R."""
    ids, a_l, b_l, s_l = [], [], [], []
    for e in range(E):
        if (e + j) % 3 == 1:
            continue
        a = np.zeros((R, k_in), np.uint16)
        a[:r] = f32_to_bf16_bits((rng.standard_normal((r, k_in)) * 0.02).astype(np.float32))
        b = np.zeros((n_out, R), np.uint16)
        b[:, :r] = f32_to_bf16_bits((rng.standard_normal((n_out, r)) * 0.02).astype(np.float32))
        ids.append(e), a_l.append(a), b_l.append(b), s_l.append(float(np.float32(rng.uniform(0.5, 2.0))))
    return ids, a_l, b_l, s_l


def _check(got, ref, scaled_delta, base, rows, what):
    g = oracle.bf16_bits_to_f64(got[rows])
    r = ref[rows]
    big = np.maximum(np.maximum(np.abs(oracle.bf16_bits_to_f64(base[rows])), np.abs(r)), np.abs(scaled_delta[rows]))
    _, ex = np.frexp(big)
    ulp = np.ldexp(1.0, np.maximum(ex - 8, -133))
    worst = (np.abs(g - r) / ulp).max()
    exact = (g == r).mean()
    note(f"{what}: exact {exact:.5f}, max |diff| {worst:.2f} ulp of the largest term")
    assert worst <= 3 and exact >= 0.999, what


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_grouped_fold_shapes(dev, case):
    import torch
    m = ops()
    name, T, k, E, bs, k_in, n_out, R, r, xg, n_ad, use_map, cap = case
    note(f"grouped fold {name}")
    rng = np.random.default_rng(101 + len(name))
    ids, _ = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    ids = ids.reshape(-1).copy()
    ids[1], ids[4] = -1, E + 2  # dropped pairs
    ids = ids.astype(np.int32)
    P = ids.size
    al = oracle.align(ids, E, bs)
    routing = m.moe_align(to_dev(ids.reshape(T, k)), E, bs)
    max_pad = len(al["sorted_ids"])
    assert routing.max_pad >= max_pad
    real = np.flatnonzero(al["sorted_ids"] < P)

    x_rows = T if xg else routing.max_pad
    x = np.full((x_rows, k_in), CANARY, np.uint16)
    if xg:
        x[:] = f32_to_bf16_bits(rng.standard_normal((T, k_in)).astype(np.float32))
    else:
        x[real] = f32_to_bf16_bits(rng.standard_normal((real.size, k_in)).astype(np.float32))
    base = np.full((routing.max_pad, n_out), CANARY, np.uint16)
    base[real] = f32_to_bf16_bits((rng.standard_normal((real.size, n_out)) * 0.05).astype(np.float32))
    ra = None
    if use_map:
        ra = rng.integers(-1, n_ad + 1, size=T).astype(np.int32)  # n_ad: past the installed adapters

    per = [_adapter_tables(rng, E, k_in, n_out, R, r, j) for j in range(n_ad)]
    o_tabs = [oracle.pack_expert_tables(list(zip(*t))) for t in per]
    dev_tabs = [m.pack_lora_tables(t[0], [bf16_dev(a) for a in t[1]], [bf16_dev(b) for b in t[2]], t[3], "cuda")
                for t in per]
    tables = dev_tabs[0] if n_ad == 1 else m.stack_lora_tables(dev_tabs, "cuda")
    o_t = o_tabs[0] if n_ad == 1 else o_tabs

    xf = oracle.bf16_bits_to_f64(x)
    bf = oracle.bf16_bits_to_f64(base[:max_pad])
    ref = oracle.lora_fold(bf, xf, o_t, al, k, row_adapter=ra, x_gather=bool(xg))
    sd = oracle.lora_fold(np.zeros_like(bf), xf, o_t, al, k, row_adapter=ra, x_gather=bool(xg))

    got = bf16_dev(base)
    window_cap = cap or routing.max_pad
    xa = torch.empty((window_cap, R), dtype=torch.bfloat16, device="cuda")
    for s, e in m.lora_windows(routing.max_pad, window_cap):
        m.moe_lora_fold(bf16_dev(x), got, tables, routing, row_adapter=to_dev(ra) if ra is not None else None,
                        xa=xa, row_offset=s, row_end=e, x_gather=bool(xg))
    gb = bits_host(got)

    def folded_row(rr):
        p = int(al["sorted_ids"][rr])
        if p >= P:
            return False
        a = 0 if ra is None else int(ra[p // k])
        if not 0 <= a < n_ad:
            return False
        e = int(np.searchsorted(al["offsets"], rr, side="right") - 1)
        return e in per[a][0]

    folded = np.array([folded_row(rr) for rr in range(max_pad)])
    assert folded.any()
    keep = np.flatnonzero(~folded)
    assert np.array_equal(gb[keep], base[keep]), "a row that is not folded changed"
    assert np.array_equal(gb[max_pad:], base[max_pad:]), "a row past the aligned total changed"
    _check(gb[:max_pad], ref, sd, base[:max_pad], np.flatnonzero(folded), name)
