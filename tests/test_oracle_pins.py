"""Pins for the CPU oracle: each check ties an oracle function to something other
than itself — the pages' own test cases, hand-worked examples with closed forms,
independent library routines, textbook special cases, invariants and brute force
on tiny inputs.  CPU only."""
import itertools
import math

import numpy as np
import pytest
import torch
from scipy.special import softmax as scipy_softmax

import oracle
from moe_synth import CONFIGS, MoeConfig, make_inputs, f32_to_bf16_bits
from conftest import golden


def bf16(a):
    return f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


# ----------------------------------------------------------------------------- number formats
def test_round_bf16_against_torch():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-30).astype(np.float32),
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        np.float32([0.0, -0.0, 1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -133, 2 ** -134,
                    3 * 2 ** -134, 1e-45, 3.3895e38]),
    ])
    # every fp32 value that sits exactly on a bf16 tie
    ties = (np.arange(1, 5000, dtype=np.uint32) << 16 | np.uint32(0x8000)).view(np.float32)
    v = np.concatenate([v, ties, -ties])
    ours = oracle.round_bf16(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_round_bf16_hand_values():
    r = oracle.round_bf16
    assert r(1 + 2 ** -8) == 1.0                      # tie -> even mantissa
    assert r(1 + 3 * 2 ** -8) == 1 + 2 ** -6          # tie -> even (up)
    assert r(1 + 2 ** -8 + 2 ** -30) == 1 + 2 ** -7   # just above the tie
    assert r(-(1 + 2 ** -8)) == -1.0
    assert r(255.5) == 256.0 and r(255.0) == 255.0
    assert r(2.0 ** 128 * 0.999) == np.inf


def test_bf16_and_f16_widening_exact():
    v = np.float32([1.5, -2.75, 3.0e-3, 65504.0])
    assert np.array_equal(oracle.bf16_bits_to_f64(bf16(v)), torch.tensor(v).bfloat16().double().numpy())
    h = np.float16([0.005, 0.02, -1.0, 6.1e-5])
    assert np.array_equal(oracle.f16_bits_to_f64(h.view(np.uint16)), h.astype(np.float64))


# ----------------------------------------------------------------------------- route
def test_route_worked_examples():
    g = golden("route_worked.json")
    for c in g["cases"]:
        l = np.float32([float(x) for x in c["logits"]])[None, :]
        ids, w = oracle.route(l, c["top_k"], c["renormalize"])
        assert ids[0].tolist() == c["ids"], c
        assert np.array_equal(w[0], np.float32(c["weights"])), (w, c)


def test_route_special_cases():
    rng = np.random.default_rng(2)
    # one expert: weight exactly 1
    ids, w = oracle.route(rng.standard_normal((5, 1)).astype(np.float32), 1)
    assert (ids == 0).all() and (w == 1.0).all()
    # k = E with renormalisation = the full softmax, in descending order
    l = rng.standard_normal((50, 6)).astype(np.float32)
    ids, w = oracle.route(l, 6, True)
    full = scipy_softmax(l.astype(np.float64), axis=1)
    assert np.array_equal(w, np.take_along_axis(full, ids, 1).astype(np.float32))
    # without renormalisation the weights are the softmax probabilities themselves
    l = rng.standard_normal((50, 16)).astype(np.float32)
    ids, w = oracle.route(l, 3, False)
    assert np.array_equal(w, np.take_along_axis(scipy_softmax(l.astype(np.float64), axis=1), ids, 1)
                          .astype(np.float32))


def test_route_brute_force_ids_and_sum():
    rng = np.random.default_rng(3)
    for E, k in [(8, 2), (64, 6), (128, 8), (5, 5)]:
        l = rng.standard_normal((300, E)).astype(np.float32)
        l[:10, 1] = l[:10, 3]                          # plant exact ties
        ids, w = oracle.route(l, k, True)
        ref = np.argsort(-l, axis=1, kind="stable")[:, :k]
        assert np.array_equal(ids, ref)
        assert np.all(np.abs(w.astype(np.float64).sum(1) - 1) <= k * 2.0 ** -24)
        # renormalised weights are proportional to exp(logit)
        lsel = np.take_along_axis(l.astype(np.float64), ids, 1)
        ref_w = scipy_softmax(lsel, axis=1)
        assert np.allclose(w, ref_w, rtol=2 ** -23, atol=0)


# ----------------------------------------------------------------------------- align
def _check_align_invariants(ids_flat, E, bs, al):
    P = len(ids_flat)
    counts, off, sid, eid, inv = al["counts"], al["offsets"], al["sorted_ids"], al["expert_ids"], al["inv"]
    assert oracle.check_group_arrays(E, [("counts", len(counts))], off.tolist()) is None
    valid = (ids_flat >= 0) & (ids_flat < E)
    assert counts.sum() == valid.sum()
    assert np.array_equal(counts, np.bincount(ids_flat[valid], minlength=E))
    assert off[0] == 0 and (off % bs == 0).all() and al["total"] == off[-1] <= len(sid)
    assert np.array_equal(np.diff(off), -(-counts // bs) * bs)
    # brute force: a stable sort of the pairs by expert gives the real rows in order
    order = np.argsort(np.where(valid, ids_flat, E), kind="stable")[: valid.sum()]
    real_rows = np.concatenate([np.arange(off[e], off[e] + counts[e]) for e in range(E)] or [[]]).astype(int)
    assert np.array_equal(sid[real_rows], order)
    # everything else is the sentinel P; inverse map round-trips
    mask = np.ones(len(sid), bool)
    mask[real_rows] = False
    assert (sid[mask] == P).all()
    assert np.array_equal(inv[order], real_rows)
    assert (inv[~valid] == -1).all()
    for b in range(len(eid)):
        if b * bs < al["total"]:
            e = np.searchsorted(off, b * bs, side="right") - 1
            assert eid[b] == e
        else:
            assert eid[b] == -1


def test_align_worked_examples():
    for c in golden("align_worked.json")["cases"]:
        ids = np.asarray(c["topk_ids"])
        al = oracle.align(ids, c["num_experts"], c["block_size"], c["max_pad"])
        for key in ("counts", "offsets", "sorted_ids", "expert_ids", "inv"):
            assert al[key].tolist() == c[key], key
        assert al["total"] == c["total"]
        assert oracle.max_padded(ids.size, c["num_experts"], c["block_size"]) == c["max_pad"]


@pytest.mark.parametrize("E,k,bs,T", [(8, 2, 16, 64), (128, 8, 64, 300), (64, 6, 16, 16), (3, 1, 128, 7),
                                      (256, 4, 32, 100), (1, 1, 16, 5)])
def test_align_invariants_random(E, k, bs, T):
    rng = np.random.default_rng(E * 1000 + T)
    ids = rng.integers(0, E, size=(T, k))
    al = oracle.align(ids, E, bs)
    assert len(al["sorted_ids"]) == oracle.max_padded(T * k, E, bs)
    _check_align_invariants(ids.reshape(-1), E, bs, al)


def test_align_drops_out_of_range_and_empty():
    ids = np.array([[0, 5], [-1, 2], [2, 2]])
    al = oracle.align(ids, 3, 4)
    _check_align_invariants(ids.reshape(-1), 3, 4, al)
    assert al["inv"][1] == -1 and al["inv"][2] == -1
    al0 = oracle.align(np.zeros((0, 2), dtype=np.int32), 4, 16)
    assert al0["total"] == 0 and (al0["sorted_ids"] == 0).all() and (al0["expert_ids"] == -1).all()


def test_align_max_pad_is_tight():
    # all pairs on distinct experts with one pair each reach the bound exactly
    E, bs = 10, 16
    ids = np.arange(E)[:, None]
    al = oracle.align(ids, E, bs)
    assert al["total"] == E * bs == oracle.max_padded(E, E, bs)


def test_group_arrays_page_cases():
    for c in golden("group_arrays_cases.json")["cases"]:
        msg = oracle.check_group_arrays(c["num_experts"], [tuple(x) for x in c["per_expert"]], c["offsets"])
        assert (msg is None) == c["ok"], (c, msg)
        if "message_contains" in c:
            assert c["message_contains"] in msg


# ----------------------------------------------------------------------------- GPTQ
def _pack_reference(q, z):
    """Independent packer: build each int32 word from its nibbles with Python ints."""
    K, N = q.shape
    qw = np.zeros((K // 8, N), dtype=np.int64)
    for k in range(K):
        for n in range(N):
            qw[k // 8, n] |= int(q[k, n]) << (4 * (k % 8))
    G_, _ = z.shape
    qz = np.zeros((G_, N // 8), dtype=np.int64)
    for g in range(G_):
        for n in range(N):
            qz[g, n // 8] |= int(z[g, n]) << (4 * (n % 8))
    to32 = lambda a: a.astype(np.uint32).view(np.int32)
    return to32(qw), to32(qz)


def test_gptq_unpack_and_dequant():
    rng = np.random.default_rng(4)
    K, N, G = 64, 16, 32
    q = rng.integers(0, 16, (K, N))
    z = rng.integers(0, 16, (K // G, N))
    s = np.float16(rng.uniform(0.005, 0.02, (K // G, N)))
    qw, qz = _pack_reference(q, z)
    assert np.array_equal(oracle.gptq_unpack_q(qw), q)
    assert np.array_equal(oracle.gptq_unpack_z(qz), z)
    w = {"qweight": qw[None], "qzeros": qz[None], "scales": s.view(np.uint16)[None], "group_size": G}
    W = oracle.gptq_dequant_expert(w, 0)
    for k, n in itertools.product(range(0, K, 7), range(N)):
        assert W[k, n] == (q[k, n] - z[k // G, n]) * float(s[k // G, n])
    # q == z gives an exact zero; a power-of-two scale gives exact integers
    w2 = {"qweight": _pack_reference(q, q[::G][: K // G])[0][None], "qzeros": _pack_reference(q, q[:K // G])[1][None],
          "scales": np.full((1, K // G, N), np.float16(2.0 ** -3)).view(np.uint16), "group_size": G}
    q2 = oracle.gptq_unpack_q(w2["qweight"][0])
    z2 = oracle.gptq_unpack_z(w2["qzeros"][0])
    W2 = oracle.gptq_dequant_expert(w2, 0)
    assert np.array_equal(W2 * 8, (q2 - z2[np.arange(K) // G]).astype(np.float64))
    w3 = dict(w)
    w3["qzeros"] = _pack_reference(q, np.stack([q[g * G] for g in range(K // G)]))[1][None]
    W3 = oracle.gptq_dequant_expert(w3, 0)
    assert all(W3[g * G, n] == 0.0 for g in range(K // G) for n in range(N))


def test_gptq_generator_layout_matches_page():
    cfg = CONFIGS["decode_int4"].with_(T=4, H=256, I=128, E=3)
    d = make_inputs(cfg)
    g = d["gate"]
    assert g["qweight"].shape == (3, 256 // 8, 128) and g["qweight"].dtype == np.int32
    assert g["scales"].shape == (3, 256 // 128, 128)
    assert g["qzeros"].shape == (3, 256 // 128, 128 // 8) and g["qzeros"].dtype == np.int32
    s = oracle.f16_bits_to_f64(g["scales"])
    assert s.min() >= 0.0049 and s.max() <= 0.0201


# ----------------------------------------------------------------------------- GEMMs and the whole layer
def _dense_brute_force(d, ids, w):
    """Every token through every expert; the gate weight is zero for unselected experts."""
    cfg = d["cfg"]
    wg, wu, wd = oracle.moe_oracle._weights(d)
    X = oracle.bf16_bits_to_f64(d["x"])
    gate = np.zeros((cfg.T, cfg.E))
    for t in range(cfg.T):
        for j in range(cfg.top_k):
            gate[t, ids[t, j]] += float(w[t, j])
    out = np.zeros((cfg.T, cfg.H))
    for e in range(cfg.E):
        Wg, Wu, Wd = (oracle.expert_matrix(m, e) for m in (wg, wu, wd))
        a = X @ Wg.T
        f = ((a * (1 / (1 + np.exp(-a)))) * (X @ Wu.T)) @ Wd.T
        out += gate[:, e:e + 1] * f
    return out


@pytest.mark.parametrize("E,k,bs", [(1, 1, 16), (2, 1, 16), (8, 2, 16), (8, 2, 64), (4, 4, 32)])
def test_layer_matches_dense_brute_force(E, k, bs):
    cfg = MoeConfig("t", T=40, H=64, I=32, E=E, top_k=k, block_size=bs, seed=E * 10 + k)
    d = make_inputs(cfg)
    r = oracle.moe_layer(d)
    ref = _dense_brute_force(d, r["ids"], r["w"])
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-14)
    tok = oracle.moe_tokens(d, range(cfg.T))
    assert np.allclose(tok, ref, rtol=1e-12, atol=1e-14)


def test_layer_int4_matches_dense_brute_force():
    cfg = MoeConfig("t", T=12, H=256, I=128, E=5, top_k=3, block_size=16, weights="int4_gptq",
                    group_size=128, seed=9)
    d = make_inputs(cfg)
    r = oracle.moe_layer(d)
    assert np.allclose(r["out"], _dense_brute_force(d, r["ids"], r["w"]), rtol=1e-12, atol=1e-12)


def test_single_expert_is_textbook_swiglu():
    cfg = MoeConfig("t", T=16, H=64, I=48, E=1, top_k=1, block_size=16, seed=5)
    d = make_inputs(cfg)
    out = oracle.moe_layer(d)["out"]
    x = torch.from_numpy(oracle.bf16_bits_to_f64(d["x"]))
    Wg, Wu, Wd = (torch.from_numpy(oracle.bf16_bits_to_f64(d[k][0])) for k in ("wg", "wu", "wd"))
    ref = (torch.nn.functional.silu(x @ Wg.T) * (x @ Wu.T)) @ Wd.T
    assert np.allclose(out, ref.numpy(), rtol=1e-12, atol=1e-15)


def test_grouped_gemm_sentinel_rows_undefined():
    cfg = CONFIGS["tiny"]
    d = make_inputs(cfg)
    r = oracle.moe_layer(d)
    sid = r["align"]["sorted_ids"]
    pad = sid >= cfg.P
    assert np.isnan(r["h"][pad]).all() and np.isnan(r["y"][pad]).all()
    assert np.isfinite(r["h"][~pad]).all()


# ----------------------------------------------------------------------------- fp8 prefill
def test_e4m3_decode_against_torch():
    c = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f64(c)
    ref = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[~np.isnan(ours)], ref[~np.isnan(ref)])
    assert oracle.e4m3_to_f64(np.uint8([0x7E, 0x01, 0x08, 0x38]))[[0, 1, 2, 3]].tolist() == [448.0, 2.0 ** -9,
                                                                                               2.0 ** -6, 1.0]


def test_e4m3_round_against_torch():
    rng = np.random.default_rng(5)
    v = np.concatenate([(rng.standard_normal(200000) * 40).astype(np.float32),
                        (rng.standard_normal(20000) * 0.005).astype(np.float32),
                        np.float32([0.0, -0.0, 448, 463.99, 2 ** -9, 2 ** -10, 3 * 2 ** -10, 1.0625, 1.1875,
                                    -1.0625, 2 ** -6, 15 * 2 ** -10])])
    # every value halfway between two neighbouring codes (ties go to the even mantissa)
    vals = oracle.e4m3_to_f64(np.arange(0x7E, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids])
    v = v[np.abs(v) < 464]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_round(v), ref)


def test_quantize_rows_fp8_closed_forms():
    x = np.array([[1.0, -0.5, 0.25, 0.0],          # amax 1 -> +-448 for the amax element
                  [0.0, 0.0, 0.0, 0.0],            # zero row: scale 1, all codes 0
                  [-3.0, 1.5, 0.75, 3.0]])         # amax 3, reached twice with both signs
    q, s = oracle.quantize_rows_fp8(x)
    assert s.dtype == np.float32 and s[1] == 1.0 and (q[1] == 0).all()
    assert q[0, 0] == 0x7E and q[2, 0] == 0xFE and q[2, 3] == 0x7E
    assert s[0] == np.float32(1.0) / np.float32(448.0)
    # halves of the amax are exact powers of two below 448: 224, 112 (and their signs)
    assert oracle.e4m3_to_f64(q[0]).tolist() == [448.0, -224.0, 112.0, 0.0]
    back = oracle.e4m3_to_f64(q) * s[:, None].astype(np.float64)
    assert np.allclose(back, x, rtol=2 ** -4, atol=0)


def test_fp8_gemms_match_dequantised_definition():
    """The fp8 GEMMs are the plain SwiGLU / down products of the values torch decodes from the
    codes, scaled per token row and per output channel."""
    cfg = MoeConfig("t", T=24, H=64, I=48, E=3, top_k=2, block_size=16, weights="fp8", seed=21)
    d = make_inputs(cfg)
    r = oracle.moe_layer(d)
    al = r["align"]
    f64 = lambda c: torch.from_numpy(np.ascontiguousarray(c)).view(torch.float8_e4m3fn).to(torch.float64)
    X = f64(r["xq"]) * torch.from_numpy(r["sx"]).double()[:, None]
    sid = al["sorted_ids"]
    for rr in np.flatnonzero(sid < cfg.P):
        t, e = sid[rr] // cfg.top_k, al["expert_ids"][rr // cfg.block_size]
        Wg = f64(d["fp8_gate"]["codes"][e]) * torch.from_numpy(d["fp8_gate"]["scales"][e]).double()[:, None]
        Wu = f64(d["fp8_up"]["codes"][e]) * torch.from_numpy(d["fp8_up"]["scales"][e]).double()[:, None]
        h = torch.nn.functional.silu(Wg @ X[t]) * (Wu @ X[t])
        assert np.allclose(r["h"][rr], h.numpy(), rtol=1e-12, atol=1e-15)
        Wd = f64(d["fp8_down"]["codes"][e]) * torch.from_numpy(d["fp8_down"]["scales"][e]).double()[:, None]
        y = Wd @ (f64(r["hq"][rr]) * float(r["sh"][rr]))
        assert np.allclose(r["y"][rr], y.numpy(), rtol=1e-12, atol=1e-15)


def test_fp8_layer_sorted_equals_per_token():
    cfg = MoeConfig("t", T=30, H=64, I=32, E=5, top_k=2, block_size=16, weights="fp8", seed=22)
    d = make_inputs(cfg)
    r = oracle.moe_layer(d)
    tok = oracle.moe_tokens(d, range(cfg.T))
    assert np.allclose(r["out"], tok, rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------- combine
def test_combine_worked_example():
    g = golden("combine_worked.json")
    y = np.asarray(g["y"])
    out = oracle.combine(y, np.asarray(g["inv"]), np.float32(g["topk_w"]), 2, 2)
    assert np.array_equal(out, np.asarray(g["out"]))
    out2 = oracle.combine(y, None, np.float32(g["topk_w"]), 2, 2)
    assert np.array_equal(out2, np.asarray(g["out_slot_major"]))


# ----------------------------------------------------------------------------- LoRA fold
def _fold_case(c, *, delta_round=True, xa_round=True):
    """Run the oracle fold on one closed-form case (one row, one adapted expert)."""
    x = np.asarray(c["x"])[None, :]
    A = bf16(np.asarray(c["A"]))
    B = bf16(np.asarray(c["B"]))
    al = oracle.align(np.array([[0]]), 1, 1)
    tabs = oracle.pack_expert_tables([(0, A, B, c["scale"])])
    return oracle.lora_fold(np.asarray(c["base"])[None, :], x, tabs, al, 1)[0]


def test_lora_fold_rounding_pins():
    for c in golden("lora_fold_pins.json")["cases"]:
        assert np.array_equal(_fold_case(c), np.asarray(c["folded_bf16"])), c["name"]


def test_lora_fold_identities_and_windows():
    cfg = CONFIGS["lora_prefill"].with_(T=96, H=128, I=64, E=8, top_k=2, block_size=16,
                                        lora_rank=4, lora_max_rank=8)
    d = make_inputs(cfg)
    r = oracle.moe_layer(d)
    al = r["align"]
    xs = oracle.round_bf16(np.nan_to_num(r["h"]))
    base = oracle.round_bf16(np.nan_to_num(r["y"]))
    tabs = oracle.moe_oracle._lora_tables(d)
    full = oracle.lora_fold(base, xs, tabs, al, cfg.top_k)
    # chunked windows give the same bits as one call over everything
    chunked = base.copy()
    for s, e in oracle.lora_windows(len(al["sorted_ids"]), 40):
        chunked = oracle.lora_fold(chunked, xs, tabs, al, cfg.top_k, row_offset=s, row_end=e)
    assert np.array_equal(chunked, full)
    # only real rows of adapted (even) experts change
    P = cfg.P
    changed = np.any(full != base, axis=1)
    sid = al["sorted_ids"]
    for rr in range(len(sid)):
        e = np.searchsorted(al["offsets"], rr, side="right") - 1
        adapted = sid[rr] < P and e < cfg.E and e % 2 == 0
        if not adapted:
            assert not changed[rr]
    assert changed.sum() > 0
    # scale 0 leaves every row bit-identical
    a, b, s, n = tabs
    z = oracle.lora_fold(base, xs, (a, b, [0.0] * n, n), al, cfg.top_k)
    assert np.array_equal(z, base)
    # a per-token adapter map with all entries < 0 skips every row
    skip = oracle.lora_fold(base, xs, tabs, al, cfg.top_k, row_adapter=-np.ones(cfg.T, np.int32))
    assert np.array_equal(skip, base)


def _gather_case(c, x_gather):
    """One closed-form fold case through the slot-major gather fold (one slot, expert 0)."""
    x = np.asarray(c["x"])[None, :]
    tabs = oracle.pack_expert_tables([(0, bf16(np.asarray(c["A"])), bf16(np.asarray(c["B"])), c["scale"])])
    return oracle.lora_gather_fold(np.asarray(c["base"])[None, :], x, tabs, np.array([0]), 1,
                                   x_gather=x_gather)[0]


def test_lora_gather_fold_rounding_pins():
    for c in golden("lora_fold_pins.json")["cases"]:
        for xg in (False, True):
            assert np.array_equal(_gather_case(c, xg), np.asarray(c["folded_bf16"])), (c["name"], xg)


def test_lora_gather_fold_identity_closed_forms():
    """A_e = B_e = I and scale_e = 2^-(e+1) on a zero base: slot s ends up holding exactly
    scale_e * x[x row], which names the expert, the x row and the output row it used."""
    T, k, R, E = 5, 3, 8, 6
    n = T * k
    eye = bf16(np.eye(R))
    tabs = oracle.pack_expert_tables([(e, eye, eye, 2.0 ** -(e + 1)) for e in range(0, E, 2)])  # odd: unadapted
    assert tabs[3] == E - 1
    rng = np.random.default_rng(7)
    xs = oracle.round_bf16(rng.standard_normal((n, R)))        # bf16 values: the fold is exact
    ids = rng.integers(0, E, n)
    ids[[1, 4]] = [-1, E + 3]                                   # outside the table: skipped
    zero = np.zeros((n, R))

    def expect(xrow_of, rows=None, skip_tok=()):
        want = np.zeros((n, R))
        for s in range(n):
            e = ids[s]
            if e < 0 or e >= E - 1 or e % 2 or s // k in skip_tok:
                continue
            r = s if rows is None else rows[s]
            if r < 0:
                continue
            want[r] = 2.0 ** -(e + 1) * xs[xrow_of(s, r)]
        return want

    down = oracle.lora_gather_fold(zero, xs, tabs, ids, k)
    assert np.array_equal(down, expect(lambda s, r: r))
    gate_up = oracle.lora_gather_fold(zero, xs[:T], tabs, ids, k, x_gather=True)
    assert np.array_equal(gate_up, expect(lambda s, r: s // k))
    # adapter ids: 0 is the one installed adapter; a negative id is the base; id 3 names no
    # installed adapter, so its token is not folded either
    adapter = np.array([0, -1, 3, -2, 0], np.int32)
    skipped = oracle.lora_gather_fold(zero, xs, tabs, ids, k, row_adapter=adapter)
    assert np.array_equal(skipped, expect(lambda s, r: r, skip_tok=(1, 2, 3)))
    perm = rng.permutation(n).astype(np.int32)
    perm[[2, 9]] = -1
    mapped = oracle.lora_gather_fold(zero, xs, tabs, ids, k, row_map=perm)
    assert np.array_equal(mapped, expect(lambda s, r: r, rows=perm))


def test_lora_gather_fold_on_sorted_rows_equals_grouped_fold():
    """Through the inverse map, the slot-major fold on the sorted buffers is the grouped fold."""
    cfg = CONFIGS["lora_prefill"].with_(T=40, H=64, I=96, E=6, top_k=3, block_size=16,
                                        lora_rank=4, lora_max_rank=8)
    d = make_inputs(cfg)
    r = oracle.moe_layer(d)
    al = r["align"]
    xs = oracle.round_bf16(np.nan_to_num(r["h"]))
    base = oracle.round_bf16(np.nan_to_num(r["y"]))
    tabs = oracle.moe_oracle._lora_tables(d)
    ids = np.asarray(r["ids"]).reshape(-1)
    adapter = np.where(np.arange(cfg.T) % 5 == 2, -1, 0).astype(np.int32)
    grouped = oracle.lora_fold(base, xs, tabs, al, cfg.top_k, row_adapter=adapter)
    gathered = oracle.lora_gather_fold(base, xs, tabs, ids, cfg.top_k, row_adapter=adapter, row_map=al["inv"])
    assert np.array_equal(gathered, grouped)
    assert np.any(grouped != base)


def test_gate_up_lora_rounding_pin():
    """Gate and up are bf16 values before SiLU on the gate/up LoRA path (closed form)."""
    for c in golden("gate_up_lora_pins.json")["cases"]:
        x = bf16(np.asarray(c["x"])[None, :])
        al = oracle.align(np.array([[0]]), 1, 16)
        g = bf16(np.asarray(c["gate"]))[None]
        u = bf16(np.asarray(c["up"]))[None]
        h = oracle.grouped_gate_up_lora(x, g, u, al, 1, None, None)
        assert np.array_equal(h[0], np.asarray(c["h_bf16"])), c["name"]


def test_lora_fold_x_gather_closed_form():
    """Gate/up form of the grouped fold: with A = B = I, scale 2^-(e+1) and a zero base, sorted
    row r ends up holding scale_e * x[token of r] exactly."""
    T, k, R, E = 6, 2, 8, 4
    rng = np.random.default_rng(3)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    al = oracle.align(ids, E, 16)
    eye = bf16(np.eye(R))
    tabs = oracle.pack_expert_tables([(e, eye, eye, 2.0 ** -(e + 1)) for e in (0, 2)])
    xt = oracle.round_bf16(rng.standard_normal((T, R)))
    rows = len(al["sorted_ids"])
    y = oracle.lora_fold(np.zeros((rows, R)), xt, tabs, al, k, x_gather=True)
    want = np.zeros((rows, R))
    for r in range(rows):
        p = al["sorted_ids"][r]
        if p >= T * k:
            continue
        e = ids.reshape(-1)[p]
        if e in (0, 2):
            want[r] = 2.0 ** -(e + 1) * xt[p // k]
    assert np.array_equal(y, want)
    g = oracle.lora_gather_fold(np.zeros((rows, R)), xt, tabs, ids, k, x_gather=True, row_map=al["inv"])
    assert np.array_equal(g, want)


def _dense_brute_force_gate_up_lora(d, ids, w):
    """Every token through every expert with the gate/up and down folds, no sorting."""
    cfg = d["cfg"]
    wg, wu, wd = oracle.moe_oracle._weights(d)
    X = oracle.bf16_bits_to_f64(d["x"])
    gate = np.zeros((cfg.T, cfg.E))
    for t in range(cfg.T):
        for j in range(cfg.top_k):
            gate[t, ids[t, j]] += float(w[t, j])
    rb, f64 = oracle.round_bf16, oracle.bf16_bits_to_f64
    lids = list(d["lora_ids"])
    out = np.zeros((cfg.T, cfg.H))
    for e in range(cfg.E):
        i = lids.index(e) if e in lids else None
        proj = []
        for wm, key in ((wg, "gate"), (wu, "up")):
            v = rb(X @ oracle.expert_matrix(wm, e).T)
            if i is not None:
                xa = rb(X @ f64(d[f"lora_{key}_a"][i]).T)
                v = rb(v + float(d[f"lora_{key}_scale"][i]) * rb(xa @ f64(d[f"lora_{key}_b"][i]).T))
            proj.append(v)
        h = rb(proj[0] / (1 + np.exp(-proj[0])) * proj[1])
        y = h @ oracle.expert_matrix(wd, e).T
        if i is not None:
            y = y + float(d["lora_scale"][i]) * rb(rb(h @ f64(d["lora_a"][i]).T) @ f64(d["lora_b"][i]).T)
        out += gate[:, e:e + 1] * y
    return out


def test_layer_gate_up_lora_matches_dense_brute_force():
    cfg = MoeConfig("t", T=30, H=64, I=48, E=6, top_k=2, block_size=16, lora_rank=4, lora_max_rank=8,
                    lora_gate_up=True, seed=17)
    d = make_inputs(cfg)
    r = oracle.moe_layer(d)
    ref = _dense_brute_force_gate_up_lora(d, r["ids"], r["w"])
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-14)
    tok = oracle.moe_tokens(d, range(cfg.T))
    assert np.allclose(tok, ref, rtol=1e-12, atol=1e-14)
    # the gate/up folds change the result (they are not below the comparison)
    plain = dict(d)
    for key in ("lora_gate_a", "lora_up_a"):
        plain.pop(key)
    assert not np.allclose(oracle.moe_layer(plain)["out"], ref, rtol=1e-6, atol=1e-9)


def test_pack_expert_tables_and_windows():
    assert oracle.pack_expert_tables([]) is None
    a, b, s, n = oracle.pack_expert_tables([(2, "A2", "B2", 0.5), (0, "A0", "B0", 1.5), (2, "A2b", "B2b", 0.25)])
    assert n == 3 and a == ["A0", None, "A2b"] and b == ["B0", None, "B2b"] and s == [1.5, 0.0, 0.25]
    assert oracle.lora_window_tiles(0, 16320) == math.ceil(16320 / 64)
    assert oracle.lora_window_tiles(100, 100) == 1 and oracle.lora_window_tiles(0, 1) == 1
    w = oracle.lora_windows(10000, 4096)
    assert w == [(0, 4096), (4096, 8192), (8192, 10000)]
    with pytest.raises(ValueError):
        oracle.lora_windows(10, 0)


# ----------------------------------------------------------------------------- expert selection, pinned by hand-built stacks
# The brute forces above read each expert's matrix through the oracle's own readers.  These two
# build the stacked [E, N, K] bf16 slabs and the [E, K/8, N] GPTQ slabs from per-expert matrices
# they hold themselves, and evaluate the layer from those matrices, so a reader that picks the
# wrong slab (always expert 0, a neighbour) cannot agree with them.  Routing here is also
# recomputed independently: a stable argsort for the ids and scipy's softmax for the weights.

def _exact_bf16_bits(v):
    """bf16 bit patterns of values that bf16 holds exactly (asserted: the low fp32 half is zero)."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32)
    assert not np.any(u & np.uint32(0xFFFF)), "value not exact in bf16"
    return (u >> np.uint32(16)).astype(np.uint16)


def _independent_routing(logits, k):
    l = np.asarray(logits, np.float32)
    ids = np.argsort(-l, axis=1, kind="stable")[:, :k]
    p = scipy_softmax(l.astype(np.float64), axis=1)
    ps = np.take_along_axis(p, ids, 1)
    w = (ps / ps.sum(1, keepdims=True)).astype(np.float32).astype(np.float64)
    return ids, w


def _layer_from_matrices(x, ids, w, Wg, Wu, Wd):
    """out[t] = sum_j w[t,j] Wd[e] (silu(Wg[e] x_t) * (Wu[e] x_t)), e = ids[t,j]; matrices [E, N, K]."""
    T, k = ids.shape
    out = np.zeros((T, Wd.shape[1]))
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            g, u = Wg[e] @ x[t], Wu[e] @ x[t]
            out[t] += w[t, j] * (Wd[e] @ (g / (1.0 + np.exp(-g)) * u))
    return out


@pytest.mark.parametrize("E,k", [(3, 1), (5, 2), (8, 3)])
def test_expert_selection_bf16_hand_built_stacks(E, k):
    T, H, I = 20, 32, 16
    rng = np.random.default_rng(100 + E)
    # small integers / 64: at most 4 significant bits, exact in bf16; each expert also gets its
    # own offset (e + 1) / 64 on every entry so no two experts' matrices coincide
    mats = [rng.integers(-6, 7, (E, n, m)) / 64.0 + (np.arange(E) + 1)[:, None, None] / 64.0
            for n, m in ((I, H), (I, H), (H, I))]
    x = rng.integers(-4, 5, (T, H)) / 8.0
    logits = rng.standard_normal((T, E)).astype(np.float32)
    cfg = MoeConfig("t", T=T, H=H, I=I, E=E, top_k=k, block_size=16)
    d = {"cfg": cfg, "logits": logits, "x": _exact_bf16_bits(x),
         "wg": _exact_bf16_bits(mats[0]), "wu": _exact_bf16_bits(mats[1]), "wd": _exact_bf16_bits(mats[2])}
    ids, w = _independent_routing(logits, k)
    ref = _layer_from_matrices(x, ids, w, *mats)
    assert len(np.unique(ids)) >= 2          # several experts are in play, including e > 0
    r = oracle.moe_layer(d)
    assert np.array_equal(r["ids"], ids)
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(oracle.moe_tokens(d, range(T)), ref, rtol=1e-12, atol=1e-12)


def test_expert_selection_int4_hand_built_stacks():
    T, H, I, E, k, G = 12, 64, 32, 4, 2, 32
    rng = np.random.default_rng(77)

    def proj(K, N):
        # per expert: nibbles q, zero points z and power-of-two scales (exact in fp16), packed with
        # the independent packer; the dense matrix [N, K] is formed here from q, z, s directly
        q = rng.integers(0, 16, (E, K, N))
        z = rng.integers(0, 16, (E, K // G, N))
        s = np.float16(2.0) ** rng.integers(-7, -3, (E, K // G, N)).astype(np.float16)
        qw = np.stack([_pack_reference(q[e], z[e])[0] for e in range(E)])
        qz = np.stack([_pack_reference(q[e], z[e])[1] for e in range(E)])
        dense = np.stack([((q[e] - np.repeat(z[e], G, axis=0)) * np.repeat(s[e].astype(np.float64), G, axis=0)).T
                          for e in range(E)])
        return {"qweight": qw, "qzeros": qz, "scales": s.view(np.uint16), "group_size": G}, dense

    (wg, Wg), (wu, Wu), (wd, Wd) = proj(H, I), proj(H, I), proj(I, H)
    assert not np.allclose(Wg[0], Wg[1])
    x = rng.integers(-4, 5, (T, H)) / 8.0
    logits = rng.standard_normal((T, E)).astype(np.float32)
    cfg = MoeConfig("t", T=T, H=H, I=I, E=E, top_k=k, block_size=16, weights="int4_gptq", group_size=G)
    d = {"cfg": cfg, "logits": logits, "x": _exact_bf16_bits(x), "gate": wg, "up": wu, "down": wd}
    ids, w = _independent_routing(logits, k)
    ref = _layer_from_matrices(x, ids, w, Wg, Wu, Wd)
    assert len(np.unique(ids)) >= 2
    r = oracle.moe_layer(d)
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(oracle.moe_tokens(d, range(T)), ref, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- several adapters in one batch
# atlas moe_lora_grouped.rs, MoeExpertRoute: the adapter of a mixed batch's token comes from the per-row
# moe_row_adapter (< 0: base), not from the tables.  Reading: row a of the stacked tables is adapter a.

def _two_adapter_tables(R, E):
    """A_e = B_e = I for both adapters; adapter 0 adapts even experts with scale 2^-(e+1), adapter 1
    adapts experts 1, 2 (mod 3 != 0) with scale 2^-(e+8), so a folded value names its adapter and
    its expert (powers of two keep the bf16 fold exact)."""
    eye = bf16(np.eye(R))
    t0 = oracle.pack_expert_tables([(e, eye, eye, 2.0 ** -(e + 1)) for e in range(0, E, 2)])
    t1 = oracle.pack_expert_tables([(e, eye, eye, 2.0 ** -(e + 8)) for e in range(E) if e % 3])
    return [t0, t1]


def _scale_of(a, e):
    if a == 0 and e % 2 == 0:
        return 2.0 ** -(e + 1)
    if a == 1 and e % 3:
        return 2.0 ** -(e + 8)
    return None


def test_two_adapters_closed_form_grouped_and_gather():
    T, k, R, E, bs = 12, 2, 8, 6, 16
    rng = np.random.default_rng(21)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    ra = np.array([0, 1, -1, 1, 0, 7, 1, 0, -3, 1, 1, 0], np.int32)   # 7: no such adapter
    tabs = _two_adapter_tables(R, E)
    al = oracle.align(ids, E, bs)
    P = T * k
    xs = oracle.round_bf16(rng.standard_normal((len(al["sorted_ids"]), R)))   # bf16 values: exact fold
    got = oracle.lora_fold(np.zeros(xs.shape), xs, tabs, al, k, row_adapter=ra)
    want = np.zeros(xs.shape)
    for r, p in enumerate(al["sorted_ids"]):
        if p >= P:
            continue
        e, a = ids.reshape(-1)[p], ra[p // k]
        sc = _scale_of(a, e) if a >= 0 else None
        if sc is not None:
            want[r] = sc * xs[r]
    assert np.array_equal(got, want)
    assert (want != 0).any(axis=1).sum() > 4          # both adapters fold some rows
    # the slot-major gather fold: the same rule per slot
    xs2 = oracle.round_bf16(rng.standard_normal((P, R)))
    got2 = oracle.lora_gather_fold(np.zeros((P, R)), xs2, tabs, ids.reshape(-1), k, row_adapter=ra)
    want2 = np.zeros((P, R))
    for s in range(P):
        a = ra[s // k]
        sc = _scale_of(a, ids.reshape(-1)[s]) if a >= 0 else None
        if sc is not None:
            want2[s] = sc * xs2[s]
    assert np.array_equal(got2, want2)
    # without a map every token is adapter 0
    got3 = oracle.lora_gather_fold(np.zeros((P, R)), xs2, tabs, ids.reshape(-1), k)
    want3 = np.array([(_scale_of(0, e) or 0.0) * xs2[s] for s, e in enumerate(ids.reshape(-1))])
    assert np.array_equal(got3, want3)


def _dense_brute_force_adapters(d, ids, w):
    """Every token through every expert, the folds of its own adapter (read straight from the adapter
    dicts), no sorting."""
    cfg = d["cfg"]
    X = oracle.bf16_bits_to_f64(d["x"])
    rb, f64 = oracle.round_bf16, oracle.bf16_bits_to_f64
    Wg, Wu, Wd = (f64(d[key]) for key in ("wg", "wu", "wd"))
    out = np.zeros((cfg.T, cfg.H))
    for t in range(cfg.T):
        a = int(d["row_adapter"][t])
        ad = d["lora_adapters"][a] if a >= 0 else None
        lids = list(ad["lora_ids"]) if ad is not None else []
        for j in range(cfg.top_k):
            e = int(ids[t, j])
            i = lids.index(e) if e in lids else None
            proj = []
            for Wm, pre in ((Wg, "lora_gate"), (Wu, "lora_up")):
                v = rb(Wm[e] @ X[t])
                if i is not None and f"{pre}_a" in ad:
                    v = rb(v + float(ad[f"{pre}_scale"][i]) * rb(f64(ad[f"{pre}_b"][i]) @ rb(f64(ad[f"{pre}_a"][i]) @ X[t])))
                proj.append(v)
            h = rb(proj[0] / (1 + np.exp(-proj[0])) * proj[1])
            y = Wd[e] @ h
            if i is not None:
                y = y + float(ad["lora_scale"][i]) * rb(f64(ad["lora_b"][i]) @ rb(f64(ad["lora_a"][i]) @ h))
            out[t] += float(w[t, j]) * y
    return out


def test_layer_two_adapters_matches_dense_brute_force():
    cfg = MoeConfig("t", T=36, H=64, I=48, E=6, top_k=2, block_size=16, lora_rank=4, lora_max_rank=8,
                    lora_gate_up=True, lora_adapters=3, seed=23)
    d = make_inputs(cfg)
    assert set(np.unique(d["row_adapter"])) == {-1, 0, 1, 2}
    r = oracle.moe_layer(d)
    ref = _dense_brute_force_adapters(d, r["ids"], r["w"])
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-14)
    assert np.allclose(oracle.moe_tokens(d, range(cfg.T)), ref, rtol=1e-12, atol=1e-14)
    # each adapter matters: relabelling the tokens changes the result
    d2 = dict(d, row_adapter=np.where(d["row_adapter"] == 1, 2, np.where(d["row_adapter"] == 2, 1, d["row_adapter"])))
    assert not np.allclose(oracle.moe_layer(d2)["out"], ref, rtol=1e-6, atol=1e-9)
