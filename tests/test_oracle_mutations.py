"""Plant plausible mistakes in the oracle (CPU only) and check that the pins catch each.

Every mutation replaces one oracle function for the duration of a check and
runs the pins that cover it; at least one must fail.  This shows that the pins
are sensitive to a dropped term, a wrong index or order, a swapped operand and
a wrong rounding rule anywhere in the oracle.
"""
import contextlib

import numpy as np
import pytest

import oracle
import oracle.moe_oracle as om
import test_oracle_pins as pins


@contextlib.contextmanager
def patched(name, fn):
    old_mod, old_pkg = getattr(om, name), getattr(oracle, name)
    setattr(om, name, fn)
    setattr(oracle, name, fn)
    try:
        yield
    finally:
        setattr(om, name, old_mod)
        setattr(oracle, name, old_pkg)


def caught(name, fn, checks):
    with patched(name, fn):
        for check in checks:
            try:
                check()
            except (AssertionError, ValueError, IndexError):
                return True
    return False


# ----------------------------------------------------------------------------- mutants
def route_ties_high_first(logits, top_k, renormalize=True):
    logits = np.asarray(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, top_k), np.int32)
    w = np.empty((T, top_k), np.float32)
    for t in range(T):
        l = logits[t].astype(np.float64)
        sel = np.lexsort((-np.arange(E), -l))[:top_k]
        p = np.exp(l - l.max()); p /= p.sum()
        ws = p[sel] / p[sel].sum() if renormalize else p[sel]
        ids[t], w[t] = sel, ws.astype(np.float32)
    return ids, w


def route_no_renorm(logits, top_k, renormalize=True):
    return om._orig_route(logits, top_k, False)


def route_softmax_over_selected_only(logits, top_k, renormalize=True):
    ids, w = om._orig_route(logits, top_k, True)
    return ids, w  # drops the full-softmax denominator even when not renormalising


def align_descending_within_expert(topk_ids, num_experts, block_size, max_pad=None):
    al = om._orig_align(topk_ids, num_experts, block_size, max_pad)
    sid, inv = al["sorted_ids"].copy(), al["inv"].copy()
    off, cnt = al["offsets"], al["counts"]
    for e in range(num_experts):
        a, b = off[e], off[e] + cnt[e]
        sid[a:b] = sid[a:b][::-1]
        inv[sid[a:b]] = np.arange(a, b)
    return dict(al, sorted_ids=sid, inv=inv)


def align_unpadded(topk_ids, num_experts, block_size, max_pad=None):
    al = om._orig_align(topk_ids, num_experts, 1, max_pad)
    return dict(al, block_size=block_size, expert_ids=al["expert_ids"][: (len(al["sorted_ids"]) // block_size)])


def align_sentinel_minus_one(topk_ids, num_experts, block_size, max_pad=None):
    al = om._orig_align(topk_ids, num_experts, block_size, max_pad)
    sid = al["sorted_ids"].copy()
    sid[sid == al["num_pairs"]] = -1
    return dict(al, sorted_ids=sid)


def gptq_zero_plus_one(w, e):
    G = int(w["group_size"])
    q = om.gptq_unpack_q(w["qweight"][e])
    z = om.gptq_unpack_z(w["qzeros"][e]) + 1
    s = om.f16_bits_to_f64(w["scales"][e])
    g = np.arange(q.shape[0]) // G
    return (q - z[g]).astype(np.float64) * s[g]


def unpack_q_reversed(qweight_e):
    u = np.asarray(qweight_e).view(np.uint32)
    K8, N = u.shape
    q = np.empty((K8 * 8, N), np.int64)
    for s in range(8):
        q[s::8] = (u >> np.uint32(4 * (7 - s))) & np.uint32(0xF)
    return q


def gate_up_token_mod(x_bits, w_gate, w_up, al, top_k, rows=None):
    sid = al["sorted_ids"]
    h = np.full((len(sid), om.out_dim(w_gate)), np.nan)
    for e, rr in om._rows_by_expert(al, rows).items():
        X = om.bf16_bits_to_f64(x_bits[sid[rr] % top_k])
        h[rr] = om.silu(X @ om.expert_matrix(w_gate, e).T) * (X @ om.expert_matrix(w_up, e).T)
    return h


def gate_up_swapped(x_bits, w_gate, w_up, al, top_k, rows=None):
    return om._orig_gate_up(x_bits, w_up, w_gate, al, top_k, rows)


def combine_ignores_inv(y, inv, topk_w, T, top_k):
    return om._orig_combine(y, None, topk_w, T, top_k)


def combine_drops_weight(y, inv, topk_w, T, top_k):
    return om._orig_combine(y, inv, np.ones_like(np.asarray(topk_w, np.float32)), T, top_k)


def round_bf16_ties_away(v):
    v = np.asarray(v, np.float64)
    _, e = np.frexp(v)
    q = np.maximum(e - 8, -133)
    m = np.ldexp(v, -q)
    return np.ldexp(np.sign(m) * np.floor(np.abs(m) + 0.5), q)


def fold_no_xa_round(y, x, tables, al, top_k, row_adapter=None, row_offset=0, row_end=None, bf16_base=True):
    real = om.round_bf16
    calls = {"n": 0}

    def rb(v):
        calls["n"] += 1
        # the first rounding of every row is the shrink result: skip it
        return v if calls["n"] % 3 == 1 else real(v)
    om.round_bf16 = rb
    try:
        return om._orig_fold(y, x, tables, al, top_k, row_adapter, row_offset, row_end, bf16_base)
    finally:
        om.round_bf16 = real


def fold_no_delta_round(y, x, tables, al, top_k, row_adapter=None, row_offset=0, row_end=None, bf16_base=True):
    real = om.round_bf16
    calls = {"n": 0}

    def rb(v):
        calls["n"] += 1
        return v if calls["n"] % 3 == 2 else real(v)
    om.round_bf16 = rb
    try:
        return om._orig_fold(y, x, tables, al, top_k, row_adapter, row_offset, row_end, bf16_base)
    finally:
        om.round_bf16 = real


def gather_x_row_is_slot(y, x, tables, indices, top_k, x_gather=False, row_adapter=None, row_map=None):
    # the gate/up form reads x row s (clamped into x) instead of the owning token s // top_k
    if not x_gather:
        return om._orig_gather(y, x, tables, indices, top_k, False, row_adapter, row_map)
    n = len(np.ravel(indices))
    xx = np.stack([x[min(s, len(x) - 1)] for s in range(n)])
    return om._orig_gather(y, xx, tables, indices, top_k, False, row_adapter, row_map)


def gather_adapter_by_slot(y, x, tables, indices, top_k, x_gather=False, row_adapter=None, row_map=None):
    # the adapter map indexed by slot (clamped into the map) instead of by token
    if row_adapter is None:
        return om._orig_gather(y, x, tables, indices, top_k, x_gather, None, row_map)
    n = len(np.ravel(indices))
    ra = np.asarray(row_adapter)[np.minimum(np.arange(n), len(row_adapter) - 1)]
    if not x_gather:
        return om._orig_gather(y, x, tables, indices, 1, False, ra, row_map)
    xx = np.stack([x[s // top_k] for s in range(n)])
    return om._orig_gather(y, xx, tables, indices, 1, False, ra, row_map)


def gather_ignores_row_map(y, x, tables, indices, top_k, x_gather=False, row_adapter=None, row_map=None):
    return om._orig_gather(y, x, tables, indices, top_k, x_gather, row_adapter, None)


def gather_no_delta_round(y, x, tables, indices, top_k, x_gather=False, row_adapter=None, row_map=None):
    real = om.round_bf16
    calls = {"n": 0}

    def rb(v):
        calls["n"] += 1
        return v if calls["n"] % 3 == 2 else real(v)
    om.round_bf16 = rb
    try:
        return om._orig_gather(y, x, tables, indices, top_k, x_gather, row_adapter, row_map)
    finally:
        om.round_bf16 = real


def gate_up_lora_gate_unrounded(x_bits, w_gate, w_up, al, top_k, tabs_gate, tabs_up, row_adapter=None):
    real = om.round_bf16
    calls = {"n": 0}

    def rb(v):
        calls["n"] += 1
        return v if calls["n"] == 1 else real(v)  # the first expert's gate values stay unrounded
    om.round_bf16 = rb
    try:
        return om._orig_gate_up_lora(x_bits, w_gate, w_up, al, top_k, tabs_gate, tabs_up, row_adapter)
    finally:
        om.round_bf16 = real


def gate_up_lora_tables_swapped(x_bits, w_gate, w_up, al, top_k, tabs_gate, tabs_up, row_adapter=None):
    return om._orig_gate_up_lora(x_bits, w_gate, w_up, al, top_k, tabs_up, tabs_gate, row_adapter)


def fold_x_gather_by_row(y, x, tables, al, top_k, row_adapter=None, row_offset=0, row_end=None, bf16_base=True,
                         x_gather=False):
    if not x_gather:
        return om._orig_fold(y, x, tables, al, top_k, row_adapter, row_offset, row_end, bf16_base)
    # reads x at the sorted row (clamped into x) instead of at the row's token
    rows = len(al["sorted_ids"])
    xx = np.stack([x[min(r, len(x) - 1)] for r in range(rows)])
    return om._orig_fold(y, xx, tables, al, top_k, row_adapter, row_offset, row_end, bf16_base)


def e4m3_bias8(codes):
    return om._orig_e4m3(codes) / 2.0


def quantize_scale_447(x):
    xf = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(xf), axis=1)
    sc = np.where(amax > 0, amax / np.float32(447.0), np.float32(1.0)).astype(np.float32)
    f = np.where(amax > 0, np.float32(447.0) / np.maximum(amax, np.float32(1e-30)), np.float32(1.0))
    return om.e4m3_round((xf * f[:, None].astype(np.float32)).astype(np.float32)), sc


def fp8_gate_up_scale_by_column(xq, sx, w_gate, w_up, al, top_k):
    # the activation scale taken per output column instead of per token row
    h = om._orig_fp8_gate_up(xq, np.ones_like(sx), w_gate, w_up, al, top_k)
    return h * np.resize(sx, h.shape[1])[None, :]


def expert_matrix_always_first(w, e):
    return om._orig_expert_matrix(w, 0)


def expert_matrix_next_expert(w, e):
    E = w["qweight"].shape[0] if isinstance(w, dict) else w.shape[0]
    return om._orig_expert_matrix(w, (e + 1) % E)


def gptq_dequant_always_first(w, e):
    return om._orig_gptq_dequant(w, 0)


def adapter_tables_ignores_id(tables, a):
    # every non-negative adapter id gets adapter 0's tables
    return om._orig_adapter_tables(tables, 0 if a >= 0 else a)


def token_adapter_ignores_map(row_adapter, t):
    return 0


om._orig_route = om.route
om._orig_align = om.align
om._orig_gate_up = om.grouped_gate_up
om._orig_combine = om.combine
om._orig_fold = om.lora_fold
om._orig_gather = om.lora_gather_fold
om._orig_gate_up_lora = om.grouped_gate_up_lora
om._orig_e4m3 = om.e4m3_to_f64
om._orig_fp8_gate_up = om.grouped_gate_up_fp8
om._orig_expert_matrix = om.expert_matrix
om._orig_adapter_tables = om.adapter_tables
om._orig_gptq_dequant = om.gptq_dequant_expert

ROUTE_PINS = [pins.test_route_worked_examples, pins.test_route_special_cases, pins.test_route_brute_force_ids_and_sum]
ALIGN_PINS = [pins.test_align_worked_examples, lambda: pins.test_align_invariants_random(8, 2, 16, 64)]
LAYER_PINS = [lambda: pins.test_layer_matches_dense_brute_force(8, 2, 16), pins.test_single_expert_is_textbook_swiglu]
GATHER_PINS = [pins.test_lora_gather_fold_rounding_pins, pins.test_lora_gather_fold_identity_closed_forms,
               pins.test_lora_gather_fold_on_sorted_rows_equals_grouped_fold]
GATE_UP_LORA_PINS = [pins.test_gate_up_lora_rounding_pin, pins.test_layer_gate_up_lora_matches_dense_brute_force]
FP8_PINS = [pins.test_e4m3_decode_against_torch, pins.test_quantize_rows_fp8_closed_forms,
            pins.test_fp8_gemms_match_dequantised_definition]
INT4_PINS = [pins.test_gptq_unpack_and_dequant, pins.test_layer_int4_matches_dense_brute_force]
# pins that build the stacked expert slabs by hand and never read them through the oracle
ADAPTER_PINS = [pins.test_two_adapters_closed_form_grouped_and_gather,
                pins.test_layer_two_adapters_matches_dense_brute_force]
SELECTION_PINS = [lambda: pins.test_expert_selection_bf16_hand_built_stacks(5, 2),
                  pins.test_expert_selection_int4_hand_built_stacks]

MUTANTS = [
    ("route", route_ties_high_first, ROUTE_PINS),
    ("route", route_no_renorm, ROUTE_PINS),
    ("route", route_softmax_over_selected_only, ROUTE_PINS),
    ("align", align_descending_within_expert, ALIGN_PINS),
    ("align", align_unpadded, ALIGN_PINS),
    ("align", align_sentinel_minus_one, ALIGN_PINS),
    ("gptq_dequant_expert", gptq_zero_plus_one, INT4_PINS),
    ("gptq_unpack_q", unpack_q_reversed, INT4_PINS),
    ("expert_matrix", expert_matrix_always_first, SELECTION_PINS),
    ("expert_matrix", expert_matrix_next_expert, SELECTION_PINS),
    ("gptq_dequant_expert", gptq_dequant_always_first, SELECTION_PINS),
    ("adapter_tables", adapter_tables_ignores_id, ADAPTER_PINS),
    ("token_adapter", token_adapter_ignores_map, ADAPTER_PINS),
    ("grouped_gate_up", gate_up_token_mod, LAYER_PINS),
    ("grouped_gate_up", gate_up_swapped, LAYER_PINS),
    ("combine", combine_ignores_inv, [pins.test_combine_worked_example] + LAYER_PINS),
    ("combine", combine_drops_weight, [pins.test_combine_worked_example] + LAYER_PINS),
    ("round_bf16", round_bf16_ties_away, [pins.test_round_bf16_against_torch, pins.test_round_bf16_hand_values]),
    ("lora_fold", fold_no_xa_round, [pins.test_lora_fold_rounding_pins]),
    ("lora_fold", fold_no_delta_round, [pins.test_lora_fold_rounding_pins]),
    ("lora_gather_fold", gather_x_row_is_slot, GATHER_PINS),
    ("lora_gather_fold", gather_adapter_by_slot, GATHER_PINS),
    ("lora_gather_fold", gather_ignores_row_map, GATHER_PINS),
    ("lora_gather_fold", gather_no_delta_round, GATHER_PINS),
    ("grouped_gate_up_lora", gate_up_lora_gate_unrounded, GATE_UP_LORA_PINS),
    ("grouped_gate_up_lora", gate_up_lora_tables_swapped, GATE_UP_LORA_PINS),
    ("lora_fold", fold_x_gather_by_row, [pins.test_lora_fold_x_gather_closed_form]),
    ("e4m3_to_f64", e4m3_bias8, FP8_PINS),
    ("quantize_rows_fp8", quantize_scale_447, FP8_PINS),
    ("grouped_gate_up_fp8", fp8_gate_up_scale_by_column, FP8_PINS),
]


@pytest.mark.parametrize("name,fn,checks", MUTANTS, ids=[f"{n}:{f.__name__}" for n, f, _ in MUTANTS])
def test_pins_catch_planted_mistake(name, fn, checks):
    assert caught(name, fn, checks), f"no pin caught mutant {fn.__name__} of {name}"


def test_pins_pass_unmutated():
    for _, _, checks in MUTANTS[:1]:
        for c in ROUTE_PINS + ALIGN_PINS + LAYER_PINS + INT4_PINS:
            c()
