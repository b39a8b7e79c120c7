"""The Python binding refuses buffers smaller than a call implies, before any pointer is taken.

The C ABI sees pointers and scalars only, so a too-small ``out`` or a weight stack with fewer
experts than the routing could only be caught here.  These run on CPU tensors: each call must
fail with the binding's shape message, not with the later "must live on a HIP device" check,
which shows the refusal comes before any launch could be enqueued.
"""
import pytest
import torch

import mixture_experts_routed_route_amd as m
from mixture_experts_routed_route_amd._lib import MOE_OP_DOWN, MOE_OP_GATE_UP_SILU

T, H, I, E, K, BS = 8, 64, 32, 4, 2, 16


def routing():
    return m.Routing.allocate(T * K, K, E, BS, "cpu")


def w(e=E, n=I, k=H):
    return m.Bf16Weight(torch.zeros((e, n, k), dtype=torch.bfloat16))


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def test_gemm_rejects_expert_count_mismatch():
    r = routing()
    with pytest.raises(ValueError, match="experts"):
        m.moe_grouped_gemm(MOE_OP_GATE_UP_SILU, bf(T, H), w(e=E - 1), w(e=E - 1), r, out=bf(r.max_pad, I))


def test_gemm_rejects_wrong_width_and_short_inputs():
    r = routing()
    with pytest.raises(ValueError, match="width must be K"):
        m.moe_grouped_gemm(MOE_OP_GATE_UP_SILU, bf(T, H + 8), w(), w(), r, out=bf(r.max_pad, I))
    with pytest.raises(ValueError, match="rows"):
        m.moe_grouped_gemm(MOE_OP_GATE_UP_SILU, bf(T - 1, H), w(), w(), r, out=bf(r.max_pad, I))
    with pytest.raises(ValueError, match="rows"):   # down reads max_pad sorted rows
        m.moe_grouped_gemm(MOE_OP_DOWN, bf(r.max_pad - 1, I), w(n=H, k=I), None, r, out=bf(r.max_pad, H))
    with pytest.raises(ValueError, match="one shape"):
        m.moe_grouped_gemm(MOE_OP_GATE_UP_SILU, bf(T, H), w(), w(n=I + 8), r, out=bf(r.max_pad, I))


def test_gemm_rejects_small_out():
    r = routing()
    with pytest.raises(ValueError, match="out is"):
        m.moe_grouped_gemm(MOE_OP_GATE_UP_SILU, bf(T, H), w(), w(), r, out=bf(r.max_pad - 16, I))
    with pytest.raises(ValueError, match="out is"):
        m.moe_grouped_gemm(MOE_OP_GATE_UP_SILU, bf(T, H), w(), w(), r, out=bf(r.max_pad, I - 8))


def test_gemm_fp8_rejects_short_scales():
    r = routing()
    f8 = m.Fp8Weight(torch.zeros((E, I, H), dtype=torch.uint8), torch.zeros((E, I), dtype=torch.float32))
    with pytest.raises(ValueError, match="a_scale"):
        m.moe_grouped_gemm_fp8(MOE_OP_GATE_UP_SILU, torch.zeros((T, H), dtype=torch.uint8),
                               torch.zeros(T - 1, dtype=torch.float32), f8, f8, r, out=bf(r.max_pad, I))


def test_combine_rejects_mismatched_out_and_inverse_map():
    ys = bf(40, H)
    tw = torch.zeros((T, K), dtype=torch.float32)
    with pytest.raises(ValueError, match="out is"):
        m.moe_combine(ys, torch.zeros(T * K, dtype=torch.int32), tw, out=bf(T, H - 8))
    with pytest.raises(ValueError, match="out is"):
        m.moe_combine(ys, torch.zeros(T * K, dtype=torch.int32), tw, out=bf(T - 1, H))
    with pytest.raises(ValueError, match="inv_sorted"):
        m.moe_combine(ys, torch.zeros(T * K - 1, dtype=torch.int32), tw, out=bf(T, H))


def test_route_and_align_reject_short_outputs():
    lg = torch.zeros((T, E), dtype=torch.float32)
    with pytest.raises(ValueError, match="topk_ids"):
        m.moe_route(lg, K, True, torch.zeros(T * K - 1, dtype=torch.int32), torch.zeros((T, K)))
    r = routing()
    r.sorted_ids = r.sorted_ids[:-1]
    with pytest.raises(ValueError, match="sorted_ids"):
        m.moe_align(torch.zeros((T, K), dtype=torch.int32), E, BS, out=r)


def test_lora_fold_rejects_mismatched_buffers():
    r = routing()
    tabs = m.LoraTables(torch.zeros(E, dtype=torch.int64), torch.zeros(E, dtype=torch.int64),
                        torch.zeros(E, dtype=torch.float32), E, I, H, 32)
    xa = bf(r.max_pad, 32)
    with pytest.raises(ValueError, match="x is"):
        m.moe_lora_fold(bf(r.max_pad, I + 8), bf(r.max_pad, H), tabs, r, xa=xa)
    with pytest.raises(ValueError, match="rows"):
        m.moe_lora_fold(bf(r.max_pad - 1, I), bf(r.max_pad, H), tabs, r, xa=xa)
    with pytest.raises(ValueError, match="base is"):
        m.moe_lora_fold(bf(r.max_pad, I), bf(r.max_pad - 1, H), tabs, r, xa=xa)
    with pytest.raises(ValueError, match="row_adapter"):
        m.moe_lora_fold(bf(r.max_pad, I), bf(r.max_pad, H), tabs, r, xa=xa,
                        row_adapter=torch.zeros(T - 1, dtype=torch.int32))


def test_down_lora_rejects_mismatched_buffers():
    r = routing()
    tabs = m.LoraTables(torch.zeros(E, dtype=torch.int64), torch.zeros(E, dtype=torch.int64),
                        torch.zeros(E, dtype=torch.float32), E, I, H, 32)
    xa = bf(r.max_pad, 32)
    wd = w(n=H, k=I)
    with pytest.raises(ValueError, match="xa must be"):
        m.moe_grouped_gemm_down_lora(bf(r.max_pad, I), wd, r, tabs, bf(r.max_pad - 16, 32), out=bf(r.max_pad, H))
    with pytest.raises(ValueError, match="tables are"):
        m.moe_grouped_gemm_down_lora(bf(r.max_pad, I), w(n=H, k=I + 8), r, tabs, xa, out=bf(r.max_pad, H))
    with pytest.raises(ValueError, match="rows"):
        m.moe_grouped_gemm_down_lora(bf(r.max_pad - 1, I), wd, r, tabs, xa, out=bf(r.max_pad, H))
    with pytest.raises(ValueError, match="out is"):
        m.moe_grouped_gemm_down_lora(bf(r.max_pad, I), wd, r, tabs, xa, out=bf(r.max_pad - 16, H))
    with pytest.raises(ValueError, match="row_adapter"):
        m.moe_grouped_gemm_down_lora(bf(r.max_pad, I), wd, r, tabs, xa, out=bf(r.max_pad, H),
                                     row_adapter=torch.zeros(T - 1, dtype=torch.int32))


def test_stack_lora_tables_layout():
    """Adapter a's tables land in row a of the [n_adapters, n_tab] stack; shorter tables and
    missing adapters are padded with unadapted (zero) entries."""
    def one(n_tab, base):
        return m.LoraTables(torch.arange(base, base + n_tab, dtype=torch.int64),
                            torch.arange(base + 100, base + 100 + n_tab, dtype=torch.int64),
                            torch.full((n_tab,), float(base), dtype=torch.float32), n_tab, I, H, 32)
    st = m.stack_lora_tables([one(3, 10), None, one(5, 20)], "cpu")
    assert (st.n_tab, st.n_adapters) == (5, 3)
    assert st.a_table.tolist() == [10, 11, 12, 0, 0] + [0] * 5 + [20, 21, 22, 23, 24]
    assert st.b_table.tolist() == [110, 111, 112, 0, 0] + [0] * 5 + [120, 121, 122, 123, 124]
    assert st.scale_table.tolist() == [10.0] * 3 + [0.0] * 7 + [20.0] * 5
    with pytest.raises(ValueError):
        m.stack_lora_tables([one(3, 10), m.LoraTables(torch.zeros(2, dtype=torch.int64), torch.zeros(2, dtype=torch.int64),
                                                      torch.zeros(2), 2, I, H, 64)], "cpu")
