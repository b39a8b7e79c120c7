"""The C-ABI library loads and exports every declared symbol; its pure host helpers agree
with the oracle and with the page's validator cases; invalid arguments are rejected on
the host before anything is enqueued.  CPU only: no call here reaches a launch."""
import ctypes
import os

import numpy as np
import pytest

import oracle
from _util import header_functions
from conftest import golden


@pytest.fixture(scope="module")
def L():
    from mixture_experts_routed_route_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from mixture_experts_routed_route_amd.build import build
        build()
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    from mixture_experts_routed_route_amd import _lib
    names = header_functions()
    assert len(names) == 24, names
    for n in names:
        assert hasattr(L, n), f"{n} not exported"
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"
    assert L.moe_abi_version() == 3


def test_max_padded_and_workspace(L):
    from mixture_experts_routed_route_amd import ops
    for P, E, bs in [(128, 8, 16), (8192, 8, 64), (65536, 128, 64), (96, 64, 16), (12288, 64, 64), (0, 4, 16)]:
        assert ops.max_padded(P, E, bs) == oracle.max_padded(P, E, bs)
        assert ops.align_workspace_bytes(P, E) >= 4 * E
    assert L.moe_align_max_padded(-1, 4, 16) == -1


def test_group_arrays_page_cases(L):
    from mixture_experts_routed_route_amd import ops, MoeError
    for c in golden("group_arrays_cases.json")["cases"]:
        per = [tuple(x) for x in c["per_expert"]]
        if c["ok"]:
            ops.check_group_arrays(c["num_experts"], per, c["offsets"])
        else:
            with pytest.raises(MoeError) as ei:
                ops.check_group_arrays(c["num_experts"], per, c["offsets"])
            if "message_contains" in c:
                assert c["message_contains"] in str(ei.value)


def test_pack_tables_matches_oracle(L):
    from mixture_experts_routed_route_amd._lib import check
    entries = [(4, 0x1000, 0x2000, 0.5), (0, 0x3000, 0x4000, 1.5), (4, 0x5000, 0x6000, 2.0), (2, 7, 8, 0.25)]
    n = len(entries)
    ids = (ctypes.c_int32 * n)(*[e[0] for e in entries])
    a = (ctypes.c_uint64 * n)(*[e[1] for e in entries])
    b = (ctypes.c_uint64 * n)(*[e[2] for e in entries])
    s = (ctypes.c_float * n)(*[e[3] for e in entries])
    ao, bo, so = (ctypes.c_uint64 * 8)(), (ctypes.c_uint64 * 8)(), (ctypes.c_float * 8)()
    nt = ctypes.c_int32(-1)
    check(L.moe_lora_pack_tables(ids, a, b, s, n, ao, bo, so, 8, ctypes.byref(nt)))
    ra, rb, rs, rn = oracle.pack_expert_tables(entries)
    assert nt.value == rn == 5
    assert list(ao[:5]) == [x or 0 for x in ra] and list(bo[:5]) == [x or 0 for x in rb]
    assert list(so[:5]) == rs
    check(L.moe_lora_pack_tables(None, None, None, None, 0, None, None, None, 0, ctypes.byref(nt)))
    assert nt.value == 0
    assert L.moe_lora_pack_tables(ids, a, b, s, n, ao, bo, so, 4, ctypes.byref(nt)) == -1  # cap too small


def test_windows_match_oracle(L):
    from mixture_experts_routed_route_amd import ops
    for total, cap in [(16320, 4096), (100, 100), (0, 7), (5, 1), (73600, 16384)]:
        assert ops.lora_windows(total, cap) == oracle.lora_windows(total, cap)
    for ro, re_ in [(0, 16320), (100, 100), (0, 1), (4096, 8192), (10, 3)]:
        assert ops.lora_window_tiles(ro, re_) == oracle.lora_window_tiles(ro, re_)
    with pytest.raises(ValueError):
        ops.lora_windows(10, 0)


def _rc(L, name, *args):
    rc = getattr(L, name)(*args)
    return rc, L.moe_last_error().decode()


def test_argument_validation_rejects_before_launch(L):
    P = ctypes.c_void_p
    fake = P(1 << 20)  # never dereferenced: every call below fails validation first
    rc, msg = _rc(L, "moe_route", fake, 4, 8, 0, 1, fake, fake, None)
    assert rc == -1 and "top_k" in msg
    rc, msg = _rc(L, "moe_route", fake, 4, 300, 2, 1, fake, fake, None)
    assert rc == -2 and "256" in msg
    rc, msg = _rc(L, "moe_route", None, 4, 8, 2, 1, fake, fake, None)
    assert rc == -1 and "logits" in msg
    rc, msg = _rc(L, "moe_route", P((1 << 20) + 4), 4, 8, 2, 1, fake, fake, None)
    assert rc == -1 and "aligned" in msg
    assert _rc(L, "moe_route", None, 0, 8, 2, 1, None, None, None)[0] == 0  # no tokens: nothing to do
    rc, msg = _rc(L, "moe_align", fake, 128, 8, 24, fake, fake, fake, fake, fake, fake, 512, fake, 4096, None)
    assert rc == -1 and "block_size" in msg
    rc, msg = _rc(L, "moe_align", fake, 128, 8, 16, fake, fake, fake, fake, fake, fake, 240, fake, 4096, None)
    assert rc == -1 and "max_pad" in msg
    rc, msg = _rc(L, "moe_align", fake, 128, 8, 16, fake, fake, fake, fake, fake, fake, 256, fake, 4, None)
    assert rc == -1 and "workspace" in msg
    rc, msg = _rc(L, "moe_align", fake, 128, 512, 16, fake, fake, fake, fake, fake, fake, 99999 * 16, fake,
                  1 << 30, None)
    assert rc == -2
    from mixture_experts_routed_route_amd._lib import MoeWeight
    w = MoeWeight(0, 0, 1 << 20, None, None)
    rc, msg = _rc(L, "moe_grouped_gemm", 0, fake, ctypes.byref(w), None, fake, fake, fake, fake, 128, 2, 8, 128,
                  256, 16, 256, None, 0, None)
    assert rc == -1 and "w1" in msg
    rc, msg = _rc(L, "moe_grouped_gemm", 1, fake, ctypes.byref(w), None, fake, fake, fake, fake, 128, 2, 8, 100,
                  256, 16, 256, None, 0, None)
    assert rc == -1 and "n 100" in msg
    rc, msg = _rc(L, "moe_grouped_gemm", 1, fake, ctypes.byref(w), None, fake, fake, fake, fake, 128, 2, 8, 128,
                  256, 16, 256, fake, 64, None)
    assert rc == -1 and "workspace_bytes" in msg
    assert L.moe_grouped_gemm_workspace_bytes() > 0
    w4 = MoeWeight(1, 100, 1 << 20, fake, fake)
    rc, msg = _rc(L, "moe_grouped_gemm", 1, fake, ctypes.byref(w4), None, fake, fake, fake, fake, 128, 2, 8, 128,
                  256, 16, 256, None, 0, None)
    assert rc == -1 and "group_size" in msg
    rc, msg = _rc(L, "moe_lora_fold", fake, fake, fake, fake, fake, 63, 1, 1408, 4096, 48, fake, 64, fake, 12288, 6,
                  None, fake, 16320, 0, 16320, 16320, 0, None)
    assert rc == -1 and "max_rank" in msg
    rc, msg = _rc(L, "moe_lora_fold", fake, fake, fake, fake, fake, 63, 1, 1408, 4096, 64, fake, 64, fake, 12288, 6,
                  None, fake, 100, 0, 16320, 16320, 0, None)
    assert rc == -1 and "cap" in msg
    rc, msg = _rc(L, "moe_lora_fold", fake, fake, fake, fake, fake, 65, 1, 1408, 4096, 64, fake, 64, fake, 12288, 6,
                  None, fake, 16320, 0, 16320, 16320, 0, None)
    assert rc == -1 and "n_tab" in msg
    # gather fold: (x, x_rows, base, base_rows, indices, n_slots, top_k, x_gather, row_map, row_adapter,
    #              a_table, b_table, scale_table, n_tab, n_adapters, k_in, n_out, max_rank, xa, stream)
    g = lambda **kw: _rc(L, "moe_lora_gather_fold", *[kw.get(k, v) for k, v in (
        ("x", fake), ("x_rows", 96), ("base", fake), ("base_rows", 96), ("indices", fake), ("n_slots", 96),
        ("top_k", 6), ("x_gather", 0), ("row_map", None), ("row_adapter", None), ("a", fake), ("b", fake),
        ("s", fake), ("n_tab", 63), ("n_adapters", 1), ("k_in", 1408), ("n_out", 2048), ("max_rank", 64), ("xa", fake),
        ("stream", None))])
    assert g(x_gather=2)[0] == -1 and "x_gather" in g(x_gather=2)[1]
    assert g(n_slots=95)[0] == -1 and "n_slots" in g(n_slots=95)[1]
    assert g(max_rank=48)[0] == -1 and "max_rank" in g(max_rank=48)[1]
    assert g(n_out=100)[0] == -1 and "n_out" in g(n_out=100)[1]
    assert g(base_rows=95)[0] == -1 and "base" in g(base_rows=95)[1]
    assert g(x_rows=95)[0] == -1 and "x has 95 rows" in g(x_rows=95)[1]
    assert g(x_gather=1, x_rows=15)[0] == -1                       # token-major x needs 16 rows
    assert g(indices=None)[0] == -1 and "indices" in g(indices=None)[1]
    assert g(row_map=P((1 << 20) + 4))[0] == -1 and "aligned" in g(row_map=P((1 << 20) + 4))[1]
    assert g(n_slots=0, x=None, base=None, indices=None)[0] == 0   # no slots: nothing to do
    assert g(n_tab=0, x=None)[0] == 0                               # no adapted expert: nothing to do
    assert g(n_adapters=0)[0] == -1 and "n_adapters" in g(n_adapters=0)[1]
    rc, msg = _rc(L, "moe_lora_fold", fake, fake, fake, fake, fake, 63, 1, 1408, 4096, 64, fake, 64, fake, 12288, 6,
                  None, fake, 16320, 0, 16320, 16320, 2, None)
    assert rc == -1 and "x_gather" in msg
    rc, msg = _rc(L, "moe_silu_mul", fake, fake, fake, None, 0, 16, 100, None)
    assert rc == -1 and "n 100" in msg
    assert _rc(L, "moe_silu_mul", None, None, None, None, 0, 0, 64, None)[0] == 0   # no rows: nothing to do
    rc, msg = _rc(L, "moe_silu_mul", fake, None, fake, None, 0, 16, 64, None)
    assert rc == -1 and "up" in msg
    rc, msg = _rc(L, "moe_grouped_gemm", 3, fake, ctypes.byref(w), None, fake, fake, fake, fake, 128, 2, 8, 128,
                  256, 16, 256, None, 0, None)
    assert rc == -1 and "unknown op" in msg
    rc, msg = _rc(L, "moe_grouped_gemm", 2, fake, ctypes.byref(w), ctypes.byref(w), fake, fake, fake, fake, 128, 2,
                  8, 128, 256, 16, 256, None, 0, None)
    assert rc == -1 and "takes no w1" in msg
    rc, msg = _rc(L, "moe_quantize_fp8", fake, 16, 24, None, 0, fake, fake, None)
    assert rc == -1 and "multiple of 16" in msg
    assert _rc(L, "moe_quantize_fp8", None, 0, 64, None, 0, None, None, None)[0] == 0   # no rows
    w8 = MoeWeight(2, 0, 1 << 20, fake, None)
    rc, msg = _rc(L, "moe_grouped_gemm_fp8", 2, fake, fake, ctypes.byref(w8), None, fake, fake, fake, 128, 2, 8, 128,
                  256, 16, 256, None, 0, None)
    assert rc == -1 and "op 2" in msg
    rc, msg = _rc(L, "moe_grouped_gemm_fp8", 1, fake, fake, ctypes.byref(w), None, fake, fake, fake, 128, 2, 8, 128,
                  256, 16, 256, None, 0, None)
    assert rc == -1 and "MOE_W_FP8" in msg
    rc, msg = _rc(L, "moe_grouped_gemm_fp8", 1, fake, fake, ctypes.byref(w8), None, fake, fake, fake, 128, 2, 8, 128,
                  264, 16, 256, None, 0, None)
    assert rc == -1 and "multiple of 16" in msg
    rc, msg = _rc(L, "moe_grouped_gemm_fp8", 1, fake, fake, ctypes.byref(w8), None, fake, fake, fake, 128, 2, 8, 128,
                  256, 16, 256, fake, 64, None)
    assert rc == -1 and "workspace_bytes" in msg
    # an expert matrix of 65536 x 65552 codes is over 4 GiB: the 32-bit load offsets cannot reach it
    rc, msg = _rc(L, "moe_grouped_gemm_fp8", 1, fake, fake, ctypes.byref(w8), None, fake, fake, fake, 128, 2, 8,
                  65536, 65552, 16, 256, None, 0, None)
    assert rc == -2 and "4 GiB" in msg
    rc, msg = _rc(L, "moe_grouped_gemm", 1, fake, ctypes.byref(w8), None, fake, fake, fake, fake, 128, 2, 8, 128,
                  256, 16, 256, None, 0, None)
    assert rc == -1 and "unsupported type" in msg
    # fused gate/up LoRA: (x, w_gate, w_up, hs, sorted_ids, offsets, P, top_k, E, n, k, bs, max_pad,
    #                      a_g, b_g, s_g, n_g, a_u, b_u, s_u, n_u, n_adapters, max_rank, row_adapter, xa, ws,
    #                      ws_bytes, stream)
    lg = lambda wg, rank: _rc(L, "moe_grouped_gemm_gate_up_lora", fake, ctypes.byref(wg), ctypes.byref(wg), fake, fake,
                              fake, 128, 2, 8, 128, 256, 16, 256, fake, fake, fake, 8, fake, fake, fake, 8, 1, rank, None,
                              fake, None, 0, None)
    rc, msg = lg(w4, 64)
    assert rc == -2 and "bf16" in msg
    rc, msg = lg(w, 48)
    assert rc == -1 and "max_rank" in msg
    # fused down LoRA: (hs, w_down, ys, sorted_ids, offsets, P, top_k, E, n, k, bs, max_pad, a, b, s, n_tab,
    #                    n_adapters, max_rank, row_adapter, xa, ws, ws_bytes, stream)
    ld = lambda wd, rank, n_tab=8, n_ad=1: _rc(L, "moe_grouped_gemm_down_lora", fake, ctypes.byref(wd), fake, fake,
                                               fake, 128, 2, 8, 256, 128, 16, 256, fake, fake, fake, n_tab, n_ad,
                                               rank, None, fake, None, 0, None)
    rc, msg = ld(w4, 64)
    assert rc == -2 and "bf16" in msg
    rc, msg = ld(w, 48)
    assert rc == -1 and "max_rank" in msg
    rc, msg = ld(w, 64, n_tab=9)
    assert rc == -1 and "n_tab" in msg
    rc, msg = ld(w, 64, n_ad=0)
    assert rc == -1 and "n_adapters" in msg
    rc, msg = _rc(L, "moe_lora_fold", fake, fake, fake, fake, fake, 63, 0, 1408, 4096, 64, fake, 64, fake, 12288, 6,
                  None, fake, 16320, 0, 16320, 16320, 0, None)
    assert rc == -1 and "n_adapters" in msg
    rc, msg = _rc(L, "moe_combine", fake, None, fake, fake, 4, 2, 100, 8, None)
    assert rc == -1 and "hidden" in msg
    rc, msg = _rc(L, "moe_combine", fake, None, fake, fake, 4, 2, 128, 7, None)
    assert rc == -1 and "slot-major" in msg
