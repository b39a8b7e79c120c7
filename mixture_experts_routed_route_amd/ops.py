"""PyTorch-facing binding of the C ABI: argument checks and marshalling only.

Every step of the path runs in the HIP library; PyTorch supplies device memory and the
current stream.  Functions take and return ``torch`` tensors on a HIP device.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple, Union

import torch

from ._lib import (MOE_OP_DOWN, MOE_OP_GATE_UP_SILU, MOE_OP_GATHER, MOE_W_BF16, MOE_W_FP8, MOE_W_INT4_GPTQ,
                   MoeWeight, check, lib)

__all__ = [
    "Bf16Weight", "GptqWeight", "Fp8Weight", "Routing", "moe_quantize_fp8", "moe_grouped_gemm_fp8", "LoraTables", "max_padded", "align_workspace_bytes",
    "moe_route", "moe_align", "moe_align_noalloc", "moe_route_align", "moe_grouped_gemm", "gemm_workspace", "moe_lora_fold", "moe_lora_gather_fold", "stack_lora_tables", "moe_silu_mul", "moe_grouped_gemm_gate_up_lora", "moe_grouped_gemm_down_lora", "moe_combine", "pack_lora_tables",
    "lora_windows", "lora_window_tiles", "check_group_arrays",
]


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(ok: bool, msg: str) -> None:
    """Shape checks run before any pointer is taken: the C ABI sees no tensor sizes, so a buffer
    smaller than the call implies must be refused here, before a kernel could read or write past it."""
    if not ok:
        raise ValueError(msg)


def _rows_at_least(t: Optional[torch.Tensor], rows: int, name: str) -> None:
    if t is not None:
        _need(t.dim() >= 1 and t.shape[0] >= rows, f"{name} has {tuple(t.shape)}; needs >= {rows} rows")


def _numel_at_least(t: Optional[torch.Tensor], n: int, name: str) -> None:
    if t is not None:
        _need(t.numel() >= n, f"{name} has {t.numel()} elements; needs >= {n}")


def _check_routing(r: "Routing") -> None:
    _numel_at_least(r.counts, r.num_experts, "routing.counts")
    _numel_at_least(r.offsets, r.num_experts + 1, "routing.offsets")
    _numel_at_least(r.sorted_ids, r.max_pad, "routing.sorted_ids")
    _numel_at_least(r.expert_ids, r.max_pad // r.block_size, "routing.expert_ids")
    _numel_at_least(r.total_padded, 1, "routing.total_padded")
    _numel_at_least(r.inv_sorted, r.num_pairs, "routing.inv_sorted")


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on a HIP device (got {t.device})")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


# ----------------------------------------------------------------------------- weights
@dataclass
class Bf16Weight:
    """bf16 expert weights ``[E, N, K]`` (K contiguous)."""
    w: torch.Tensor

    @property
    def shape(self) -> Tuple[int, int, int]:
        return tuple(self.w.shape)

    def struct(self) -> MoeWeight:
        return MoeWeight(MOE_W_BF16, 0, _dev(self.w, torch.bfloat16, "weight"), None, None)


@dataclass
class GptqWeight:
    """GPTQ int4: qweight ``[E, K/8, N]`` int32, scales ``[E, K/G, N]`` fp16, qzeros ``[E, K/G, N/8]`` int32."""
    qweight: torch.Tensor
    scales: torch.Tensor
    qzeros: torch.Tensor
    group_size: int

    @property
    def shape(self) -> Tuple[int, int, int]:
        E, K8, N = self.qweight.shape
        return (E, N, K8 * 8)

    def struct(self) -> MoeWeight:
        return MoeWeight(MOE_W_INT4_GPTQ, int(self.group_size), _dev(self.qweight, torch.int32, "qweight"),
                         _dev(self.scales, torch.float16, "scales"), _dev(self.qzeros, torch.int32, "qzeros"))


@dataclass
class Fp8Weight:
    """FP8 E4M3 expert weights: codes ``[E, N, K]`` uint8, one fp32 scale per output channel ``[E, N]``."""
    codes: torch.Tensor
    scales: torch.Tensor

    @property
    def shape(self) -> Tuple[int, int, int]:
        return tuple(self.codes.shape)

    def struct(self) -> MoeWeight:
        return MoeWeight(MOE_W_FP8, 0, _dev(self.codes, torch.uint8, "codes"),
                         _dev(self.scales, torch.float32, "scales"), None)


Weight = Union[Bf16Weight, GptqWeight, Fp8Weight]


# ----------------------------------------------------------------------------- host helpers
def max_padded(num_pairs: int, num_experts: int, block_size: int) -> int:
    v = lib().moe_align_max_padded(num_pairs, num_experts, block_size)
    if v < 0:
        raise ValueError("invalid arguments")
    return int(v)


def align_workspace_bytes(num_pairs: int, num_experts: int) -> int:
    return int(lib().moe_align_workspace_bytes(num_pairs, num_experts))


def gemm_workspace(device) -> torch.Tensor:
    """A zero-filled workspace for moe_grouped_gemm's split-K tile balancing (calls leave it zeroed)."""
    n = int(lib().moe_grouped_gemm_workspace_bytes())
    return torch.zeros(n, dtype=torch.uint8, device=device)


def check_group_arrays(num_experts: int, per_expert: Sequence[Tuple[str, int]], offsets: Sequence[int]) -> None:
    n = len(per_expert)
    lens = (ctypes.c_int64 * max(n, 1))(*[int(l) for _, l in per_expert])
    names = (ctypes.c_char_p * max(n, 1))(*[s.encode() for s, _ in per_expert])
    off = (ctypes.c_int32 * max(len(offsets), 1))(*[int(o) for o in offsets])
    check(lib().moe_check_group_arrays(num_experts, lens, names, n, off, len(offsets)))


def lora_window_tiles(row_offset: int, row_end: int) -> int:
    return int(lib().moe_lora_window_tiles(row_offset, row_end))


def lora_windows(total_rows: int, cap: int) -> List[Tuple[int, int]]:
    n = lib().moe_lora_windows(total_rows, cap, None, None, 0)
    if n < 0:
        raise ValueError("grouped LoRA scratch capacity must be nonzero")
    s = (ctypes.c_int64 * max(n, 1))()
    e = (ctypes.c_int64 * max(n, 1))()
    lib().moe_lora_windows(total_rows, cap, s, e, n)
    return [(int(s[i]), int(e[i])) for i in range(n)]


# ----------------------------------------------------------------------------- A1 route
def moe_route(logits: torch.Tensor, top_k: int, renormalize: bool = True,
              topk_ids: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None):
    T, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty((T, top_k), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, top_k), dtype=torch.float32, device=logits.device)
    _numel_at_least(topk_ids, T * top_k, "topk_ids")
    _numel_at_least(topk_w, T * top_k, "topk_w")
    check(lib().moe_route(_dev(logits, torch.float32, "logits"), T, E, top_k, int(bool(renormalize)),
                          _dev(topk_ids, torch.int32, "topk_ids"), _dev(topk_w, torch.float32, "topk_w"),
                          _stream(logits)))
    return topk_ids, topk_w


# ----------------------------------------------------------------------------- A2 align
@dataclass
class Routing:
    """Outputs of moe_align (device tensors) plus the scalars that describe them."""
    counts: torch.Tensor
    offsets: torch.Tensor
    sorted_ids: torch.Tensor
    expert_ids: torch.Tensor
    total_padded: torch.Tensor
    inv_sorted: torch.Tensor
    workspace: torch.Tensor
    num_pairs: int
    top_k: int
    num_experts: int
    block_size: int
    max_pad: int

    @staticmethod
    def allocate(num_pairs: int, top_k: int, num_experts: int, block_size: int, device,
                 max_pad: Optional[int] = None) -> "Routing":
        mp = max_padded(num_pairs, num_experts, block_size) if max_pad is None else int(max_pad)
        i32 = dict(dtype=torch.int32, device=device)
        wsb = align_workspace_bytes(num_pairs, num_experts)
        return Routing(torch.empty(num_experts, **i32), torch.empty(num_experts + 1, **i32),
                       torch.empty(mp, **i32), torch.empty(mp // block_size, **i32), torch.empty(1, **i32),
                       torch.empty(max(num_pairs, 1), **i32), torch.empty(max(wsb // 4, 1), **i32),
                       num_pairs, top_k, num_experts, block_size, mp)


def moe_align(topk_ids: torch.Tensor, num_experts: int, block_size: int, max_pad: Optional[int] = None,
              out: Optional[Routing] = None) -> Routing:
    P = topk_ids.numel()
    top_k = topk_ids.shape[-1] if topk_ids.dim() == 2 else 1
    r = out if out is not None else Routing.allocate(P, top_k, num_experts, block_size, topk_ids.device, max_pad)
    if r.num_pairs != P or r.num_experts != num_experts or r.block_size != block_size:
        raise ValueError("preallocated Routing does not match the call")
    _check_routing(r)
    check(lib().moe_align(_dev(topk_ids, torch.int32, "topk_ids"), P, num_experts, block_size,
                          _dev(r.counts, torch.int32, "counts"), _dev(r.offsets, torch.int32, "offsets"),
                          _dev(r.sorted_ids, torch.int32, "sorted_ids"),
                          _dev(r.expert_ids, torch.int32, "expert_ids"),
                          _dev(r.total_padded, torch.int32, "total_padded"),
                          _dev(r.inv_sorted, torch.int32, "inv_sorted"), r.max_pad,
                          _dev(r.workspace, torch.int32, "workspace"), r.workspace.numel() * 4,
                          _stream(topk_ids)))
    return r


def moe_align_noalloc(topk_ids: torch.Tensor, num_experts: int, block_size: int, out: Routing) -> Routing:
    """moe_align into preallocated ``out`` with the library's static histogram table instead of a
    workspace (for callers that cannot allocate; calls that overlap on one GPU race)."""
    P = topk_ids.numel()
    r = out
    if r.num_pairs != P or r.num_experts != num_experts or r.block_size != block_size:
        raise ValueError("preallocated Routing does not match the call")
    _check_routing(r)
    check(lib().moe_align_noalloc(_dev(topk_ids, torch.int32, "topk_ids"), P, num_experts, block_size,
                                  _dev(r.counts, torch.int32, "counts"), _dev(r.offsets, torch.int32, "offsets"),
                                  _dev(r.sorted_ids, torch.int32, "sorted_ids"),
                                  _dev(r.expert_ids, torch.int32, "expert_ids"),
                                  _dev(r.total_padded, torch.int32, "total_padded"),
                                  _dev(r.inv_sorted, torch.int32, "inv_sorted"), r.max_pad, _stream(topk_ids)))
    return r


def moe_route_align(logits: torch.Tensor, top_k: int, renormalize: bool, block_size: int,
                    topk_ids: torch.Tensor, topk_w: torch.Tensor, out: Routing) -> Routing:
    """moe_route then moe_align on its ids, as one call (one launch when the pairs fit one chunk)."""
    T, E = logits.shape
    r = out
    if r.num_pairs != T * top_k or r.num_experts != E or r.block_size != block_size:
        raise ValueError("preallocated Routing does not match the call")
    _check_routing(r)
    _numel_at_least(topk_ids, T * top_k, "topk_ids")
    _numel_at_least(topk_w, T * top_k, "topk_w")
    check(lib().moe_route_align(_dev(logits, torch.float32, "logits"), T, E, top_k, int(bool(renormalize)),
                                _dev(topk_ids, torch.int32, "topk_ids"), _dev(topk_w, torch.float32, "topk_w"),
                                block_size, _dev(r.counts, torch.int32, "counts"),
                                _dev(r.offsets, torch.int32, "offsets"),
                                _dev(r.sorted_ids, torch.int32, "sorted_ids"),
                                _dev(r.expert_ids, torch.int32, "expert_ids"),
                                _dev(r.total_padded, torch.int32, "total_padded"),
                                _dev(r.inv_sorted, torch.int32, "inv_sorted"), r.max_pad,
                                _dev(r.workspace, torch.int32, "workspace"), r.workspace.numel() * 4,
                                _stream(logits)))
    return r


# ----------------------------------------------------------------------------- A3 / A4 grouped GEMM
def _check_gemm_shapes(op: int, a: torch.Tensor, w0, w1, routing: "Routing", out: torch.Tensor, who: str) -> None:
    E, N, K = w0.shape
    _need(E == routing.num_experts, f"{who}: the weights hold {E} experts, the routing {routing.num_experts}")
    if op == MOE_OP_GATE_UP_SILU:
        _need(w1 is not None and tuple(w1.shape) == tuple(w0.shape),
              f"{who}: gate and up weights must have one shape")
    _need(a.dim() == 2 and a.shape[1] == K, f"{who}: a is {tuple(a.shape)}; its width must be K={K}")
    rows = routing.max_pad if op == MOE_OP_DOWN else routing.num_pairs // routing.top_k
    _rows_at_least(a, rows, f"{who}: a")
    _need(out.dim() == 2 and out.shape[1] == N and out.shape[0] >= routing.max_pad,
          f"{who}: out is {tuple(out.shape)}; needs [>= {routing.max_pad}, {N}]")
    _check_routing(routing)


def moe_grouped_gemm(op: int, a: torch.Tensor, w0: Weight, w1: Optional[Weight], routing: Routing,
                     out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """op = MOE_OP_GATE_UP_SILU (a = x [T, K], w0 = gate, w1 = up), MOE_OP_DOWN (a = Hs [max_pad, K])
    or MOE_OP_GATHER (a = x [T, K], w0 = one projection, no activation).

    ``workspace`` (from ``gemm_workspace``) lets bf16 launches split the last partial wave of tiles
    over K; without it every tile is computed by one workgroup."""
    E, N, K = w0.shape
    if out is None:
        out = torch.empty((routing.max_pad, N), dtype=torch.bfloat16, device=a.device)
    _check_gemm_shapes(op, a, w0, w1, routing, out, "moe_grouped_gemm")
    s0 = w0.struct()
    s1 = w1.struct() if w1 is not None else None
    check(lib().moe_grouped_gemm(op, _dev(a, torch.bfloat16, "a"), ctypes.byref(s0),
                                 ctypes.byref(s1) if s1 is not None else None, _dev(out, torch.bfloat16, "out"),
                                 _dev(routing.sorted_ids, torch.int32, "sorted_ids"),
                                 _dev(routing.expert_ids, torch.int32, "expert_ids"),
                                 _dev(routing.offsets, torch.int32, "offsets"), routing.num_pairs, routing.top_k,
                                 routing.num_experts, N, K, routing.block_size, routing.max_pad,
                                 _dev(workspace, torch.uint8, "workspace") if workspace is not None else None,
                                 workspace.numel() if workspace is not None else 0, _stream(a)))
    return out


# ----------------------------------------------------------------------------- fp8 prefill
def moe_quantize_fp8(x: torch.Tensor, q: torch.Tensor, scale: torch.Tensor,
                     routing: Optional[Routing] = None) -> None:
    """Per-row e4m3 codes and scales of bf16 rows; with ``routing`` only the real sorted rows."""
    rows, k = x.shape
    _need(tuple(q.shape) == (rows, k), f"moe_quantize_fp8: q is {tuple(q.shape)}; needs {(rows, k)}")
    _numel_at_least(scale, rows, "moe_quantize_fp8: scale")
    if routing is not None:
        _numel_at_least(routing.sorted_ids, rows, "moe_quantize_fp8: routing.sorted_ids")
    check(lib().moe_quantize_fp8(_dev(x, torch.bfloat16, "x"), rows, k,
                                 _dev(routing.sorted_ids, torch.int32, "sorted_ids") if routing is not None else None,
                                 routing.num_pairs if routing is not None else 0, _dev(q, torch.uint8, "q"),
                                 _dev(scale, torch.float32, "scale"), _stream(x)))


def moe_grouped_gemm_fp8(op: int, a: torch.Tensor, a_scale: torch.Tensor, w0: Fp8Weight, w1: Optional[Fp8Weight],
                         routing: Routing, out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """op = MOE_OP_GATE_UP_SILU (a = x codes [T, K] by token) or MOE_OP_DOWN (a = Hs codes [max_pad, K])."""
    E, N, K = w0.shape
    if out is None:
        out = torch.empty((routing.max_pad, N), dtype=torch.bfloat16, device=a.device)
    _check_gemm_shapes(op, a, w0, w1, routing, out, "moe_grouped_gemm_fp8")
    _numel_at_least(a_scale, a.shape[0], "moe_grouped_gemm_fp8: a_scale")
    s0 = w0.struct()
    s1 = w1.struct() if w1 is not None else None
    check(lib().moe_grouped_gemm_fp8(op, _dev(a, torch.uint8, "a"), _dev(a_scale, torch.float32, "a_scale"),
                                     ctypes.byref(s0), ctypes.byref(s1) if s1 is not None else None,
                                     _dev(out, torch.bfloat16, "out"),
                                     _dev(routing.sorted_ids, torch.int32, "sorted_ids"),
                                     _dev(routing.offsets, torch.int32, "offsets"), routing.num_pairs, routing.top_k,
                                     routing.num_experts, N, K, routing.block_size, routing.max_pad,
                                     _dev(workspace, torch.uint8, "workspace") if workspace is not None else None,
                                     workspace.numel() if workspace is not None else 0, _stream(a)))
    return out


# ----------------------------------------------------------------------------- A5 LoRA fold
@dataclass
class LoraTables:
    """Device tables of the per-expert LoRA of one projection (atlas MoeExpertRoute), for
    ``n_adapters`` installed adapters: row a of the [n_adapters, n_tab] tables belongs to adapter a,
    whose tokens the per-token ``row_adapter`` map names (NULL map: adapter 0)."""
    a_table: torch.Tensor      # int64 [n_adapters * n_tab] addresses (0 = unadapted)
    b_table: torch.Tensor
    scale_table: torch.Tensor  # float32 [n_adapters * n_tab]
    n_tab: int
    k_in: int
    n_out: int
    max_rank: int
    n_adapters: int = 1
    keep: List[torch.Tensor] = field(default_factory=list)  # owners of the A/B memory


def pack_lora_tables(ids: Sequence[int], a: Sequence[torch.Tensor], b: Sequence[torch.Tensor],
                     scales: Sequence[float], device) -> Optional[LoraTables]:
    """A_e bf16 [max_rank, k_in], B_e bf16 [n_out, max_rank] on the device; tables via moe_lora_pack_tables."""
    n = len(ids)
    if n == 0:
        return None
    for t in list(a) + list(b):
        _dev(t, torch.bfloat16, "lora weight")
    cap = max(int(i) for i in ids) + 1
    ids_c = (ctypes.c_int32 * n)(*[int(i) for i in ids])
    a_c = (ctypes.c_uint64 * n)(*[t.data_ptr() for t in a])
    b_c = (ctypes.c_uint64 * n)(*[t.data_ptr() for t in b])
    s_c = (ctypes.c_float * n)(*[float(s) for s in scales])
    ao, bo, so = (ctypes.c_uint64 * cap)(), (ctypes.c_uint64 * cap)(), (ctypes.c_float * cap)()
    n_tab = ctypes.c_int32(0)
    check(lib().moe_lora_pack_tables(ids_c, a_c, b_c, s_c, n, ao, bo, so, cap, ctypes.byref(n_tab)))
    k = n_tab.value
    as_i64 = lambda arr: torch.tensor([int(v) - (1 << 64) if int(v) >= (1 << 63) else int(v) for v in arr[:k]],
                                      dtype=torch.int64)
    max_rank, k_in = a[0].shape
    n_out = b[0].shape[0]
    return LoraTables(as_i64(ao).to(device), as_i64(bo).to(device),
                      torch.tensor(list(so[:k]), dtype=torch.float32).to(device), k, k_in, n_out, max_rank,
                      keep=list(a) + list(b))


def stack_lora_tables(adapters: Sequence[Optional[LoraTables]], device) -> LoraTables:
    """The tables of several adapters as one [n_adapters, n_tab] set (adapter id = position; None =
    an id with no tables for this projection).  n_tab is the longest table; shorter ones are padded
    with unadapted entries."""
    real = [t for t in adapters if t is not None]
    if not real:
        raise ValueError("no adapter has tables")
    t0 = real[0]
    if any((t.k_in, t.n_out, t.max_rank, t.n_adapters) != (t0.k_in, t0.n_out, t0.max_rank, 1) for t in real):
        raise ValueError("stacked adapters must be single-adapter tables with one k_in, n_out and max_rank")
    n_tab = max(t.n_tab for t in real)
    n = len(adapters)
    a = torch.zeros(n * n_tab, dtype=torch.int64, device=device)
    b = torch.zeros_like(a)
    sc = torch.zeros(n * n_tab, dtype=torch.float32, device=device)
    keep: List[torch.Tensor] = []
    for i, t in enumerate(adapters):
        if t is None:
            continue
        a[i * n_tab: i * n_tab + t.n_tab] = t.a_table
        b[i * n_tab: i * n_tab + t.n_tab] = t.b_table
        sc[i * n_tab: i * n_tab + t.n_tab] = t.scale_table
        keep += t.keep
    return LoraTables(a, b, sc, n_tab, t0.k_in, t0.n_out, t0.max_rank, n_adapters=n, keep=keep)


def moe_lora_fold(x: torch.Tensor, base: torch.Tensor, tables: LoraTables, routing: Routing,
                  row_adapter: Optional[torch.Tensor] = None, xa: Optional[torch.Tensor] = None,
                  row_offset: int = 0, row_end: Optional[int] = None, x_gather: bool = False) -> torch.Tensor:
    """Fold in place into ``base`` over the window [row_offset, row_end) of the sorted rows.
    ``x_gather``: x is the token-major layer input and base a sorted gate or up output."""
    if row_end is None:
        row_end = routing.max_pad
    if xa is None:
        xa = torch.empty((max(row_end - row_offset, 1), tables.max_rank), dtype=torch.bfloat16, device=x.device)
    who = "moe_lora_fold"
    _need(x.dim() == 2 and x.shape[1] == tables.k_in, f"{who}: x is {tuple(x.shape)}; width must be {tables.k_in}")
    _rows_at_least(x, routing.num_pairs // routing.top_k if x_gather else routing.max_pad, f"{who}: x")
    _need(base.dim() == 2 and base.shape[1] == tables.n_out and base.shape[0] >= routing.max_pad,
          f"{who}: base is {tuple(base.shape)}; needs [>= {routing.max_pad}, {tables.n_out}]")
    _need(xa.dim() == 2 and xa.shape[1] == tables.max_rank, f"{who}: xa must be [cap, {tables.max_rank}]")
    _numel_at_least(row_adapter, routing.num_pairs // routing.top_k, f"{who}: row_adapter")
    _check_routing(routing)
    check(lib().moe_lora_fold(
        _dev(x, torch.bfloat16, "x"), _dev(base, torch.bfloat16, "base"), _dev(tables.a_table, torch.int64, "a_table"),
        _dev(tables.b_table, torch.int64, "b_table"), _dev(tables.scale_table, torch.float32, "scale_table"),
        tables.n_tab, tables.n_adapters, tables.k_in, tables.n_out, tables.max_rank,
        _dev(routing.offsets, torch.int32, "offsets"),
        routing.num_experts, _dev(routing.sorted_ids, torch.int32, "sorted_ids"), routing.num_pairs, routing.top_k,
        _dev(row_adapter, torch.int32, "row_adapter") if row_adapter is not None else None,
        _dev(xa, torch.bfloat16, "xa"), xa.shape[0], row_offset, row_end, routing.max_pad, int(bool(x_gather)),
        _stream(x)))
    return base


def moe_grouped_gemm_gate_up_lora(x: torch.Tensor, gate: Bf16Weight, up: Bf16Weight, routing: Routing,
                                  lora_gate: Optional[LoraTables], lora_up: Optional[LoraTables],
                                  xa: torch.Tensor, out: Optional[torch.Tensor] = None,
                                  row_adapter: Optional[torch.Tensor] = None,
                                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Hs with the gate and up LoRA folded in the gate/up GEMM's epilogue; xa: bf16 [2, max_pad, rank]."""
    E, N, K = gate.shape
    tabs = [t for t in (lora_gate, lora_up) if t is not None]
    if not tabs:
        raise ValueError("at least one of lora_gate, lora_up is needed")
    rank = tabs[0].max_rank
    if any(t.max_rank != rank or t.k_in != K or t.n_out != N for t in tabs):
        raise ValueError("gate and up tables must share max_rank and match the weights")
    n_ad = tabs[0].n_adapters
    if any(t.n_adapters != n_ad for t in tabs):
        raise ValueError("gate and up tables must hold the same adapters")
    if tuple(xa.shape) != (2, routing.max_pad, rank):
        raise ValueError(f"xa must be [2, {routing.max_pad}, {rank}]")
    if out is None:
        out = torch.empty((routing.max_pad, N), dtype=torch.bfloat16, device=x.device)
    _check_gemm_shapes(MOE_OP_GATE_UP_SILU, x, gate, up, routing, out, "moe_grouped_gemm_gate_up_lora")
    _numel_at_least(row_adapter, routing.num_pairs // routing.top_k, "moe_grouped_gemm_gate_up_lora: row_adapter")
    sg, su = gate.struct(), up.struct()

    def tab(t):
        if t is None:
            return None, None, None, 0
        return (_dev(t.a_table, torch.int64, "a_table"), _dev(t.b_table, torch.int64, "b_table"),
                _dev(t.scale_table, torch.float32, "scale_table"), t.n_tab)
    ag, bg, cg, ng = tab(lora_gate)
    au, bu, cu, nu = tab(lora_up)
    check(lib().moe_grouped_gemm_gate_up_lora(
        _dev(x, torch.bfloat16, "x"), ctypes.byref(sg), ctypes.byref(su), _dev(out, torch.bfloat16, "out"),
        _dev(routing.sorted_ids, torch.int32, "sorted_ids"), _dev(routing.offsets, torch.int32, "offsets"),
        routing.num_pairs, routing.top_k, routing.num_experts, N, K, routing.block_size, routing.max_pad,
        ag, bg, cg, ng, au, bu, cu, nu, n_ad, rank,
        _dev(row_adapter, torch.int32, "row_adapter") if row_adapter is not None else None,
        _dev(xa, torch.bfloat16, "xa"), _dev(workspace, torch.uint8, "workspace") if workspace is not None else None,
        workspace.numel() if workspace is not None else 0, _stream(x)))
    return out


def moe_grouped_gemm_down_lora(hs: torch.Tensor, down: Bf16Weight, routing: Routing, tables: LoraTables,
                               xa: torch.Tensor, out: Optional[torch.Tensor] = None,
                               row_adapter: Optional[torch.Tensor] = None,
                               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Ys with the down-projection LoRA folded in the down GEMM's epilogue; xa: bf16 [max_pad, max_rank]."""
    E, N, K = down.shape
    who = "moe_grouped_gemm_down_lora"
    _need(tables.k_in == K and tables.n_out == N,
          f"{who}: tables are [{tables.n_out} x {tables.k_in}], the weights [{N} x {K}]")
    _need(tuple(xa.shape) == (routing.max_pad, tables.max_rank), f"{who}: xa must be [{routing.max_pad}, {tables.max_rank}]")
    if out is None:
        out = torch.empty((routing.max_pad, N), dtype=torch.bfloat16, device=hs.device)
    _check_gemm_shapes(MOE_OP_DOWN, hs, down, None, routing, out, who)
    _numel_at_least(row_adapter, routing.num_pairs // routing.top_k, f"{who}: row_adapter")
    sd = down.struct()
    check(lib().moe_grouped_gemm_down_lora(
        _dev(hs, torch.bfloat16, "hs"), ctypes.byref(sd), _dev(out, torch.bfloat16, "out"),
        _dev(routing.sorted_ids, torch.int32, "sorted_ids"), _dev(routing.offsets, torch.int32, "offsets"),
        routing.num_pairs, routing.top_k, routing.num_experts, N, K, routing.block_size, routing.max_pad,
        _dev(tables.a_table, torch.int64, "a_table"), _dev(tables.b_table, torch.int64, "b_table"),
        _dev(tables.scale_table, torch.float32, "scale_table"), tables.n_tab, tables.n_adapters, tables.max_rank,
        _dev(row_adapter, torch.int32, "row_adapter") if row_adapter is not None else None,
        _dev(xa, torch.bfloat16, "xa"), _dev(workspace, torch.uint8, "workspace") if workspace is not None else None,
        workspace.numel() if workspace is not None else 0, _stream(hs)))
    return out


def moe_silu_mul(gate: torch.Tensor, up: torch.Tensor, out: torch.Tensor,
                 routing: Optional[Routing] = None) -> torch.Tensor:
    """out[r] = bf16(silu(gate[r]) * up[r]) on the real sorted rows of ``routing`` (every row without)."""
    if gate.shape != up.shape or gate.shape != out.shape:
        raise ValueError("gate, up and out must have one shape")
    rows, n = gate.shape
    check(lib().moe_silu_mul(_dev(gate, torch.bfloat16, "gate"), _dev(up, torch.bfloat16, "up"),
                             _dev(out, torch.bfloat16, "out"),
                             _dev(routing.sorted_ids, torch.int32, "sorted_ids") if routing is not None else None,
                             routing.num_pairs if routing is not None else 0, rows, n, _stream(gate)))
    return out


def moe_lora_gather_fold(x: torch.Tensor, base: torch.Tensor, tables: LoraTables, indices: torch.Tensor,
                         top_k: int, x_gather: bool = False, row_map: Optional[torch.Tensor] = None,
                         row_adapter: Optional[torch.Tensor] = None,
                         xa: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Slot-major fold in place into ``base``: slot s = flat (token, slot) row of ``indices``."""
    n_slots = indices.numel()
    if xa is None:
        xa = torch.empty((max(n_slots, 1), tables.max_rank), dtype=torch.bfloat16, device=x.device)
    if xa.shape[0] < n_slots or xa.shape[1] != tables.max_rank:
        raise ValueError(f"xa must be [>= {n_slots}, {tables.max_rank}] (got {tuple(xa.shape)})")
    if x.shape[1] != tables.k_in or base.shape[1] != tables.n_out:
        raise ValueError("x / base widths do not match the LoRA tables")
    _numel_at_least(row_map, n_slots, "moe_lora_gather_fold: row_map")
    _numel_at_least(row_adapter, n_slots // max(top_k, 1), "moe_lora_gather_fold: row_adapter")
    check(lib().moe_lora_gather_fold(
        _dev(x, torch.bfloat16, "x"), x.shape[0], _dev(base, torch.bfloat16, "base"), base.shape[0],
        _dev(indices, torch.int32, "indices"), n_slots, top_k, int(bool(x_gather)),
        _dev(row_map, torch.int32, "row_map") if row_map is not None else None,
        _dev(row_adapter, torch.int32, "row_adapter") if row_adapter is not None else None,
        _dev(tables.a_table, torch.int64, "a_table"), _dev(tables.b_table, torch.int64, "b_table"),
        _dev(tables.scale_table, torch.float32, "scale_table"), tables.n_tab, tables.n_adapters, tables.k_in,
        tables.n_out, tables.max_rank, _dev(xa, torch.bfloat16, "xa"), _stream(x)))
    return base


# ----------------------------------------------------------------------------- A6 combine
def moe_combine(ys: torch.Tensor, inv_sorted: Optional[torch.Tensor], topk_w: torch.Tensor,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    T, k = topk_w.shape
    H = ys.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=ys.device)
    _need(out.dim() == 2 and tuple(out.shape) == (T, H), f"moe_combine: out is {tuple(out.shape)}; needs {(T, H)}")
    _numel_at_least(inv_sorted, T * k, "moe_combine: inv_sorted")
    check(lib().moe_combine(_dev(ys, torch.bfloat16, "ys"),
                            _dev(inv_sorted, torch.int32, "inv_sorted") if inv_sorted is not None else None,
                            _dev(topk_w, torch.float32, "topk_w"), _dev(out, torch.bfloat16, "out"), T, k, H,
                            ys.shape[0], _stream(ys)))
    return out
