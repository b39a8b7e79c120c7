"""One routed MoE FFN layer on one GPU, chaining the C-ABI calls on the current stream:

    moe_route -> moe_align -> moe_grouped_gemm(gate/up + SiLU) -> moe_grouped_gemm(down)
              -> [LoRA fold] -> moe_combine

With LoRA tables for the gate and up projections, the gate/up step is instead

    moe_grouped_gemm(gather, gate) and (gather, up) -> a fold into each -> moe_silu_mul

because those folds update the gate and up outputs before SiLU, which the fused kernel
never writes.

A LoRA fold runs either over the sorted rows, window by window (``moe_lora_fold``), or
slot by slot through the inverse map (``moe_lora_gather_fold``).  The second has a grid of one
workgroup per (token, slot) pair instead of one per 16 sorted rows of the worst-case layout,
which is what decode batches want: there the sorted layout is mostly padding.  Over the sorted
rows with bf16 weights, the down-projection fold runs by default in the down GEMM's epilogue
(``moe_grouped_gemm_down_lora``), as the gate and up folds run in the gate/up GEMM's.

Buffers are allocated once per token count (``plan``) so a forward pass allocates
nothing and its launch grids depend on host scalars only.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np
import torch

from ._lib import MOE_OP_DOWN, MOE_OP_GATE_UP_SILU, MOE_OP_GATHER
from .ops import (Bf16Weight, Fp8Weight, GptqWeight, LoraTables, Routing, gemm_workspace, lora_windows,
                  moe_align, moe_combine, moe_grouped_gemm, moe_grouped_gemm_fp8, moe_lora_fold, moe_lora_gather_fold,
                  moe_quantize_fp8, moe_route, moe_route_align, moe_silu_mul, pack_lora_tables, stack_lora_tables,
                  moe_grouped_gemm_gate_up_lora, moe_grouped_gemm_down_lora)

FOLD_MODES = ("auto", "grouped", "gather")


@dataclass
class Buffers:
    T: int
    ids: torch.Tensor
    w: torch.Tensor
    routing: Routing
    hs: torch.Tensor
    ys: torch.Tensor
    out: torch.Tensor
    xa: Optional[torch.Tensor]    # flat bf16 shrink scratch shared by the folds
    ws: torch.Tensor
    g: Optional[torch.Tensor] = None   # gate and up outputs of the gate/up LoRA path
    u: Optional[torch.Tensor] = None
    xq: Optional[torch.Tensor] = None  # fp8 path: e4m3 codes and per-row scales of x and of Hs
    sx: Optional[torch.Tensor] = None
    hq: Optional[torch.Tensor] = None
    sh: Optional[torch.Tensor] = None


class MoeLayer:
    def __init__(self, num_experts: int, hidden: int, inter: int, top_k: int, block_size: int, gate, up, down,
                 lora: Optional[LoraTables] = None, renormalize: bool = True, lora_cap: Optional[int] = None,
                 fold: str = "auto", lora_gate: Optional[LoraTables] = None, lora_up: Optional[LoraTables] = None,
                 gate_up_fused: bool = True, down_fused: bool = True):
        if fold not in FOLD_MODES:
            raise ValueError(f"fold must be one of {FOLD_MODES}")
        if isinstance(gate, Fp8Weight) and (lora_gate is not None or lora_up is not None):
            raise ValueError("gate/up LoRA tables are not supported with fp8 weights")
        self.E, self.H, self.I, self.top_k, self.bs = num_experts, hidden, inter, top_k, block_size
        self.gate, self.up, self.down, self.lora = gate, up, down, lora
        self.lora_gate, self.lora_up = lora_gate, lora_up
        self.renormalize = renormalize
        self.lora_cap = lora_cap
        self.fold = fold
        # gate/up LoRA folded in the gate/up GEMM's epilogue (bf16 weights), else the page's order:
        # gathered gate and up, a fold into each, SiLU * up
        self.gate_up_fused = gate_up_fused and isinstance(gate, Bf16Weight)
        # down-projection LoRA folded in the down GEMM's epilogue where the fold runs over the sorted
        # rows (bf16 weights), else the shrink and expand kernels after the down GEMM
        self.down_fused = down_fused and isinstance(down, Bf16Weight)

    @property
    def fp8(self) -> bool:
        return isinstance(self.gate, Fp8Weight)

    @property
    def gate_up_lora(self) -> bool:
        return self.lora_gate is not None or self.lora_up is not None

    def _tables(self):
        return [t for t in (self.lora, self.lora_gate, self.lora_up) if t is not None]

    # ------------------------------------------------------------------ construction from host arrays
    @staticmethod
    def from_arrays(d: Dict[str, object], device, lora_cap: Optional[int] = None, fold: str = "auto",
                    gate_up_fused: bool = True, down_fused: bool = True) -> "MoeLayer":
        """Build from host numpy arrays (bf16 / fp16 as uint16 bit patterns, GPTQ words as int32)."""
        cfg = d["cfg"]
        bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to(device)
        if "wg" in d:
            gate, up, down = Bf16Weight(bf(d["wg"])), Bf16Weight(bf(d["wu"])), Bf16Weight(bf(d["wd"]))
        elif "fp8_gate" in d:
            def f8(w):
                return Fp8Weight(torch.from_numpy(w["codes"]).to(device), torch.from_numpy(w["scales"]).to(device))
            gate, up, down = f8(d["fp8_gate"]), f8(d["fp8_up"]), f8(d["fp8_down"])
        else:
            def gq(w):
                return GptqWeight(torch.from_numpy(w["qweight"]).to(device),
                                  torch.from_numpy(w["scales"]).view(torch.float16).to(device),
                                  torch.from_numpy(w["qzeros"]).to(device), int(w["group_size"]))
            gate, up, down = gq(d["gate"]), gq(d["up"]), gq(d["down"])

        def one(ad, prefix):
            if f"{prefix}_a" not in ad:
                return None
            n = len(ad["lora_ids"])
            return pack_lora_tables(list(ad["lora_ids"]), [bf(ad[f"{prefix}_a"][i]) for i in range(n)],
                                    [bf(ad[f"{prefix}_b"][i]) for i in range(n)], list(ad[f"{prefix}_scale"]),
                                    device)

        def tables(prefix):
            # one adapter's tables, or several adapters' stacked by adapter id (a mixed batch names
            # each token's adapter in its row_adapter map)
            if "lora_adapters" in d:
                per = [one(ad, prefix) for ad in d["lora_adapters"]]
                return stack_lora_tables(per, device) if any(t is not None for t in per) else None
            return one(d, prefix) if "lora_ids" in d else None
        lora = tables("lora")
        lora_gate = tables("lora_gate")
        lora_up = tables("lora_up")
        return MoeLayer(cfg.E, cfg.H, cfg.I, cfg.top_k, cfg.block_size, gate, up, down, lora, cfg.renormalize,
                        lora_cap, fold, lora_gate, lora_up, gate_up_fused, down_fused)

    # ------------------------------------------------------------------ buffers
    def plan(self, T: int, device) -> Buffers:
        P = T * self.top_k
        r = Routing.allocate(P, self.top_k, self.E, self.bs, device)
        bf = dict(dtype=torch.bfloat16, device=device)
        xa = None
        if self._tables():
            # rows: the window capacity of the grouped fold, and at least one per slot for the gather fold
            cap = max(self.lora_cap or r.max_pad, P)
            xa = torch.empty(cap * max(t.max_rank for t in self._tables()), **bf)
        b = Buffers(T, torch.empty((T, self.top_k), dtype=torch.int32, device=device),
                    torch.empty((T, self.top_k), dtype=torch.float32, device=device), r,
                    torch.empty((r.max_pad, self.I), **bf), torch.empty((r.max_pad, self.H), **bf),
                    torch.empty((T, self.H), **bf), xa, gemm_workspace(device))
        if self.gate_up_lora and self.gate_up_fused:
            rank = max(t.max_rank for t in (self.lora_gate, self.lora_up) if t is not None)
            b.g = torch.empty((2, r.max_pad, rank), **bf)  # the two shrinks of the fused path
        elif self.gate_up_lora:
            b.g = torch.empty((r.max_pad, self.I), **bf)
            b.u = torch.empty((r.max_pad, self.I), **bf)
        if self.fp8:
            u8, f32 = dict(dtype=torch.uint8, device=device), dict(dtype=torch.float32, device=device)
            b.xq, b.sx = torch.empty((T, self.H), **u8), torch.empty(max(T, 1), **f32)
            b.hq, b.sh = torch.empty((r.max_pad, self.I), **u8), torch.empty(r.max_pad, **f32)
        return b

    # ------------------------------------------------------------------ forward
    def route_align(self, logits: torch.Tensor, b: Buffers) -> None:
        moe_route_align(logits, self.top_k, self.renormalize, self.bs, b.ids, b.w, b.routing)

    def gate_up_stage(self, x: torch.Tensor, b: Buffers, row_adapter: Optional[torch.Tensor] = None) -> None:
        """Hs from x: the fused kernel, or gathered gate and up, their folds and SiLU * up; with fp8
        weights, x quantised per token and the fp8 fused kernel."""
        if self.fp8:
            moe_quantize_fp8(x, b.xq, b.sx)
            moe_grouped_gemm_fp8(MOE_OP_GATE_UP_SILU, b.xq, b.sx, self.gate, self.up, b.routing, out=b.hs,
                                 workspace=b.ws)
            return
        if not self.gate_up_lora:
            moe_grouped_gemm(MOE_OP_GATE_UP_SILU, x, self.gate, self.up, b.routing, out=b.hs, workspace=b.ws)
            return
        if self.gate_up_fused:
            moe_grouped_gemm_gate_up_lora(x, self.gate, self.up, b.routing, self.lora_gate, self.lora_up, b.g,
                                          out=b.hs, row_adapter=row_adapter, workspace=b.ws)
            return
        moe_grouped_gemm(MOE_OP_GATHER, x, self.gate, None, b.routing, out=b.g, workspace=b.ws)
        moe_grouped_gemm(MOE_OP_GATHER, x, self.up, None, b.routing, out=b.u, workspace=b.ws)
        if self.lora_gate is not None:
            self._fold(self.lora_gate, x, b.g, b, row_adapter, x_gather=True)
        if self.lora_up is not None:
            self._fold(self.lora_up, x, b.u, b, row_adapter, x_gather=True)
        moe_silu_mul(b.g, b.u, b.hs, b.routing)

    def down_stage(self, b: Buffers, row_adapter: Optional[torch.Tensor] = None) -> None:
        """Ys from Hs; with the fused down fold, the LoRA shrink and the down GEMM whose epilogue folds."""
        if self.fp8:  # the real rows of Hs quantised per row, then the fp8 down GEMM
            moe_quantize_fp8(b.hs, b.hq, b.sh, b.routing)
            moe_grouped_gemm_fp8(MOE_OP_DOWN, b.hq, b.sh, self.down, None, b.routing, out=b.ys, workspace=b.ws)
            return
        if self.down_fold_fused(b):
            R, mp = self.lora.max_rank, b.routing.max_pad
            moe_grouped_gemm_down_lora(b.hs, self.down, b.routing, self.lora, b.xa[: mp * R].view(mp, R), out=b.ys,
                                       row_adapter=row_adapter, workspace=b.ws)
            return
        moe_grouped_gemm(MOE_OP_DOWN, b.hs, self.down, None, b.routing, out=b.ys, workspace=b.ws)

    def down_fold_fused(self, b: Buffers) -> bool:
        """Whether the down-projection fold runs in the down GEMM's epilogue for these buffers: down
        tables, bf16 weights, the fold over the sorted rows, and a shrink scratch for every sorted row."""
        return (self.lora is not None and self.down_fused and self.fold_mode(b) == "grouped"
                and b.xa.numel() >= b.routing.max_pad * self.lora.max_rank)

    def experts(self, x: torch.Tensor, b: Buffers, row_adapter: Optional[torch.Tensor] = None) -> None:
        self.gate_up_stage(x, b, row_adapter)
        self.down_stage(b, row_adapter)
        self.lora_fold(b, row_adapter)

    def fold_mode(self, b: Buffers) -> str:
        """The fold used for these buffers: slot by slot when at most half of the sorted rows can be
        real (decode batches), else over the sorted rows."""
        if self.fold != "auto":
            return self.fold
        return "gather" if 2 * b.routing.num_pairs <= b.routing.max_pad else "grouped"

    def _fold(self, tables: LoraTables, x: torch.Tensor, base: torch.Tensor, b: Buffers,
              row_adapter: Optional[torch.Tensor], x_gather: bool) -> None:
        R = tables.max_rank
        if self.fold_mode(b) == "gather":
            P = b.routing.num_pairs
            xa = b.xa[: P * R].view(P, R)
            moe_lora_gather_fold(x, base, tables, b.ids, self.top_k, x_gather=x_gather,
                                 row_map=b.routing.inv_sorted, row_adapter=row_adapter, xa=xa)
            return
        cap = b.xa.numel() // R
        xa = b.xa[: cap * R].view(cap, R)
        for s, e in lora_windows(b.routing.max_pad, cap):
            moe_lora_fold(x, base, tables, b.routing, row_adapter, xa, s, e, x_gather=x_gather)

    def lora_fold(self, b: Buffers, row_adapter: Optional[torch.Tensor] = None) -> None:
        """The down-projection fold into Ys (none without down tables, or when the down GEMM folded)."""
        if self.lora is not None and not self.down_fold_fused(b):
            self._fold(self.lora, b.hs, b.ys, b, row_adapter, x_gather=False)

    def combine(self, b: Buffers) -> torch.Tensor:
        return moe_combine(b.ys, b.routing.inv_sorted, b.w, out=b.out)

    def forward(self, logits: torch.Tensor, x: torch.Tensor, b: Optional[Buffers] = None,
                row_adapter: Optional[torch.Tensor] = None) -> torch.Tensor:
        if b is None:
            b = self.plan(x.shape[0], x.device)
        self.route_align(logits, b)
        self.experts(x, b, row_adapter)
        return self.combine(b)
