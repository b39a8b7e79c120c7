"""One routed MoE FFN layer on one GPU, chaining the C-ABI calls on the current stream:

    moe_route -> moe_align -> moe_grouped_gemm(gate/up + SiLU) -> moe_grouped_gemm(down)
              -> [LoRA fold] -> moe_combine

The LoRA fold runs either over the sorted rows, window by window (``moe_lora_fold``), or
slot by slot through the inverse map (``moe_lora_gather_fold``).  The second has a grid of one
workgroup per (token, slot) pair instead of one per 16 sorted rows of the worst-case layout,
which is what decode batches want: there the sorted layout is mostly padding.

Buffers are allocated once per token count (``plan``) so a forward pass allocates
nothing and its launch grids depend on host scalars only.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np
import torch

from ._lib import MOE_OP_DOWN, MOE_OP_GATE_UP_SILU
from .ops import (Bf16Weight, GptqWeight, LoraTables, Routing, gemm_workspace, lora_windows, moe_align,
                  moe_combine, moe_grouped_gemm, moe_lora_fold, moe_lora_gather_fold, moe_route, moe_route_align,
                  pack_lora_tables)

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
    xa: Optional[torch.Tensor]
    ws: torch.Tensor


class MoeLayer:
    def __init__(self, num_experts: int, hidden: int, inter: int, top_k: int, block_size: int, gate, up, down,
                 lora: Optional[LoraTables] = None, renormalize: bool = True, lora_cap: Optional[int] = None,
                 fold: str = "auto"):
        if fold not in FOLD_MODES:
            raise ValueError(f"fold must be one of {FOLD_MODES}")
        self.E, self.H, self.I, self.top_k, self.bs = num_experts, hidden, inter, top_k, block_size
        self.gate, self.up, self.down, self.lora = gate, up, down, lora
        self.renormalize = renormalize
        self.lora_cap = lora_cap
        self.fold = fold

    # ------------------------------------------------------------------ construction from host arrays
    @staticmethod
    def from_arrays(d: Dict[str, object], device, lora_cap: Optional[int] = None, fold: str = "auto") -> "MoeLayer":
        """Build from host numpy arrays (bf16 / fp16 as uint16 bit patterns, GPTQ words as int32)."""
        cfg = d["cfg"]
        bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to(device)
        if "wg" in d:
            gate, up, down = Bf16Weight(bf(d["wg"])), Bf16Weight(bf(d["wu"])), Bf16Weight(bf(d["wd"]))
        else:
            def gq(w):
                return GptqWeight(torch.from_numpy(w["qweight"]).to(device),
                                  torch.from_numpy(w["scales"]).view(torch.float16).to(device),
                                  torch.from_numpy(w["qzeros"]).to(device), int(w["group_size"]))
            gate, up, down = gq(d["gate"]), gq(d["up"]), gq(d["down"])
        lora = None
        if "lora_ids" in d:
            a = [bf(d["lora_a"][i]) for i in range(len(d["lora_ids"]))]
            b = [bf(d["lora_b"][i]) for i in range(len(d["lora_ids"]))]
            lora = pack_lora_tables(list(d["lora_ids"]), a, b, list(d["lora_scale"]), device)
        return MoeLayer(cfg.E, cfg.H, cfg.I, cfg.top_k, cfg.block_size, gate, up, down, lora, cfg.renormalize,
                        lora_cap, fold)

    # ------------------------------------------------------------------ buffers
    def plan(self, T: int, device) -> Buffers:
        P = T * self.top_k
        r = Routing.allocate(P, self.top_k, self.E, self.bs, device)
        bf = dict(dtype=torch.bfloat16, device=device)
        xa = None
        if self.lora is not None:
            # rows: the window capacity of the grouped fold, and at least one per slot for the gather fold
            cap = max(self.lora_cap or r.max_pad, P)
            xa = torch.empty((cap, self.lora.max_rank), **bf)
        return Buffers(T, torch.empty((T, self.top_k), dtype=torch.int32, device=device),
                       torch.empty((T, self.top_k), dtype=torch.float32, device=device), r,
                       torch.empty((r.max_pad, self.I), **bf), torch.empty((r.max_pad, self.H), **bf),
                       torch.empty((T, self.H), **bf), xa, gemm_workspace(device))

    # ------------------------------------------------------------------ forward
    def route_align(self, logits: torch.Tensor, b: Buffers) -> None:
        moe_route_align(logits, self.top_k, self.renormalize, self.bs, b.ids, b.w, b.routing)

    def experts(self, x: torch.Tensor, b: Buffers, row_adapter: Optional[torch.Tensor] = None) -> None:
        moe_grouped_gemm(MOE_OP_GATE_UP_SILU, x, self.gate, self.up, b.routing, out=b.hs, workspace=b.ws)
        moe_grouped_gemm(MOE_OP_DOWN, b.hs, self.down, None, b.routing, out=b.ys, workspace=b.ws)
        self.lora_fold(b, row_adapter)

    def fold_mode(self, b: Buffers) -> str:
        """The fold used for these buffers: slot by slot when at most half of the sorted rows can be
        real (decode batches), else over the sorted rows."""
        if self.fold != "auto":
            return self.fold
        return "gather" if 2 * b.routing.num_pairs <= b.routing.max_pad else "grouped"

    def lora_fold(self, b: Buffers, row_adapter: Optional[torch.Tensor] = None) -> None:
        if self.lora is None:
            return
        if self.fold_mode(b) == "gather":
            moe_lora_gather_fold(b.hs, b.ys, self.lora, b.ids, self.top_k, row_map=b.routing.inv_sorted,
                                 row_adapter=row_adapter, xa=b.xa)
            return
        for s, e in lora_windows(b.routing.max_pad, b.xa.shape[0]):
            moe_lora_fold(b.hs, b.ys, self.lora, b.routing, row_adapter, b.xa, s, e)

    def combine(self, b: Buffers) -> torch.Tensor:
        return moe_combine(b.ys, b.routing.inv_sorted, b.w, out=b.out)

    def forward(self, logits: torch.Tensor, x: torch.Tensor, b: Optional[Buffers] = None,
                row_adapter: Optional[torch.Tensor] = None) -> torch.Tensor:
        if b is None:
            b = self.plan(x.shape[0], x.device)
        self.route_align(logits, b)
        self.experts(x, b, row_adapter)
        return self.combine(b)
