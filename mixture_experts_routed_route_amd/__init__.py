"""Routed mixture-of-experts expert path for MI355X (gfx950): hand-written HIP kernels
behind the C ABI of ``include/moe_mi355x.h``, with a thin PyTorch binding.

    moe_route -> moe_align -> moe_grouped_gemm (gate/up + SiLU, down) -> moe_lora_fold -> moe_combine

With gate/up LoRA tables: moe_grouped_gemm (gathered gate, up) -> folds -> moe_silu_mul -> down ...
"""
from ._lib import (LIB_PATH, MOE_OP_DOWN, MOE_OP_GATE_UP_SILU, MOE_OP_GATHER, MOE_W_BF16, MOE_W_INT4_GPTQ,
                   MoeError, lib)
from .layer import Buffers, MoeLayer
from .ops import *  # noqa: F401,F403
