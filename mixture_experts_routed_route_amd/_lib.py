"""ctypes view of the C ABI in ``include/moe_mi355x.h`` and ``include/moe_probes.h``
(``_lib/libmoe_mi355x.so``).

No fallback: if the library is missing, loading raises and nothing runs.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_uint64, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libmoe_mi355x.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_ELAUNCH = 0, -1, -2, -3
MOE_W_BF16, MOE_W_INT4_GPTQ, MOE_W_FP8 = 0, 1, 2
MOE_OP_GATE_UP_SILU, MOE_OP_DOWN, MOE_OP_GATHER = 0, 1, 2

# every symbol the header declares: name -> (restype, argtypes)
SIGNATURES = {
    "moe_last_error": (c_char_p, []),
    "moe_abi_version": (c_int32, []),
    "moe_align_max_padded": (c_int64, [c_int64, c_int32, c_int32]),
    "moe_align_workspace_bytes": (c_int64, [c_int64, c_int32]),
    "moe_check_group_arrays": (c_int32, [c_int32, POINTER(c_int64), POINTER(c_char_p), c_int32,
                                         POINTER(c_int32), c_int64]),
    "moe_lora_pack_tables": (c_int32, [POINTER(c_int32), POINTER(c_uint64), POINTER(c_uint64), POINTER(c_float),
                                       c_int32, POINTER(c_uint64), POINTER(c_uint64), POINTER(c_float), c_int32,
                                       POINTER(c_int32)]),
    "moe_lora_window_tiles": (c_int64, [c_int64, c_int64]),
    "moe_lora_windows": (c_int64, [c_int64, c_int64, POINTER(c_int64), POINTER(c_int64), c_int64]),
    "moe_route": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p]),
    "moe_align": (c_int32, [c_void_p, c_int64, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                            c_void_p, c_void_p, c_int64, c_void_p, c_int64, c_void_p]),
    "moe_align_noalloc": (c_int32, [c_void_p, c_int64, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_int64, c_void_p]),
    "moe_route_align": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_int32,
                                  c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_void_p,
                                  c_int64, c_void_p]),
    "moe_grouped_gemm": (c_int32, [c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_int64, c_int32, c_int32, c_int32, c_int32, c_int32, c_int64,
                                   c_void_p, c_int64, c_void_p]),
    "moe_grouped_gemm_workspace_bytes": (c_int64, []),
    "moe_lora_fold": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                c_int32, c_int32, c_void_p, c_int32, c_void_p, c_int64, c_int32, c_void_p, c_void_p,
                                c_int64, c_int64, c_int64, c_int64, c_int32, c_void_p]),
    "moe_grouped_gemm_gate_up_lora": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int64,
                                                c_int32, c_int32, c_int32, c_int32, c_int32, c_int64, c_void_p,
                                                c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_int32,
                                                c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_int64, c_void_p]),
    "moe_grouped_gemm_down_lora": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int32,
                                             c_int32, c_int32, c_int32, c_int32, c_int64, c_void_p, c_void_p,
                                             c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                             c_int64, c_void_p]),
    "moe_quantize_fp8": (c_int32, [c_void_p, c_int64, c_int32, c_void_p, c_int64, c_void_p, c_void_p, c_void_p]),
    "moe_grouped_gemm_fp8": (c_int32, [c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_int64, c_int32, c_int32, c_int32, c_int32, c_int32, c_int64,
                                       c_void_p, c_int64, c_void_p]),
    "moe_silu_mul": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_int32, c_void_p]),
    "moe_lora_gather_fold": (c_int32, [c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64, c_int32, c_int32,
                                       c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                       c_int32, c_int32, c_void_p, c_void_p]),
    "moe_combine": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int64,
                              c_void_p]),
    # include/moe_probes.h: ceiling probes, not steps of the path
    "moe_probe_stream_read": (c_int32, [c_void_p, c_int64, c_void_p, c_int32, c_void_p]),
    "moe_probe_mfma_bf16": (c_int32, [c_int64, c_void_p, c_int32, c_void_p]),
}


class MoeWeight(ctypes.Structure):
    """struct moe_weight of the header."""
    _fields_ = [("type", c_int32), ("group_size", c_int32), ("data", c_void_p), ("scales", c_void_p),
                ("qzeros", c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built ({LIB_PATH}); run "
                               "`python -m mixture_experts_routed_route_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[status {status}] {message}")
        self.status = status


def check(status: int) -> None:
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode())
