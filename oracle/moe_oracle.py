"""Plain fp64 CPU restatement of the routed-MoE expert path — test infrastructure only.

Sources (each function cites the page and the item on it that it follows):

* ferrum-kernels ``src/backend/cuda/moe.rs`` (docs.rs) — ``route_topk_softmax``,
  ``moe_build_pairs_by_token``, ``moe_align_block_size`` /
  ``moe_align_block_size_pair_ids``, ``moe_combine``, ``weighted_sum_batched``.
* ferrum-kernels ``src/backend/cuda/triton_fused_moe.rs`` (docs.rs) — module doc
  (one launch over all (token, expert) pairs, gather through sorted ids, masked
  sentinels), ``TritonStackedGptqWeight`` (stacked raw GPTQ layout),
  ``launch_fused_moe_w4a16_triton`` (sentinel = number of valid rows).
* metrale ``gpu_runtime/cutlass/grouped.rs`` — ``ensure_group_arrays`` and its
  tests; ``nvfp4_grouped_gate_up_fused`` (group row i reads token
  ``sorted_token_ids[i]``); ``nvfp4_grouped_down`` (A already in expert order).
* atlas ``spark_model/layers/ops/moe_lora_grouped.rs`` — module doc (fold math:
  shrink -> bf16 xa, expand -> bf16 delta, base += scale * fp32(delta)),
  ``MoeExpertRoute``, ``pack_expert_tables``, ``moe_lora_grouped_down``
  (windows, local-row scratch, ``moe_row_adapter``), ``grouped_down_wc``,
  ``grouped_down_windows``, ``MLG_M_TILE``, ``moe_lora_gather_bgmv`` (the
  router weight multiplies base + delta, i.e. fold before combine).

Arithmetic is fp64 on values widened exactly from their storage types (bf16,
fp16, fp32, int4).  Where the pages fix a precision the oracle follows it: the
router outputs fp32 weights, and the LoRA fold rounds its shrink and its expand
results to bf16.  Readings taken where the pages are silent are listed with
each function.  No blocking, fusion or reordering beyond the definitions: the
grouped GEMMs are one library matmul per expert over that expert's rows.
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "bf16_bits_to_f64", "f16_bits_to_f64", "round_bf16", "round_f32", "silu",
    "route", "max_padded", "align", "check_group_arrays",
    "gptq_unpack_q", "gptq_unpack_z", "gptq_dequant_expert",
    "out_dim", "expert_matrix", "grouped_gate_up", "grouped_gate_up_lora", "grouped_down",
    "pack_expert_tables", "adapter_tables", "token_adapter", "lora_windows", "lora_window_tiles", "lora_fold",
    "lora_gather_fold",
    "combine", "moe_layer", "moe_tokens",
    "e4m3_to_f64", "e4m3_round", "quantize_rows_fp8", "fp8_expert_matrix", "grouped_gate_up_fp8",
    "grouped_down_fp8",
]


# ----------------------------------------------------------------------------- number formats
def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> exact fp64 values (bf16 is the top half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits) -> np.ndarray:
    """IEEE binary16 bit patterns -> exact fp64 values."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def round_bf16(v) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value, ties to even; returned as fp64.

    bf16 keeps 8 significant bits and fp32's exponent range, so a value
    m * 2**e (0.5 <= |m| < 1) is rounded to a multiple of 2**(e-8), with the
    subnormal quantum 2**-133 as the floor; results of magnitude >= 2**128
    overflow to infinity.
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    q = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(v, -q)), q)
    big = np.abs(r) >= 2.0 ** 128
    if np.any(big):
        r = np.where(big, np.copysign(np.inf, v), r)
    return r


def round_f32(v) -> np.ndarray:
    """Round fp64 values to the nearest fp32 value (ties to even)."""
    return np.asarray(v, dtype=np.float64).astype(np.float32)


def silu(g: np.ndarray) -> np.ndarray:
    """SiLU(g) = g * sigmoid(g) = g / (1 + exp(-g))."""
    return g / (1.0 + np.exp(-g))


# ----------------------------------------------------------------------------- FP8 E4M3
# The fp8 prefill variant (atlas ``moe_lora_grouped.rs`` module doc: fp8, like bf16, is a grouped
# prefill path writing the same sorted BF16 ``expert_down_out``).  The page names no format or
# scaling; the reading taken: OCP FP8 E4M3 codes (1 sign, 4 exponent bits with bias 7, 3
# mantissa bits; no infinities; S.1111.111 is NaN), weights with one fp32 scale per output
# channel, activations quantised per row at run time with scale amax / 448.

def e4m3_to_f64(codes) -> np.ndarray:
    """FP8 E4M3 codes -> exact values (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m, -9), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def e4m3_round(v) -> np.ndarray:
    """Round values to the nearest E4M3 code, ties to an even mantissa; magnitudes that round
    above 448 give the NaN code (no saturation).  -0.0 keeps its sign."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    a = np.abs(v)
    _, ex = np.frexp(a)                    # a = f * 2**ex, 0.5 <= f < 1
    e = np.maximum(ex - 1, -6)             # unbiased exponent; below 2**-6 the subnormal quantum
    q = np.rint(np.ldexp(a, 3 - e))        # multiples of 2**(e-3); 8..16 for normals
    e = np.where(q >= 16, e + 1, e)
    q = np.where(q >= 16, q / 2, q)        # 16 * 2**(e-3) == 8 * 2**(e-2): carry into the exponent
    normal = q >= 8
    field = np.where(normal, e + 7, 0)
    mant = np.where(normal, q - 8, q).astype(np.int64)
    code = (field.astype(np.int64) << 3) | mant
    code = np.where((field > 15) | ((field == 15) & (mant == 7)), 0x7F, code)
    return (sign | code).astype(np.uint8)


def quantize_rows_fp8(x: np.ndarray):
    """Per-row dynamic FP8 quantisation of bf16 activations.  In fp32, as the GPU computes it:
    amax = max |x|; the dequantisation scale s = amax / 448 and the quantisation factor
    f = 448 / amax (both 1 for an all-zero row); codes = e4m3_round(x * f).  Every code is
    decided from the same fp32 product on both sides.  Returns (codes uint8, s fp32)."""
    xf = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(xf), axis=1) if xf.shape[1] else np.zeros(xf.shape[0], np.float32)
    pos = amax > 0
    safe = np.where(pos, amax, np.float32(1.0)).astype(np.float32)
    s = np.where(pos, safe / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    f = np.where(pos, np.float32(448.0) / safe, np.float32(1.0)).astype(np.float32)
    q = e4m3_round((xf * f[:, None]).astype(np.float32))
    return q, s


# ----------------------------------------------------------------------------- A1 route
def route(logits: np.ndarray, top_k: int, renormalize: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """Top-k softmax router: ferrum ``cuda/moe.rs``, ``route_topk_softmax``.

    Per row t of the fp32 ``logits [T, E]``: softmax over all E experts, keep
    the k most probable, and with ``norm_topk_prob`` divide the k kept
    probabilities by their sum.  Outputs are i32 ids and f32 weights ``[T, k]``
    (the types ``try_gpu_route_topk_into_host`` reads back).

    Readings (the page gives no kernel body):
      * selection order: descending logit, ties -> lower expert index (softmax
        is monotone, so this is the order of the probabilities; selection is a
        comparison of the fp32 logits, exact on every implementation);
      * probabilities: p_i = exp(l_i - max l) / sum_j exp(l_j - max l), in fp64;
      * renormalised weight w_j = p_{id_j} / sum_{j'} p_{id_j'} (sum in slot
        order), then rounded once to fp32.
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not 1 <= top_k <= E:
        raise ValueError("top_k must be in [1, E]")
    ids = np.empty((T, top_k), dtype=np.int32)
    w = np.empty((T, top_k), dtype=np.float32)
    idx = np.arange(E)
    for t in range(T):
        l = logits[t].astype(np.float64)
        order = np.lexsort((idx, -l))          # primary: -l ascending; secondary: index
        sel = order[:top_k]
        ex = np.exp(l - l.max())
        p = ex / ex.sum()
        ps = p[sel]
        if renormalize:
            kept = 0.0
            for j in range(top_k):         # the kept probabilities summed in slot order
                kept += ps[j]
            ws = ps / kept
        else:
            ws = ps
        ids[t] = sel
        w[t] = round_f32(ws)
    return ids, w


# ----------------------------------------------------------------------------- A2 align
def max_padded(num_pairs: int, num_experts: int, block_size: int) -> int:
    """Worst-case padded row count: every expert may add up to block_size-1 pad rows.

    ferrum ``cuda/moe.rs``, ``moe_align_block_size`` takes this capacity as
    ``sorted_max_size`` without giving a formula; the bound below is the
    smallest that holds for every routing.
    """
    bs = block_size
    return -(-(num_pairs + num_experts * (bs - 1)) // bs) * bs


def align(topk_ids: np.ndarray, num_experts: int, block_size: int,
          max_pad: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Block-size alignment of the flat (token, slot) pairs by expert.

    ferrum ``cuda/moe.rs``: ``moe_build_pairs_by_token`` (per-expert counts,
    ``expert_offsets``, pair -> packed row map) and ``moe_align_block_size`` /
    ``moe_align_block_size_pair_ids`` (block-padded ``sorted_token_ids``, one
    expert id per block, ``total_tokens_post_pad``).  Sentinel value = the
    number of valid rows (ferrum ``triton_fused_moe.rs``,
    ``launch_fused_moe_w4a16_triton``); inactive blocks hold a negative id
    (``maybe_dump_moe_routing`` counts ``expert_id >= 0``).

    Readings: sorted entries are flat pair ids p = t*top_k + j (the
    ``_pair_ids`` variant); rows of one expert are in ascending p; offsets are
    block padded (``offsets[E] == total``); unused blocks hold -1; an id outside
    [0, E) is dropped (not counted, ``inv = -1``).

    Returns counts [E], offsets [E+1], sorted_ids [max_pad], expert_ids
    [max_pad // bs], total (int), inv [P] — all int32 except total.
    """
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    P = ids.size
    E, bs = int(num_experts), int(block_size)
    if max_pad is None:
        max_pad = max_padded(P, E, bs)
    counts = [0] * E
    for p in range(P):
        e = ids[p]
        if 0 <= e < E:
            counts[e] += 1
    offsets = [0] * (E + 1)
    for e in range(E):
        padded = -(-counts[e] // bs) * bs
        offsets[e + 1] = offsets[e] + padded
    total = offsets[E]
    if total > max_pad:
        raise ValueError("max_pad too small")
    sorted_ids = [P] * max_pad
    expert_ids = [-1] * (max_pad // bs)
    inv = [-1] * P
    cursor = offsets[:E]
    cursor = list(cursor)
    for p in range(P):
        e = ids[p]
        if 0 <= e < E:
            sorted_ids[cursor[e]] = p
            inv[p] = cursor[e]
            cursor[e] += 1
    for e in range(E):
        for b in range(offsets[e] // bs, offsets[e + 1] // bs):
            expert_ids[b] = e
    i32 = lambda a: np.asarray(a, dtype=np.int32)
    return {"counts": i32(counts), "offsets": i32(offsets), "sorted_ids": i32(sorted_ids),
            "expert_ids": i32(expert_ids), "total": int(total), "inv": i32(inv),
            "num_pairs": P, "block_size": bs, "num_experts": E}


def check_group_arrays(num_experts: int, per_expert: Sequence[Tuple[str, int]],
                       offsets: Sequence[int]) -> Optional[str]:
    """Group-array invariants: metrale ``cutlass/grouped.rs``, ``ensure_group_arrays``.

    ``offsets`` has num_experts+1 entries, every per-expert array has
    num_experts entries (the message names the first that does not),
    offsets[0] >= 0 and offsets never decrease (equal neighbours = an empty
    expert).  Returns None when all hold, else the message.
    """
    if len(offsets) != num_experts + 1:
        return f"expert_offsets len {len(offsets)} != num_experts+1 {num_experts + 1}"
    for name, n in per_expert:
        if n != num_experts:
            return f"{name} len {n} != num_experts {num_experts}"
    if offsets[0] < 0:
        return f"expert_offsets[0] = {offsets[0]} is negative"
    for a, b in zip(offsets[:-1], offsets[1:]):
        if b < a:
            return f"expert_offsets is not non-decreasing ({a} then {b})"
    return None


# ----------------------------------------------------------------------------- GPTQ int4 weights
def gptq_unpack_q(qweight_e: np.ndarray) -> np.ndarray:
    """qweight ``[K/8, N]`` int32 -> q ``[K, N]``: K index 8*i + s sits in nibble s of word i.

    Layout from ferrum ``triton_fused_moe.rs`` (module doc,
    ``TritonStackedGptqWeight``); nibble order (low nibble = lowest K) is the
    reading taken for the raw GPTQ packing.
    """
    u = np.asarray(qweight_e).view(np.uint32)
    K8, N = u.shape
    q = np.empty((K8 * 8, N), dtype=np.int64)
    for s in range(8):
        q[s::8, :] = (u >> np.uint32(4 * s)) & np.uint32(0xF)
    return q


def gptq_unpack_z(qzeros_e: np.ndarray) -> np.ndarray:
    """qzeros ``[K/G, N/8]`` int32 -> z ``[K/G, N]``: N index 8*i + s sits in nibble s of word i."""
    u = np.asarray(qzeros_e).view(np.uint32)
    Gn, N8 = u.shape
    z = np.empty((Gn, N8 * 8), dtype=np.int64)
    for s in range(8):
        z[:, s::8] = (u >> np.uint32(4 * s)) & np.uint32(0xF)
    return z


def gptq_dequant_expert(w: Dict[str, np.ndarray], e: int) -> np.ndarray:
    """Dequantised weight of expert e as ``[K, N]`` fp64: W[k, n] = (q[k, n] - z[k//G, n]) * s[k//G, n].

    Stacked per-expert tensors as in ferrum ``triton_fused_moe.rs``
    (``TritonStackedGptqWeight``: qweight [E,K/8,N], scales [E,K/G,N] fp16,
    qzeros [E,K/G,N/8]).  Reading: the zero point is used as stored (no +1)
    and groups are contiguous runs of G along K (no act-order permutation).
    The product has at most 15 significant bits, so it is exact in fp64.
    """
    G = int(w["group_size"])
    q = gptq_unpack_q(w["qweight"][e])
    z = gptq_unpack_z(w["qzeros"][e])
    s = f16_bits_to_f64(w["scales"][e])
    g = np.arange(q.shape[0]) // G
    return (q - z[g, :]).astype(np.float64) * s[g, :]


def out_dim(w) -> int:
    """Output width N of a stacked expert weight in either storage format."""
    return int(w["qweight"].shape[2]) if isinstance(w, dict) else int(w.shape[1])


def expert_matrix(w, e: int) -> np.ndarray:
    """Weight of expert e as ``[N_out, K_in]`` fp64 for either storage format.

    bf16 weights are stored ``[E, N, K]`` (K contiguous, the nn.Linear
    convention); GPTQ weights are stored K-major and are transposed here.
    """
    if isinstance(w, dict):
        return gptq_dequant_expert(w, e).T
    return bf16_bits_to_f64(w[e])


# ----------------------------------------------------------------------------- A3 / A4 grouped GEMMs
def _rows_by_expert(al: Dict[str, np.ndarray], rows: Optional[np.ndarray] = None):
    """Real sorted rows grouped by the expert of their block: {e: rows}."""
    P, bs = al["num_pairs"], al["block_size"]
    sid, eid = al["sorted_ids"], al["expert_ids"]
    r_all = np.arange(int(al["total"])) if rows is None else np.asarray(rows)
    real = r_all[(sid[r_all] >= 0) & (sid[r_all] < P)]
    out: Dict[int, np.ndarray] = {}
    for r in real:
        e = int(eid[r // bs])
        if e >= 0:
            out.setdefault(e, []).append(int(r))
    return {e: np.asarray(v, dtype=np.int64) for e, v in out.items()}


def grouped_gate_up(x_bits: np.ndarray, w_gate, w_up, al: Dict[str, np.ndarray], top_k: int,
                    rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Grouped gate/up GEMM with SiLU(gate) * up, over block-aligned sorted rows.

    For every real sorted row r (sorted id p < P) with token t = p // top_k and
    expert e = expert_ids[r // block_size]:
    h[r] = silu(Wg[e] x[t]) * (Wu[e] x[t]).

    Gather through sorted ids: metrale ``cutlass/grouped.rs``,
    ``nvfp4_grouped_gate_up_fused``; ferrum ``triton_fused_moe.rs`` module doc
    (``expert_ids[pid_m]`` picks the block's expert, sentinel rows masked).
    SiLU(gate) * up: atlas ``moe_lora_grouped.rs`` (``moe_lora_gather_bgmv``:
    the post-SwiGLU activation).  Sentinel / padding rows are left NaN (they are
    never defined).  ``rows`` restricts the evaluation to a subset.
    """
    P = al["num_pairs"]
    sid = al["sorted_ids"]
    h = np.full((len(sid), out_dim(w_gate)), np.nan)
    for e, rr in _rows_by_expert(al, rows).items():
        t = sid[rr] // top_k
        X = bf16_bits_to_f64(x_bits[t])
        g = X @ expert_matrix(w_gate, e).T
        u = X @ expert_matrix(w_up, e).T
        h[rr] = silu(g) * u
    return h


def grouped_gate_up_lora(x_bits: np.ndarray, w_gate, w_up, al: Dict[str, np.ndarray], top_k: int,
                         tabs_gate, tabs_up, row_adapter: Optional[np.ndarray] = None) -> np.ndarray:
    """Gate/up with LoRA folded into each projection before SiLU: atlas ``moe_lora_grouped.rs``,
    ``moe_lora_grouped_down`` with ``x_gather`` = 1 (token-major input, base = the sorted BF16
    ``expert_gate_out`` / ``expert_up_out``), then ``moe_lora_gather_bgmv``'s ``moe_silu_mul``
    into a BF16 buffer.

    For every real sorted row: g = bf16(Wg[e] x[t]), u = bf16(Wu[e] x[t]); each is folded
    with its own tables (a projection without tables is left as it is; ``row_adapter`` picks the
    adapter of each token as in ``lora_fold``); h = bf16(silu(g) * u).
    Unlike the fused path, gate and up are rounded to bf16 before SiLU, as the page's path
    materialises them.  Sentinel rows are NaN.
    """
    sid = al["sorted_ids"]
    X = bf16_bits_to_f64(x_bits)
    g = np.full((len(sid), out_dim(w_gate)), np.nan)
    u = np.full_like(g, np.nan)
    for e, rr in _rows_by_expert(al).items():
        xt = X[sid[rr] // top_k]
        g[rr] = round_bf16(xt @ expert_matrix(w_gate, e).T)
        u[rr] = round_bf16(xt @ expert_matrix(w_up, e).T)
    if tabs_gate is not None:
        g = lora_fold(g, X, tabs_gate, al, top_k, row_adapter, x_gather=True)
    if tabs_up is not None:
        u = lora_fold(u, X, tabs_up, al, top_k, row_adapter, x_gather=True)
    return round_bf16(silu(g) * u)


def grouped_down(h: np.ndarray, w_down, al: Dict[str, np.ndarray],
                 rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Grouped down GEMM: y[r] = Wd[e] h[r] for every real sorted row r.

    The input is already in expert order (metrale ``cutlass/grouped.rs``,
    ``nvfp4_grouped_down``); the output is the sorted ``expert_down_out``
    (atlas ``moe_lora_grouped.rs`` module doc).  Sentinel rows stay NaN.
    """
    y = np.full((h.shape[0], out_dim(w_down)), np.nan)
    for e, rr in _rows_by_expert(al, rows).items():
        y[rr] = h[rr] @ expert_matrix(w_down, e).T
    return y


_E4M3_VALUES: Optional[np.ndarray] = None


def fp8_expert_matrix(w: Dict[str, np.ndarray], e: int) -> np.ndarray:
    """Dequantised [N, K] matrix of one FP8 expert: value(code) * scale of its output channel
    (the values of all 256 codes are decoded once and looked up)."""
    global _E4M3_VALUES
    if _E4M3_VALUES is None:
        _E4M3_VALUES = e4m3_to_f64(np.arange(256, dtype=np.uint8))
    return _E4M3_VALUES[w["codes"][e]] * w["scales"][e].astype(np.float64)[:, None]


def grouped_gate_up_fp8(xq: np.ndarray, sx: np.ndarray, w_gate, w_up, al: Dict[str, np.ndarray],
                        top_k: int, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """FP8 gate/up with SiLU * up over the sorted rows: for real row r (token t, expert e),
    g = s_x[t] * sum_k x(t, k) Wg(e, n, k) with x = e4m3 values of the quantised token row and W
    the dequantised weights; likewise u; h = silu(g) * u.  Sentinel rows are NaN.  ``rows``
    restricts the evaluation to a subset."""
    sid = al["sorted_ids"]
    h = np.full((len(sid), w_gate["codes"].shape[1]), np.nan)
    X = e4m3_to_f64(xq) * np.asarray(sx, np.float64)[:, None]
    for e, rr in _rows_by_expert(al, rows).items():
        xt = X[sid[rr] // top_k]
        h[rr] = silu(xt @ fp8_expert_matrix(w_gate, e).T) * (xt @ fp8_expert_matrix(w_up, e).T)
    return h


def grouped_down_fp8(hq: np.ndarray, sh: np.ndarray, w_down, al: Dict[str, np.ndarray],
                     rows: Optional[np.ndarray] = None) -> np.ndarray:
    """FP8 down over the sorted rows: y[r] = s_h[r] * (values of hq[r]) Wd(e)^T, dequantised.
    ``rows`` restricts the evaluation to a subset."""
    y = np.full((hq.shape[0], w_down["codes"].shape[1]), np.nan)
    H = e4m3_to_f64(hq) * np.asarray(sh, np.float64)[:, None]
    for e, rr in _rows_by_expert(al, rows).items():
        y[rr] = H[rr] @ fp8_expert_matrix(w_down, e).T
    return y


# ----------------------------------------------------------------------------- A5 LoRA fold
def pack_expert_tables(entries: Iterable[Tuple[int, object, object, float]]):
    """Dense per-expert tables: atlas ``moe_lora_grouped.rs``, ``pack_expert_tables``.

    ``entries`` = (expert_id, a, b, scale).  Table length n = max id + 1; slots
    of unadapted experts hold a null handle (None here, address 0 on the
    device) and scale 0.0; a repeated id keeps its last entry; no entries ->
    None.  Returns (a_list, b_list, scale_list, n).
    """
    entries = list(entries)
    if not entries:
        return None
    n = max(int(e) for e, *_ in entries) + 1
    a: List[object] = [None] * n
    b: List[object] = [None] * n
    s: List[float] = [0.0] * n
    for e, ea, eb, es in entries:
        a[int(e)], b[int(e)], s[int(e)] = ea, eb, float(es)
    return a, b, s, n


def adapter_tables(tables, a: int):
    """The per-expert tables adapter ``a`` folds with, or None.

    atlas ``moe_lora_grouped.rs``, ``MoeExpertRoute``: the per-expert tables are built at adapter
    install, and the adapter of a mixed batch's token comes from the per-row ``moe_row_adapter``
    (< 0 = base, no fold), not from the tables.  Reading: ``tables`` is either one adapter's
    (a, b, scale, n) tuple, which is adapter 0 (the page's single-adapter path with a null map), or
    a list of such tuples (or None) indexed by adapter id; any other id folds nothing.
    """
    if isinstance(tables, list):
        return tables[a] if 0 <= a < len(tables) else None
    return tables if a == 0 else None


def token_adapter(row_adapter: Optional[np.ndarray], t: int) -> int:
    """Adapter id of token t: row_adapter[t], or 0 without a map (the single-adapter path)."""
    return 0 if row_adapter is None else int(row_adapter[t])


def lora_window_tiles(row_offset: int, row_end: int, m_tile: int = 64) -> int:
    """Tiles of one window: max(1, ceil((row_end - row_offset) / 64)).

    atlas ``moe_lora_grouped.rs``, ``grouped_down_wc`` with ``MLG_M_TILE`` = 64
    (a window that is empty or inverted counts as zero rows).
    """
    n = max(0, row_end - row_offset)
    return max(1, -(-n // m_tile))


def lora_windows(total_rows: int, cap: int) -> List[Tuple[int, int]]:
    """Contiguous [start, end) windows of at most ``cap`` rows covering 0..total_rows.

    atlas ``moe_lora_grouped.rs``, ``grouped_down_windows`` (cap must be > 0).
    """
    if cap <= 0:
        raise ValueError("grouped LoRA scratch capacity must be nonzero")
    return [(s, min(s + cap, total_rows)) for s in range(0, total_rows, cap)]


def lora_fold(y: np.ndarray, x: np.ndarray, tables, al: Dict[str, np.ndarray], top_k: int,
              row_adapter: Optional[np.ndarray] = None, row_offset: int = 0,
              row_end: Optional[int] = None, bf16_base: bool = True, x_gather: bool = False) -> np.ndarray:
    """Down-projection LoRA fold over sorted rows: atlas ``moe_lora_grouped.rs``.

    For every sorted row r in the window [row_offset, row_end) that is real
    (sorted id < P), whose token t has adapter a = row_adapter[t] >= 0 (a = 0
    without a map), and whose expert e (the span [offsets[e], offsets[e+1])
    holding r) is adapted by that adapter (``adapter_tables(tables, a)`` exists,
    e < its length and its entry is non-null):

        xa    = bf16(A_e  x[r])      (shrink, [max_rank])
        delta = bf16(B_e  xa)        (expand, [n_out])
        y[r] += scale_e * delta

    ``x`` holds the bf16 post-SiLU sorted activations (module doc and
    ``moe_lora_grouped_down``: x = post-SiLU sorted activations, base =
    sorted ``expert_down_out``).  With ``x_gather`` (the same launcher's
    gate/up form) ``x`` is the token-major layer input and row r reads token
    sorted_ids[r] // top_k; the base is then a sorted gate or up output.  With ``bf16_base`` the base rows are bf16
    and the folded row is bf16(base + scale * delta); otherwise y is kept in
    fp64.  Rows outside the window, sentinel rows and unadapted rows are left
    as they are.  ``tables`` = (a_list, b_list, scale_list, n) from
    ``pack_expert_tables`` with A_e [max_rank, k_in] and B_e [n_out, max_rank]
    as bf16 bit arrays, or a list of those, one per adapter id.  Returns a new
    array.
    """
    P = al["num_pairs"]
    sid, off = al["sorted_ids"], al["offsets"]
    E = len(off) - 1
    y = np.array(y, dtype=np.float64, copy=True)
    mats: Dict[int, Tuple[np.ndarray, np.ndarray]] = {}
    if row_end is None:
        row_end = len(sid)
    for r in range(max(0, row_offset), min(row_end, len(sid))):
        p = int(sid[r])
        if p < 0 or p >= P:
            continue
        e = next((k for k in range(E) if off[k] <= r < off[k + 1]), None)
        a = token_adapter(row_adapter, p // top_k)
        tab = adapter_tables(tables, a) if a >= 0 else None
        if e is None or tab is None:
            continue
        a_tab, b_tab, s_tab, n_tab = tab
        if e >= n_tab or a_tab[e] is None or b_tab[e] is None:
            continue
        if (a, e) not in mats:
            mats[(a, e)] = (bf16_bits_to_f64(a_tab[e]), bf16_bits_to_f64(b_tab[e]))
        A, B = mats[(a, e)]
        xa = round_bf16(A @ x[p // top_k if x_gather else r])
        delta = round_bf16(B @ xa)
        if bf16_base:
            y[r] = round_bf16(y[r] + np.float64(np.float32(s_tab[e])) * delta)
        else:
            y[r] = y[r] + np.float64(np.float32(s_tab[e])) * delta
    return y


def lora_gather_fold(y: np.ndarray, x: np.ndarray, tables, indices: np.ndarray, top_k: int,
                     x_gather: bool = False, row_adapter: Optional[np.ndarray] = None,
                     row_map: Optional[np.ndarray] = None) -> np.ndarray:
    """Slot-major LoRA fold of decode: atlas ``moe_lora_grouped.rs``, ``moe_lora_gather_bgmv``.

    There is no sorting: flat (token, slot) row s < n_slots = len(indices)
    takes its expert from ``indices[s]`` and its adapter from
    ``row_adapter[s // top_k]`` (``gather_row_token``; < 0 skips, None is
    adapter 0 for every row; ``tables`` as in ``lora_fold``).  The x row is the slot itself for the down fold and the owning
    token s // top_k with ``x_gather`` (the gate/up fold over token-major x).
    The arithmetic is that of the grouped fold (module doc):

        xa    = bf16(A_e  x[x row])
        delta = bf16(B_e  xa)
        y[s]  = bf16(y[s] + scale_e * delta)

    Readings where the page is silent: an expert id outside [0, table length)
    or with a null table entry leaves the row as it is (as in the grouped
    fold).  ``row_map`` (not on the page) lets the same fold run on buffers in
    another row order: slot s then reads and writes row ``row_map[s]`` of y
    (and of x without ``x_gather``), and a negative entry skips the slot; None
    is the page's slot-major layout.  Returns a new array.
    """
    y = np.array(y, dtype=np.float64, copy=True)
    ids = np.asarray(indices).reshape(-1)
    for s in range(len(ids)):
        e = int(ids[s])
        a = token_adapter(row_adapter, s // top_k)
        tab = adapter_tables(tables, a) if a >= 0 else None
        if tab is None:
            continue
        a_tab, b_tab, s_tab, n_tab = tab
        if e < 0 or e >= n_tab or a_tab[e] is None or b_tab[e] is None:
            continue
        row = s if row_map is None else int(row_map[s])
        if row < 0:
            continue
        xrow = s // top_k if x_gather else row
        A, B = bf16_bits_to_f64(a_tab[e]), bf16_bits_to_f64(b_tab[e])
        xa = round_bf16(A @ x[xrow])
        delta = round_bf16(B @ xa)
        y[row] = round_bf16(y[row] + np.float64(np.float32(s_tab[e])) * delta)
    return y


# ----------------------------------------------------------------------------- A6 combine
def combine(y: np.ndarray, inv: Optional[np.ndarray], topk_w: np.ndarray, T: int,
            top_k: int) -> np.ndarray:
    """Top-k weighted combine: ferrum ``cuda/moe.rs``, ``moe_combine`` / ``weighted_sum_batched``.

    out[t] = sum_{j<k} w[t, j] * y[row(t, j)], j ascending, where row(t, j) =
    inv[t*k + j] (``moe_combine``'s pair -> packed-row map); a negative entry
    (a dropped pair) contributes nothing.  With ``inv`` None the rows are
    slot-major, row(t, j) = t*k + j (``weighted_sum_batched``).  fp64.
    """
    w = np.asarray(topk_w, dtype=np.float32).astype(np.float64).reshape(T, top_k)
    H = y.shape[1]
    out = np.zeros((T, H))
    for t in range(T):
        for j in range(top_k):
            row = t * top_k + j if inv is None else int(inv[t * top_k + j])
            if row < 0:
                continue
            out[t] += w[t, j] * y[row]
    return out


# ----------------------------------------------------------------------------- whole layer
def _adapter_dicts(d) -> List[Dict[str, object]]:
    """The installed adapters: ``d["lora_adapters"]`` (one dict per adapter id) when the inputs carry
    several, else the inputs themselves when they carry one adapter's tables, else none."""
    if "lora_adapters" in d:
        return list(d["lora_adapters"])
    return [d] if "lora_ids" in d else []


def _pack_one(ad, proj: str):
    pre = "lora" if proj == "down" else f"lora_{proj}"
    if f"{pre}_a" not in ad:
        return None
    return pack_expert_tables((int(e), ad[f"{pre}_a"][i], ad[f"{pre}_b"][i], float(ad[f"{pre}_scale"][i]))
                              for i, e in enumerate(ad["lora_ids"]))


def _lora_tables(d, proj: str = "down"):
    """Tables of one projection: one adapter's tuple, a list indexed by adapter id (several
    adapters), or None when no adapter has tables for it."""
    ads = _adapter_dicts(d)
    tabs = [_pack_one(ad, proj) for ad in ads]
    if all(t is None for t in tabs):
        return None
    return tabs if "lora_adapters" in d else tabs[0]


def _weights(d):
    if "wg" in d:
        return d["wg"], d["wu"], d["wd"]
    return d["gate"], d["up"], d["down"]


def moe_layer(d: Dict[str, object], max_pad: Optional[int] = None) -> Dict[str, object]:
    """The whole path on the sorted layout: route -> align -> gate/up -> down -> [fold] -> combine.

    The fold (when the inputs carry LoRA tables) runs before the combine, so
    the router weight multiplies base + delta (atlas ``moe_lora_grouped.rs``,
    ``moe_lora_gather_bgmv``), on the bf16 post-SiLU activations bf16(h).
    With gate/up tables the gate/up step is ``grouped_gate_up_lora``.
    Intermediates stay fp64 otherwise.
    """
    cfg = d["cfg"]
    ids, w = route(d["logits"], cfg.top_k, cfg.renormalize)
    al = align(ids, cfg.E, cfg.block_size, max_pad)
    if "fp8_gate" in d:
        return _moe_layer_fp8(d, ids, w, al)
    wg, wu, wd = _weights(d)
    ra = d.get("row_adapter")
    tg, tu = _lora_tables(d, "gate"), _lora_tables(d, "up")
    if tg is None and tu is None:
        h = grouped_gate_up(d["x"], wg, wu, al, cfg.top_k)
    else:
        h = grouped_gate_up_lora(d["x"], wg, wu, al, cfg.top_k, tg, tu, ra)
    y = grouped_down(h, wd, al)
    tabs = _lora_tables(d)
    if tabs is not None:
        y = lora_fold(y, round_bf16(np.nan_to_num(h)), tabs, al, cfg.top_k, ra, bf16_base=False)
    out = combine(y, al["inv"], w, cfg.T, cfg.top_k)
    return {"ids": ids, "w": w, "align": al, "h": h, "y": y, "out": out}


def _token_delta(tables, a: int, e: int, xin: np.ndarray) -> Optional[np.ndarray]:
    """scale * bf16(B bf16(A xin)) of adapter a's expert e for one activation row, or None when that
    adapter does not adapt e (or a < 0, the base)."""
    tab = adapter_tables(tables, a) if (tables is not None and a >= 0) else None
    if tab is None or e >= tab[3] or tab[0][e] is None or tab[1][e] is None:
        return None
    xa = round_bf16(xin @ bf16_bits_to_f64(tab[0][e]).T)
    return np.float64(np.float32(tab[2][e])) * round_bf16(xa @ bf16_bits_to_f64(tab[1][e]).T)


def _moe_tokens_fp8(d, tokens, ids, w) -> np.ndarray:
    """The fp8 layer output for selected tokens, per (token, expert) pair (pairs grouped by
    expert only so that each expert's matrices are dequantised once)."""
    cfg = d["cfg"]
    xq, sx = quantize_rows_fp8(bf16_bits_to_f64(d["x"][tokens]))
    X = e4m3_to_f64(xq) * sx.astype(np.float64)[:, None]
    tabs = _lora_tables(d)
    by_e: Dict[int, List[Tuple[int, int]]] = {}
    for i, t in enumerate(tokens):
        for j in range(cfg.top_k):
            by_e.setdefault(int(ids[t, j]), []).append((i, j))
    out = np.zeros((len(tokens), cfg.H))
    for e, lst in sorted(by_e.items()):
        Wg, Wu, Wd = (fp8_expert_matrix(d[k], e) for k in ("fp8_gate", "fp8_up", "fp8_down"))
        for i, j in lst:
            h = silu(Wg @ X[i]) * (Wu @ X[i])
            hs = round_bf16(h)
            hq, sh = quantize_rows_fp8(hs[None, :])
            y = Wd @ (e4m3_to_f64(hq[0]) * np.float64(sh[0]))
            dl = _token_delta(tabs, token_adapter(d.get("row_adapter"), tokens[i]), e, hs)
            if dl is not None:
                y = y + dl
            out[i] += np.float64(w[tokens[i], j]) * y
    return out


def _moe_layer_fp8(d, ids, w, al) -> Dict[str, object]:
    """FP8 prefill: x quantised per token; gate/up + SiLU * up; Hs rounded to bf16 (the buffer
    the GPU writes) and quantised per sorted row; down; the fold, if any, on bf16 Hs; combine."""
    cfg = d["cfg"]
    xq, sx = quantize_rows_fp8(bf16_bits_to_f64(d["x"]))
    h = grouped_gate_up_fp8(xq, sx, d["fp8_gate"], d["fp8_up"], al, cfg.top_k)
    hs = round_bf16(np.nan_to_num(h))
    hq, sh = quantize_rows_fp8(hs)
    y = grouped_down_fp8(hq, sh, d["fp8_down"], al)
    real = al["sorted_ids"] < cfg.P
    y[~real] = np.nan
    tabs = _lora_tables(d)
    if tabs is not None:
        y = lora_fold(y, hs, tabs, al, cfg.top_k, d.get("row_adapter"), bf16_base=False)
    out = combine(y, al["inv"], w, cfg.T, cfg.top_k)
    return {"ids": ids, "w": w, "align": al, "h": np.where(real[:, None], h, np.nan), "y": y, "out": out,
            "xq": xq, "sx": sx, "hq": hq, "sh": sh}


def moe_tokens(d: Dict[str, object], tokens: Sequence[int],
               routing: Optional[Tuple[np.ndarray, np.ndarray]] = None) -> np.ndarray:
    """The layer output for selected tokens straight from the per-token definition.

    out[t] = sum_j w[t, j] * FFN_{id[t, j]}(x[t]) with
    FFN_e(x) = Wd[e] (silu(Wg[e] x) * (Wu[e] x)) and, for adapted experts, the
    fold delta added to FFN_e(x) before weighting.  No sorting or padding:
    used on sampled tokens of full-size workloads.  Returns [len(tokens), H].
    """
    cfg = d["cfg"]
    ids, w = routing if routing is not None else route(d["logits"], cfg.top_k, cfg.renormalize)
    if "fp8_gate" in d:
        return _moe_tokens_fp8(d, list(tokens), ids, w)
    wg, wu, wd = _weights(d)
    tabs = _lora_tables(d)
    tabs_gu = (_lora_tables(d, "gate"), _lora_tables(d, "up"))
    tokens = list(tokens)
    ra = d.get("row_adapter")
    by_e: Dict[int, List[Tuple[int, int]]] = {}
    for i, t in enumerate(tokens):
        for j in range(cfg.top_k):
            by_e.setdefault(int(ids[t, j]), []).append((i, j))
    out = np.zeros((len(tokens), cfg.H))
    contrib = {}
    for e, lst in sorted(by_e.items()):
        X = bf16_bits_to_f64(d["x"][[tokens[i] for i, _ in lst]])
        adapters = [token_adapter(ra, tokens[i]) for i, _ in lst]
        if tabs_gu == (None, None):
            h = silu(X @ expert_matrix(wg, e).T) * (X @ expert_matrix(wu, e).T)
        else:
            gu = []
            for wm, tb in zip((wg, wu), tabs_gu):
                v = round_bf16(X @ expert_matrix(wm, e).T)
                for q, a in enumerate(adapters):
                    dl = _token_delta(tb, a, e, X[q])
                    if dl is not None:
                        v[q] = round_bf16(v[q] + dl)
                gu.append(v)
            h = round_bf16(silu(gu[0]) * gu[1])
        yy = h @ expert_matrix(wd, e).T
        for q, a in enumerate(adapters):
            dl = _token_delta(tabs, a, e, round_bf16(h[q]))
            if dl is not None:
                yy[q] = yy[q] + dl
        for (i, j), row in zip(lst, yy):
            contrib[(i, j)] = row
    for i, t in enumerate(tokens):
        for j in range(cfg.top_k):
            out[i] += np.float64(w[t, j]) * contrib[(i, j)]
    return out
