"""Seeded synthetic inputs for the routed-MoE expert path.

This module only draws random tensors and lays them out in the storage formats
the path consumes (bf16 / fp16 bit patterns, packed GPTQ int4 words).  It holds
none of the method's arithmetic: routing, alignment, the expert FFN, the LoRA
fold and the combine live in ``oracle/`` (reference) and in the HIP library
(product), and both take their inputs from here.

Streams: ``SeedSequence(seed).spawn(6)`` gives one child per part, in the order

    logits -> x -> gate -> up -> down -> LoRA

and each part that is stored per expert spawns one grandchild per expert, so the
expert slabs are independent PCG64 streams that can be drawn in parallel threads
with the same result.  Within a stream the draws are taken in the order listed
below.

* router logits: fp32 N(0,1) (drawn in fp64, rounded once to fp32); the skewed
  workload adds a per-expert bias ``-beta * s * ln(rank_e)`` with
  ``rank = 1 + permutation(E)`` (Zipf exponent s = 1.2, beta = 1.05), which
  leaves roughly ten experts with no token at seed 0.
* activations x: N(0,1) drawn in fp32, rounded to bf16 (RNE).
* bf16 expert weights: N(0, 0.02) drawn in fp32, rounded to bf16.  Layout is
  ``[E, N, K]`` (K contiguous): gate/up ``[E, I, H]``, down ``[E, H, I]``.
* GPTQ int4 expert weights (per projection, K = contraction, N = outputs):
  nibbles q ~ U{0..15} drawn as ``[E, K, N]`` and packed eight consecutive K
  values per int32, lowest K in the lowest nibble -> ``qweight [E, K/8, N]``;
  scales ~ U(0.005, 0.02) drawn in fp32, rounded to fp16 -> ``[E, K/G, N]``;
  zero points z ~ U{0..15} drawn as ``[E, K/G, N]`` and packed eight
  consecutive N values per int32, lowest N in the lowest nibble ->
  ``qzeros [E, K/G, N/8]``.
* LoRA (down projection): even expert ids 0, 2, 4, ... are adapted.  For each
  adapted expert A_e ``[rank, I]`` then B_e ``[H, rank]`` ~ N(0, 0.01) in bf16
  (all A's are drawn before all B's), then scale_e ~ U(0.5, 2.0).  The real
  rank is zero-padded to ``max_rank``: A rows and B columns past ``rank`` are 0.
* Several adapters (``lora_adapters`` > 1, a mixed batch): adapter 0 is the
  one above; adapter j >= 1 adapts the experts e with (e + j) % 3 == 0, its
  tables drawn the same way, after everything above (so adapter 0 is the same
  with or without the others).  Then each token's adapter id is drawn
  uniformly from {-1 (base, no fold), 0, .., lora_adapters - 1}.  The adapters
  are ``d["lora_adapters"]`` (one dict per id) and the map ``d["row_adapter"]``.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import numpy as np

__all__ = ["MoeConfig", "CONFIGS", "make_inputs", "make_router_logits", "f32_to_bf16_bits", "bf16_bits_to_f32"]


@dataclass(frozen=True)
class MoeConfig:
    name: str
    T: int            # tokens
    H: int            # hidden size
    I: int            # expert intermediate size
    E: int            # experts
    top_k: int
    block_size: int
    weights: str = "bf16"          # "bf16" | "int4_gptq" | "fp8"
    group_size: int = 128          # GPTQ group size along K
    logits: str = "normal"         # "normal" | "zipf"
    zipf_s: float = 1.2
    zipf_beta: float = 1.05
    lora_rank: int = 0             # 0 = no LoRA fold
    lora_max_rank: int = 0
    lora_gate_up: bool = False     # also LoRA tables for the gate and up projections
    lora_adapters: int = 1         # adapters installed; > 1 draws a per-token adapter map
    renormalize: bool = True
    seed: int = 0

    @property
    def P(self) -> int:
        return self.T * self.top_k

    @property
    def max_pad(self) -> int:
        bs = self.block_size
        return -(-(self.P + self.E * (bs - 1)) // bs) * bs

    @property
    def max_blocks(self) -> int:
        return self.max_pad // self.block_size

    def with_(self, **kw) -> "MoeConfig":
        return replace(self, **kw)


CONFIGS: Dict[str, MoeConfig] = {
    "tiny": MoeConfig("tiny", T=64, H=256, I=128, E=8, top_k=2, block_size=16),
    "mixtral_prefill": MoeConfig("mixtral_prefill", T=4096, H=4096, I=14336, E=8, top_k=2,
                                 block_size=64),
    "finegrained_skewed": MoeConfig("finegrained_skewed", T=8192, H=2048, I=768, E=128,
                                    top_k=8, block_size=64, logits="zipf"),
    "decode_int4": MoeConfig("decode_int4", T=16, H=2048, I=1408, E=64, top_k=6,
                             block_size=16, weights="int4_gptq", group_size=128),
    "lora_prefill": MoeConfig("lora_prefill", T=2048, H=4096, I=1408, E=64, top_k=6,
                              block_size=64, lora_rank=16, lora_max_rank=64),
    "decode_lora": MoeConfig("decode_lora", T=16, H=2048, I=1408, E=64, top_k=6, block_size=16,
                             weights="int4_gptq", group_size=128, lora_rank=16, lora_max_rank=64),
    "fp8_prefill": MoeConfig("fp8_prefill", T=4096, H=4096, I=14336, E=8, top_k=2, block_size=64,
                             weights="fp8"),
    "lora_all_prefill": MoeConfig("lora_all_prefill", T=2048, H=4096, I=1408, E=64, top_k=6,
                                  block_size=64, lora_rank=16, lora_max_rank=64, lora_gate_up=True),
}


# --------------------------------------------------------------------------- storage formats
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    """N(0, std^2) drawn in fp32 from one stream and stored as bf16 bits."""
    v = rng.standard_normal(tuple(shape), dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return f32_to_bf16_bits(v)


def _rng(ss: np.random.SeedSequence) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(ss))


def _per_expert(ss: np.random.SeedSequence, E: int, fn, threads: int):
    """Run ``fn(rng_e, e)`` for every expert on its own stream, in a thread pool."""
    kids = ss.spawn(E)
    if threads <= 1 or E == 1:
        return [fn(_rng(kids[e]), e) for e in range(E)]
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(lambda e: fn(_rng(kids[e]), e), range(E)))


def _pack_nibbles(q: np.ndarray, axis: int) -> np.ndarray:
    """Pack 4-bit values 8-per-int32 along ``axis`` (lowest index -> lowest nibble)."""
    q = np.moveaxis(q.astype(np.uint32), axis, -1)
    n = q.shape[-1]
    assert n % 8 == 0
    q = q.reshape(q.shape[:-1] + (n // 8, 8))
    word = np.zeros(q.shape[:-1], dtype=np.uint32)
    for i in range(8):
        word |= q[..., i] << np.uint32(4 * i)
    return np.moveaxis(word.view(np.int32), -1, axis)


def _fp8(ss: np.random.SeedSequence, E: int, N: int, K: int, threads: int) -> Dict[str, np.ndarray]:
    """FP8 E4M3 expert weights: codes [E, N, K] (uint8) and one fp32 scale per output channel
    [E, N].  Codes are drawn directly: random sign, exponent field uniform in 4..10 (magnitudes
    1/8 .. 15), random 3-bit mantissa, so every code is finite; scales ~ U(0.002, 0.006)."""
    codes = np.empty((E, N, K), dtype=np.uint8)
    scales = np.empty((E, N), dtype=np.float32)

    def one(rng, e):
        sign = rng.integers(0, 2, size=(N, K), dtype=np.uint8) << 7
        expo = rng.integers(4, 11, size=(N, K), dtype=np.uint8) << 3
        mant = rng.integers(0, 8, size=(N, K), dtype=np.uint8)
        codes[e] = sign | expo | mant
        scales[e] = rng.uniform(0.002, 0.006, size=N).astype(np.float32)

    _per_expert(ss, E, one, threads)
    return {"codes": codes, "scales": scales}


def _gptq(ss: np.random.SeedSequence, E: int, K: int, N: int, G: int,
          threads: int) -> Dict[str, np.ndarray]:
    qweight = np.empty((E, K // 8, N), dtype=np.int32)
    scales = np.empty((E, K // G, N), dtype=np.uint16)
    qzeros = np.empty((E, K // G, N // 8), dtype=np.int32)

    def one(rng, e):
        q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
        qweight[e] = _pack_nibbles(q, axis=0)                                # [K/8, N]
        s = rng.uniform(0.005, 0.02, size=(K // G, N)).astype(np.float32)
        scales[e] = s.astype(np.float16).view(np.uint16)                     # [K/G, N]
        z = rng.integers(0, 16, size=(K // G, N), dtype=np.uint8)
        qzeros[e] = _pack_nibbles(z, axis=1)                                 # [K/G, N/8]

    _per_expert(ss, E, one, threads)
    return {"qweight": qweight, "scales": scales, "qzeros": qzeros, "group_size": G}


def make_logits(cfg: MoeConfig, rng: np.random.Generator) -> np.ndarray:
    z = rng.standard_normal((cfg.T, cfg.E))
    if cfg.logits == "zipf":  # permutation drawn after the logits, same stream
        rank = 1 + rng.permutation(cfg.E)
        bias = -cfg.zipf_beta * cfg.zipf_s * np.log(rank.astype(np.float64))
        z = z + bias[None, :]
    elif cfg.logits != "normal":
        raise ValueError(cfg.logits)
    return np.ascontiguousarray(z.astype(np.float32))


def make_router_logits(cfg: MoeConfig, seed: Optional[int] = None) -> np.ndarray:
    """Only the router logits of ``make_inputs`` (same stream, same values)."""
    ss = np.random.SeedSequence(cfg.seed if seed is None else seed).spawn(6)[0]
    return make_logits(cfg, _rng(ss))


def make_inputs(cfg: MoeConfig, seed: Optional[int] = None, threads: int = 8) -> Dict[str, object]:
    """Draw every input of one MoE layer call for ``cfg`` (host numpy arrays)."""
    ss_logits, ss_x, ss_gate, ss_up, ss_down, ss_lora = np.random.SeedSequence(
        cfg.seed if seed is None else seed).spawn(6)
    T, H, I, E = cfg.T, cfg.H, cfg.I, cfg.E
    d: Dict[str, object] = {"cfg": cfg}
    d["logits"] = make_logits(cfg, _rng(ss_logits))
    d["x"] = _normal_bf16(_rng(ss_x), (T, H), 1.0)
    if cfg.weights == "bf16":
        for key, ss, shape in (("wg", ss_gate, (I, H)), ("wu", ss_up, (I, H)), ("wd", ss_down, (H, I))):
            w = np.empty((E,) + shape, dtype=np.uint16)

            def one(rng, e, w=w, shape=shape):
                w[e] = _normal_bf16(rng, shape, 0.02)

            _per_expert(ss, E, one, threads)
            d[key] = w
    elif cfg.weights == "int4_gptq":
        G = cfg.group_size
        d["gate"] = _gptq(ss_gate, E, H, I, G, threads)
        d["up"] = _gptq(ss_up, E, H, I, G, threads)
        d["down"] = _gptq(ss_down, E, I, H, G, threads)
    elif cfg.weights == "fp8":
        d["fp8_gate"] = _fp8(ss_gate, E, I, H, threads)
        d["fp8_up"] = _fp8(ss_up, E, I, H, threads)
        d["fp8_down"] = _fp8(ss_down, E, H, I, threads)
    else:
        raise ValueError(cfg.weights)
    if cfg.lora_rank:
        rng = _rng(ss_lora)
        r, R = cfg.lora_rank, cfg.lora_max_rank
        ids = np.arange(0, E, 2, dtype=np.int32)
        n = len(ids)
        a_real = _normal_bf16(rng, (n, r, I), 0.01)
        b_real = _normal_bf16(rng, (n, H, r), 0.01)
        scale = rng.uniform(0.5, 2.0, size=n).astype(np.float32)
        a = np.zeros((n, R, I), dtype=np.uint16)
        a[:, :r, :] = a_real
        b = np.zeros((n, H, R), dtype=np.uint16)
        b[:, :, :r] = b_real
        d["lora_ids"] = ids
        d["lora_a"] = a
        d["lora_b"] = b
        d["lora_scale"] = scale
        if cfg.lora_gate_up:
            # drawn after the down tables, so those stay the same with or without these
            for proj in ("gate", "up"):
                ga = np.zeros((n, R, H), dtype=np.uint16)
                ga[:, :r, :] = _normal_bf16(rng, (n, r, H), 0.01)
                gb = np.zeros((n, I, R), dtype=np.uint16)
                gb[:, :, :r] = _normal_bf16(rng, (n, I, r), 0.01)
                d[f"lora_{proj}_a"] = ga
                d[f"lora_{proj}_b"] = gb
                d[f"lora_{proj}_scale"] = rng.uniform(0.5, 2.0, size=n).astype(np.float32)
        if cfg.lora_adapters > 1:
            keys = [k for k in d if k.startswith("lora_")]
            adapters = [{k: d[k] for k in keys}]
            for j in range(1, cfg.lora_adapters):
                ids_j = np.array([e for e in range(E) if (e + j) % 3 == 0], dtype=np.int32)
                nj = len(ids_j)
                ad = {"lora_ids": ids_j}
                projs = [("lora", I, H)] + ([("lora_gate", H, I), ("lora_up", H, I)] if cfg.lora_gate_up else [])
                for pre, k_in, n_out in projs:
                    aa = np.zeros((nj, R, k_in), dtype=np.uint16)
                    aa[:, :r, :] = _normal_bf16(rng, (nj, r, k_in), 0.01)
                    bb = np.zeros((nj, n_out, R), dtype=np.uint16)
                    bb[:, :, :r] = _normal_bf16(rng, (nj, n_out, r), 0.01)
                    ad[f"{pre}_a"], ad[f"{pre}_b"] = aa, bb
                    ad[f"{pre}_scale"] = rng.uniform(0.5, 2.0, size=nj).astype(np.float32)
                adapters.append(ad)
            d["lora_adapters"] = adapters
            d["row_adapter"] = rng.integers(-1, cfg.lora_adapters, size=T).astype(np.int32)
    return d
