"""Why the fold's GPU bar is "within 3 bf16 ulps of the largest term" and not "within 1 ulp of the
result", shown on the CPU with restated fp32 summation orders.

The fold rounds its shrink and its expand to bf16 (atlas moe_lora_grouped.rs module doc).  An fp32
sum in any order lands within an ulp or so of the exact sum before each rounding, so an xa or delta
value next to a bf16 rounding boundary can round the other way; the final base + scale * delta rounds
once more.  A delta one bf16 ulp off moves scale * delta by under 2 ulps of itself; where base and
scale * delta nearly cancel, that is many ulps of the small result.  Two checks:

* the order of gather_shrink_kernel / gather_expand_kernel (lora_fold.hip), restated here, meets the
  bar on the rank-128 GPU case (on that case it is in fact exact);
* a plain sequential fp32 order on another draw stays within 2 ulps of the largest term while
  missing the result by tens of ulps: a bar on the result alone would reject a correct fold.

CPU only."""
import numpy as np

import oracle
from moe_synth import f32_to_bf16_bits


def _f32(v):
    return np.asarray(v, dtype=np.float64).astype(np.float32)


def _fma(a, b, c):
    """fp32 fma of bf16 operands: the product is exact in fp64, the sum rounded once to fp32 (exact
    in fp64 except where the addends are more than 29 binades apart, below fp32's rounding point)."""
    return _f32(a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64))


def _dot8(a, b, acc):
    for i in range(8):
        acc = _fma(a[..., i], b[..., i], acc)
    return acc


def _butterfly(lanes, offsets):
    """shfl_xor reduction over the lane axis (axis 0): every lane ends with the same sum."""
    idx = np.arange(lanes.shape[0])
    for o in offsets:
        lanes = _f32(lanes.astype(np.float64) + lanes[idx ^ o].astype(np.float64))
    return lanes[0]


def emulate_gather_shrink(xr, A):
    """xa[slot, j] as gather_shrink_kernel sums it: wave w of 4 takes the 128-wide k chunks starting
    at w*128 + 512*m (m ascending); lane c of 16 takes 8 consecutive k of each chunk as an fma chain;
    the 16 lanes reduce by shfl_xor 8, 4, 2, 1; the four waves' sums add as (w0 + w1) + (w2 + w3).
    xr: [S, k_in], A: [S, R, k_in] fp32 (bf16 values)."""
    S, R, k_in = A.shape
    waves = []
    for w in range(4):
        lanes = np.zeros((16, S, R), np.float32)
        for c in range(16):
            acc = np.zeros((S, R), np.float32)
            m = 0
            while w * 128 + 512 * m < k_in:
                k = w * 128 + 512 * m + c * 8
                if k < k_in:
                    acc = _dot8(xr[:, None, k:k + 8], A[:, :, k:k + 8], acc)
                m += 1
            lanes[c] = acc
        waves.append(_butterfly(lanes, (8, 4, 2, 1)))
    s01 = _f32(waves[0].astype(np.float64) + waves[1])
    s23 = _f32(waves[2].astype(np.float64) + waves[3])
    return _f32(oracle.round_bf16(_f32(s01.astype(np.float64) + s23)))


def emulate_gather_expand(xa, B, scale, base):
    """base + scale * delta as gather_expand_kernel computes it: lane c of 8 sums ranks c*8 .. c*8+7
    and then c*8+64 .. c*8+71 (fma chains), the 8 lanes reduce by shfl_xor 4, 2, 1, delta is rounded
    to bf16 and folded with one fp32 fma, then rounded to bf16.  xa: [S, R], B: [S, n_out, R]."""
    S, n_out, R = B.shape
    lanes = np.zeros((8, S, n_out), np.float32)
    for c in range(8):
        acc = np.zeros((S, n_out), np.float32)
        for i in range(2):
            r0 = c * 8 + 64 * i
            if r0 < R:
                acc = _dot8(xa[:, None, r0:r0 + 8], B[:, :, r0:r0 + 8], acc)
        lanes[c] = acc
    delta = oracle.round_bf16(_butterfly(lanes, (4, 2, 1)))
    return oracle.round_bf16(_f32(np.float64(1.0) * scale[:, None] * delta + base.astype(np.float64)))


def _case(seed, T=33, k=4, E=12, k_in=640, n_out=136, R=128):
    """Router ids, even experts adapted, bf16 tables, x and base, as the rank-128 GPU case draws them."""
    rng = np.random.default_rng(seed)
    ids, _ = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    ids = ids.reshape(-1)
    adapted = list(range(0, E, 2))
    A_l, B_l, s_l = [], [], []
    for _ in adapted:
        A_l.append(f32_to_bf16_bits((rng.standard_normal((R, k_in)) * 0.01).astype(np.float32)))
        B_l.append(f32_to_bf16_bits((rng.standard_normal((n_out, R)) * 0.01).astype(np.float32)))
        s_l.append(float(np.float32(rng.uniform(0.5, 2.0))))
    x = f32_to_bf16_bits(rng.standard_normal((T * k, k_in)).astype(np.float32))
    base = f32_to_bf16_bits((rng.standard_normal((T * k, n_out)) * 0.05).astype(np.float32))
    tabs = oracle.pack_expert_tables(list(zip(adapted, A_l, B_l, s_l)))
    ref = oracle.lora_gather_fold(oracle.bf16_bits_to_f64(base), oracle.bf16_bits_to_f64(x), tabs, ids, k)
    sd = oracle.lora_gather_fold(np.zeros(base.shape), oracle.bf16_bits_to_f64(x), tabs, ids, k)
    slots = np.array([s for s, e in enumerate(ids) if e % 2 == 0], dtype=np.int64)
    f = lambda b: oracle.bf16_bits_to_f64(b).astype(np.float32)
    A = np.stack([f(A_l[adapted.index(ids[s])]) for s in slots])
    B = np.stack([f(B_l[adapted.index(ids[s])]) for s in slots])
    sc = np.array([s_l[adapted.index(ids[s])] for s in slots], np.float32)
    return f(x[slots]), A, B, sc, f(base[slots]), ref[slots], sd[slots]


def _errors(emu, base, ref, sd):
    """(share bit-exact, max |diff| in ulps of the largest of |base|, |result|, |scale*delta|,
    max |diff| in ulps of the result)."""
    g = emu.astype(np.float64)
    M = np.maximum(np.maximum(np.abs(base), np.abs(ref)), np.abs(sd))
    _, ex = np.frexp(M)
    of_largest = np.abs(g - ref) / np.ldexp(1.0, np.maximum(ex - 8, -133))
    _, exr = np.frexp(np.abs(ref))
    of_result = np.abs(g - ref) / np.ldexp(1.0, np.maximum(exr - 8, -133))
    return (g == ref).mean(), of_largest.max(), of_result.max()


def _sequential_shrink(xr, A):
    S, R, k_in = A.shape
    acc = np.zeros((S, R), np.float32)
    for k0 in range(0, k_in, 8):
        acc = _dot8(xr[:, None, k0:k0 + 8], A[:, :, k0:k0 + 8], acc)
    return _f32(oracle.round_bf16(acc))


def _sequential_expand(xa, B, scale, base):
    S, n_out, R = B.shape
    acc = np.zeros((S, n_out), np.float32)
    for r0 in range(0, R, 8):
        acc = _dot8(xa[:, None, r0:r0 + 8], B[:, :, r0:r0 + 8], acc)
    return oracle.round_bf16(_f32(np.float64(1.0) * scale[:, None] * oracle.round_bf16(acc) + base.astype(np.float64)))


def test_kernel_order_meets_the_bar_on_the_rank128_case():
    xr, A, B, sc, base, ref, sd = _case(31 + len("r128_k4"))
    emu = emulate_gather_expand(emulate_gather_shrink(xr, A), B, sc, base)
    exact, of_largest, of_result = _errors(emu, base, ref, sd)
    print(f"kernel order: exact {exact:.5f}, {of_largest:.2f} ulps of the largest term, {of_result:.2f} of the result")
    assert exact >= 0.999 and of_largest <= 3.0


def test_another_fp32_order_needs_the_largest_term_bar():
    xr, A, B, sc, base, ref, sd = _case(1)
    emu = _sequential_expand(_sequential_shrink(xr, A), B, sc, base)
    exact, of_largest, of_result = _errors(emu, base, ref, sd)
    print(f"sequential order: exact {exact:.5f}, {of_largest:.2f} ulps of the largest term, "
          f"{of_result:.2f} of the result")
    assert exact >= 0.99 and of_largest <= 3.0
    assert of_result > 3.0    # a near-cancelled result: a bar on the result alone would fail here
