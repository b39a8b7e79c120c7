"""CPU models of the addressing of every kernel that computes addresses from device-resident ids
(besides the bf16 GEMM, modelled in test_gemm_addressing): the int4 GEMM, the fp8 form of the bf16
GEMM (byte addressing and scales; its schedule is the bf16 one), the LoRA epilogue of the bf16 GEMM (gate/up and down), the grouped fold's shrink and expand,
and the gather fold.  Each model restates the kernel's integer arithmetic and yields every
(buffer, index, extent) a launch can address; the tests show all of them in bounds on the routings of
the workloads and on tight routings whose padded total reaches the sorted capacity.  CPU only."""
import numpy as np
import pytest

import oracle
from moe_synth import CONFIGS, make_router_logits


def _spans(al, E, max_pad):
    off = al["offsets"]
    lo = [min(max(int(off[e]), 0), max_pad) for e in range(E)]
    hi = [min(max(int(off[e + 1]), lo[e]), max_pad) for e in range(E)]
    return lo, hi


# ----------------------------------------------------------------------------- int4 GEMM
def int4_touched(al, P, top_k, E, N, K, G, bs, gate_up, a_tok=False):
    """gemm_int4_kernel: grid (max_pad/16, N/64); workgroup = 16 sorted rows x 64 columns; the
    tile's expert from expert_ids[r0 / bs]; wave (proj, part) streams its K groups; lane
    (m = lane % 16, kq = lane / 16) loads qweight rows g*G/8 + kq + 4*st at columns ncol..ncol+3."""
    max_pad = len(al["sorted_ids"])
    sid, eid = al["sorted_ids"], al["expert_ids"]
    T = P // top_k
    STEPS = G // 32
    nsplit = 2 if gate_up else 4
    ngroups = K // G
    per = -(-ngroups // nsplit)
    for bx in range(max_pad // 16):
        r0 = bx * 16
        yield "expert_ids", r0 // bs, len(eid)
        e = int(eid[r0 // bs])
        for m in range(16):
            yield "sorted_ids", min(r0 + m, max_pad - 1), max_pad
        if e < 0 or e >= E:
            continue
        srcs = []
        for m in range(16):
            p = int(sid[min(r0 + m, max_pad - 1)]) if r0 + m < max_pad else -1
            srcs.append((p // top_k if (gate_up or a_tok) else r0 + m) if 0 <= p < P else -1)
        for by in range(N // 64):
            n0 = by * 64
            for wave in range(4):
                part = wave & 1 if gate_up else wave
                g_begin, g_end = part * per, min(ngroups, part * per + per)
                g0 = min(g_begin, ngroups - 1)
                groups = range(g0, g0 + max(1, g_end - g_begin))   # a wave without groups loads g0 once
                for lane in range(0, 64, 15):                         # lanes 0, 15, 30, 45, 60 cover m, kq ends
                    m, kq = lane & 15, lane >> 4
                    ncol = n0 + 4 * m
                    for g in groups:
                        for st in range(STEPS):
                            krow = g * (G // 8) + kq + 4 * st
                            yield "qweight", (e * (K // 8) + krow) * N + ncol + 3, E * (K // 8) * N
                        yield "scales", (e * (K // G) + g) * N + ncol + 3, E * (K // G) * N
                        yield "qzeros", (e * (K // G) + g) * (N // 8) + ncol // 8, E * (K // G) * (N // 8)
                        if any(s >= 0 for s in srcs):
                            src = srcs[m]
                            arow = src if src >= 0 else (0 if (gate_up or a_tok) else r0)
                            for st in range(STEPS):
                                yield "A", arow * K + g * G + st * 32 + kq * 8 + 7, (T if (gate_up or a_tok) else max_pad) * K
            for row in range(16):
                if srcs[row] >= 0:
                    yield "C", (r0 + row) * N + n0 + 63, max_pad * N


# ----------------------------------------------------------------------------- fp8 GEMM
def fp8_touched(al, P, top_k, E, N, K, BM, gate_up):
    """The fp8 form of gemm_bf16_kernel: the bf16 tiles in bytes (BM-row tiles of each expert span x
    a 256-row weight panel; the persistent schedule and split tail are the bf16 ones, modelled in
    test_gemm_addressing).  Per tile: the sorted ids, the rows' activation scales (s_as), the A rows
    (a row without a token reads token 0 or the tile's first sorted row), the panel's weight rows
    (clamped to N - 1), the channel scales of the wave columns (clamped to N - 1) and the stored C
    rows.  A and W are 1-byte codes, so the last byte of a row is at row * K + K - 1."""
    max_pad = len(al["sorted_ids"])
    sid = al["sorted_ids"]
    T_tok = P // top_k
    lo, hi = _spans(al, E, max_pad)
    BP = 256
    ncol = BP // 2 if gate_up else BP
    a_rows = T_tok if gate_up else max_pad
    for e in range(E):
        for t in range(-(-(hi[e] - lo[e]) // BM)):
            r0 = lo[e] + t * BM
            r_end = min(r0 + BM, hi[e])
            rows = []
            for i in range(BM):
                r = r0 + i
                src = -1
                if r < r_end:
                    yield "sorted_ids", r, max_pad
                    p = int(sid[r])
                    if 0 <= p < P:
                        src = p // top_k if gate_up else r
                        yield "a_scale", src, a_rows
                rows.append(src)
                srow = src if src >= 0 else (0 if gate_up else r0)
                yield "A", srow * K + K - 1, a_rows * K
            for n0 in range(0, -(-N // ncol) * ncol, ncol):
                for prow in range(BP):
                    n = min((n0 + (prow & (BP // 2 - 1))) if gate_up else (n0 + prow), N - 1)
                    yield "W", (e * N + n) * K + K - 1, E * N * K
                for wn in range(2):
                    for j in range(2 if gate_up else 4):
                        for fr in range(32):
                            cj = min(n0 + (wn * 64 if gate_up else wn * 128) + j * 32 + fr, N - 1)
                            yield "w_scale", e * N + cj, E * N
                for i in range(BM):
                    if rows[i] >= 0:
                        yield "C", (r0 + i) * N + min(n0 + ncol, N) - 1, max_pad * N


# ----------------------------------------------------------------------------- gate/up LoRA epilogue
def lora_epilogue_touched(al, P, top_k, E, N, BM, rank, n_tab, n_ad, ra, gate_up=True):
    """The LoRA epilogue of gemm_bf16_kernel (a 4 x 2 wave grid of 64 x 128 per wave in a 256-row
    tile, 2 x 2 in a 128-row tile; a 256-row weight panel): xa rows min(r0 + wm*WM + i*32 + fr,
    max_pad - 1) of [max_pad, rank], B_e rows of [N, rank] at min(n0 + wn*64 + jj*32 + fr, N - 1) for
    gate/up (128 output columns per panel, each projection's two blocks) or min(n0 + wn*128 + pj*64 +
    jj*32 + fr, N - 1) for down (256 output columns per panel, pass pj folding blocks 2 pj, 2 pj + 1),
    table entries a * n_tab + e for the adapters of the tile's rows, and row_adapter at each row's
    token."""
    max_pad = len(al["sorted_ids"])
    sid = al["sorted_ids"]
    lo, hi = _spans(al, E, max_pad)
    NW = 8 if BM == 256 else 4
    WM = BM // (NW // 2)
    for e in range(E):
        for t in range(-(-(hi[e] - lo[e]) // BM)):
            r0 = lo[e] + t * BM
            r_end = min(r0 + BM, hi[e])
            ads = set()
            for i in range(BM):
                r = r0 + i
                if r < r_end and 0 <= sid[r] < P:
                    tok = int(sid[r]) // top_k
                    yield "row_adapter", tok, P // top_k
                    a = int(ra[tok]) if ra is not None else 0
                    if 0 <= a < n_ad:
                        ads.add(a)
            ncol = 128 if gate_up else 256
            for n_t in range(-(-N // ncol)):
                n0 = n_t * ncol
                for wm in range(NW // 2):
                    for i in range(2):
                        for fr in (0, 31):
                            yield "xa", min(r0 + wm * WM + i * 32 + fr, max_pad - 1), max_pad
                for wn in range(2):
                    for pj in range(2):
                        for jj in range(2):
                            for fr in (0, 31):
                                col = n0 + (wn * 64 if gate_up else wn * 128 + pj * 64) + jj * 32 + fr
                                yield "B_e", min(col, N - 1) * rank + rank - 1, N * rank
                if e < n_tab:
                    for a in ads:
                        yield "table", a * n_tab + e, n_ad * n_tab


# ----------------------------------------------------------------------------- grouped fold
def grouped_fold_touched(al, P, top_k, E, k_in, n_out, max_rank, n_tab, n_ad, ra, row_offset, row_end, cap,
                         x_gather, x_rows):
    """lora_shrink_kernel and lora_expand_fold_kernel over the window's 64-row tiles from base16 =
    row_offset rounded down to 16 (every workgroup first stages the offsets and, when n_ad * n_tab <=
    4096, every adapter's table entries of the experts below n_tab, to take the tiles of adapted
    experts first; each tile is then cut into 16-row sub-tiles, the shrink taking a 32-row half per
    workgroup): only rows inside the window and the expert span are read through sorted_ids; folded
    rows read their x row, write and read xa at r - row_offset, read and write base; x row 0 and xa
    row 0 stand in for the rows of a sub-tile that are not folded; A_e rows < max_rank, B_e rows <
    n_out."""
    max_pad = len(al["sorted_ids"])
    sid, off = al["sorted_ids"], al["offsets"]
    yield "offsets", E, E + 1
    if n_ad * n_tab <= 4096:
        for a in range(n_ad):
            for e in range(min(n_tab, E)):
                yield "table", a * n_tab + e, n_ad * n_tab
    base16 = row_offset // 16 * 16
    for sub0 in range(base16, row_end, 16):
        if off[0] > sub0 or off[E] <= sub0:
            continue
        e = max(i for i in range(E) if off[i] <= sub0)
        if e >= n_tab:
            continue
        span_end = int(off[e + 1])
        yield "x", k_in - 1, x_rows * k_in              # row 0: the rows that are not folded
        yield "xa", max_rank - 1, cap * max_rank
        for m in range(16):
            r = sub0 + m
            if r < row_offset or r >= row_end or r >= span_end:
                continue
            yield "sorted_ids", r, max_pad
            p = int(sid[r])
            if not 0 <= p < P:
                continue
            yield "row_adapter", p // top_k, P // top_k
            a = int(ra[p // top_k]) if ra is not None else 0
            if not 0 <= a < n_ad:
                continue
            yield "table", a * n_tab + e, n_ad * n_tab
            xrow = p // top_k if x_gather else r
            yield "x", xrow * k_in + k_in - 1, x_rows * k_in
            yield "A_e", (max_rank - 1) * k_in + k_in - 1, max_rank * k_in
            yield "xa", (r - row_offset) * max_rank + max_rank - 1, cap * max_rank
            yield "base", r * n_out + n_out - 1, max_pad * n_out
            yield "B_e", (n_out - 1) * max_rank + max_rank - 1, n_out * max_rank


# ----------------------------------------------------------------------------- gather fold
def gather_touched(indices, n_slots, top_k, x_gather, row_map, ra, n_tab, n_ad, x_rows, base_rows, k_in, n_out,
                   max_rank):
    """gather_shrink_kernel / gather_expand_kernel: one workgroup per (slot, chunk); a slot whose id,
    adapter, map entry or x row falls outside its table or buffer is skipped before any other access."""
    for s in range(n_slots):
        yield "indices", s, n_slots
        e = int(indices[s])
        if e < 0 or e >= n_tab:
            continue
        yield "row_adapter" if ra is not None else "none", s // top_k, n_slots // top_k
        a = int(ra[s // top_k]) if ra is not None else 0
        if a < 0 or a >= n_ad:
            continue
        yield "table", a * n_tab + e, n_ad * n_tab
        row = int(row_map[s]) if row_map is not None else s
        if row < 0 or row >= base_rows:
            continue
        xrow = s // top_k if x_gather else row
        if xrow >= x_rows:
            continue
        yield "x", xrow * k_in + k_in - 1, x_rows * k_in
        yield "xa", s * max_rank + max_rank - 1, n_slots * max_rank
        for jb in range(max_rank // 16):
            yield "A_e", (jb * 16 + 15) * k_in + k_in - 1, max_rank * k_in
        for by in range(-(-n_out // 256)):
            for wave in range(4):
                n0 = by * 256 + wave * 64
                if n0 >= n_out:
                    continue
                yield "base", row * n_out + min(n0 + 63, n_out - 1), base_rows * n_out
                yield "B_e", min(n0 + 63, n_out - 1) * max_rank + max_rank - 1, n_out * max_rank


# ----------------------------------------------------------------------------- routings
def _routings():
    out = []
    for name in ("tiny", "decode_int4", "lora_prefill"):
        cfg = CONFIGS[name]
        ids, _ = oracle.route(make_router_logits(cfg), cfg.top_k)
        out.append((name, cfg.top_k, cfg.E, cfg.block_size, ids))
    # padded total exactly at the capacity: every expert holds a multiple of bs plus one pair
    for E, bs, per in ((2, 64, 8 * 64 + 1), (3, 16, 5 * 16 + 1), (8, 16, 7 * 16 + 1), (5, 128, 3 * 128 + 1)):
        out.append((f"tight_E{E}_bs{bs}", 1, E, bs, np.repeat(np.arange(E), per).reshape(-1, 1)))
    # ids outside [0, E) are dropped by the alignment
    rng = np.random.default_rng(3)
    ids = rng.integers(-2, 10, (50, 2)).astype(np.int32)
    out.append(("dropped_ids", 2, 8, 16, ids))
    return out


def _check(gen, what):
    n = 0
    for kind, idx, lim in gen:
        assert 0 <= idx < lim, f"{what}: {kind} index {idx} outside [0, {lim})"
        n += 1
    return n


@pytest.mark.parametrize("case", _routings(), ids=lambda c: c[0])
def test_int4_gemm_addresses_in_bounds(case):
    name, top_k, E, bs, ids = case
    al = oracle.align(ids, E, bs)
    P = ids.size
    for gate_up, N, K in ((True, 128, 256), (False, 64, 128)):
        for G in (32, 64, 128):
            if K % G == 0:
                assert _check(int4_touched(al, P, top_k, E, N, K, G, bs, gate_up), f"{name} int4 G={G}") > 0
    _check(int4_touched(al, P, top_k, E, 64, 128, 64, bs, False, a_tok=True), f"{name} int4 gathered")


@pytest.mark.parametrize("case", _routings(), ids=lambda c: c[0])
@pytest.mark.parametrize("BM", [256, 128])
def test_fp8_gemm_addresses_in_bounds(case, BM):
    name, top_k, E, bs, ids = case
    al = oracle.align(ids, E, bs)
    P = ids.size
    for gate_up, N, K in ((True, 264, 2048), (False, 136, 1040)):
        assert _check(fp8_touched(al, P, top_k, E, N, K, BM, gate_up), f"{name} fp8 BM={BM}") > 0


@pytest.mark.parametrize("case", _routings(), ids=lambda c: c[0])
def test_lora_epilogue_addresses_in_bounds(case):
    name, top_k, E, bs, ids = case
    al = oracle.align(ids, E, bs)
    P = ids.size
    T = P // top_k
    ra = np.random.default_rng(1).integers(-1, 4, T).astype(np.int32)   # ids past n_ad included
    for BM in (128, 256):
        for n_tab, n_ad, rmap in ((E, 1, None), (max(1, E - 1), 3, ra)):
            for gate_up, N in ((True, 200), (False, 200), (False, 520)):
                _check(lora_epilogue_touched(al, P, top_k, E, N, BM, 64, n_tab, n_ad, rmap, gate_up),
                       f"{name} epilogue gate_up={gate_up} N={N}")


@pytest.mark.parametrize("case", _routings(), ids=lambda c: c[0])
def test_grouped_fold_addresses_in_bounds(case):
    name, top_k, E, bs, ids = case
    al = oracle.align(ids, E, bs)
    P = ids.size
    T = P // top_k
    max_pad = len(al["sorted_ids"])
    ra = np.random.default_rng(2).integers(-1, 4, T).astype(np.int32)
    for x_gather in (False, True):
        x_rows = T if x_gather else max_pad
        for cap in (max_pad, 100, 17):
            for s, e in oracle.lora_windows(max_pad, cap):
                for n_tab, n_ad, rmap in ((E, 1, None), (max(1, E // 2), 3, ra)):
                    _check(grouped_fold_touched(al, P, top_k, E, 96, 136, 64, n_tab, n_ad, rmap, s, e, cap, x_gather,
                                                x_rows), f"{name} fold window {s}-{e}")


@pytest.mark.parametrize("case", _routings(), ids=lambda c: c[0])
def test_gather_fold_addresses_in_bounds(case):
    name, top_k, E, bs, ids = case
    al = oracle.align(ids, E, bs)
    P = ids.size
    T = P // top_k
    flat = ids.reshape(-1)
    ra = np.random.default_rng(4).integers(-1, 4, T).astype(np.int32)
    max_pad = len(al["sorted_ids"])
    for x_gather in (False, True):
        # slot-major buffers, and the sorted buffers through the inverse map
        for row_map, base_rows in ((None, P), (al["inv"], max_pad)):
            x_rows = T if x_gather else base_rows
            for n_tab, n_ad, rmap in ((E, 1, None), (E + 3, 2, ra)):
                _check(gather_touched(flat, P, top_k, x_gather, row_map, rmap, n_tab, n_ad, x_rows, base_rows, 96,
                                      520, 64), f"{name} gather")
