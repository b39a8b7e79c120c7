"""CPU model of the bf16 grouped GEMM's addressing (tile decode from expert_offsets, the A row
each tile row loads, the weight rows of a panel, the rows it stores), checked against the
buffer extents.  It restates the kernel's integer arithmetic so that every row a launch can
touch is shown to be in bounds on the CPU, including routings whose padded total reaches the
sorted capacity (a tile's row range then runs past the end of the buffer)."""
import numpy as np
import pytest

import oracle
from moe_synth import CONFIGS, MoeConfig, make_router_logits

BP = 256


def touched_rows(P, top_k, E, N, al, gate_up, BM):
    """Yield (kind, index, limit) for every A row, weight row and C row a launch can address."""
    max_pad = len(al["sorted_ids"])
    T = P // top_k
    sid, off = al["sorted_ids"], al["offsets"]
    ncol = BP // 2 if gate_up else BP
    lo = [min(max(int(off[e]), 0), max_pad) for e in range(E)]
    hi = [min(max(int(off[e + 1]), lo[e]), max_pad) for e in range(E)]
    nt = [-(-(hi[e] - lo[e]) // BM) for e in range(E)]
    first = np.concatenate([[0], np.cumsum(nt)])
    for e in range(E):
        for t in range(nt[e]):
            r0 = lo[e] + t * BM
            r_end = min(r0 + BM, hi[e])
            for row in range(BM):
                r = r0 + row
                src = -1
                if r < r_end and 0 <= sid[r] < P:
                    src = sid[r] // top_k if gate_up else r
                srow = src if src >= 0 else (0 if gate_up else r0)
                yield "A", srow, (T if gate_up else max_pad)
                if src >= 0:
                    yield "C", r, max_pad
    for n_t in range(-(-N // ncol)):
        for prow in range(BP):
            n = n_t * ncol + (prow % (BP // 2) if gate_up else prow)
            yield "B", min(n, N - 1), N


def _cases():
    out = []
    for name, cfg in CONFIGS.items():
        if cfg.P > 20000:
            continue
        ids, _ = oracle.route(make_router_logits(cfg), cfg.top_k)
        out.append((name, cfg.P, cfg.top_k, cfg.E, cfg.block_size, ids))
    # padded total exactly at the capacity: every expert holds a multiple of bs plus one pair
    for E, bs, per in ((2, 64, 8 * 64 + 1), (3, 64, 5 * 64 + 1), (8, 16, 7 * 16 + 1), (5, 128, 3 * 128 + 1)):
        ids = np.repeat(np.arange(E), per).reshape(-1, 1)
        out.append((f"tight_E{E}_bs{bs}", E * per, 1, E, bs, ids))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c[0])
def test_every_addressed_row_in_bounds(case):
    name, P, top_k, E, bs, ids = case
    al = oracle.align(ids, E, bs)
    for gate_up in (True, False):
        for BM in (128, 256):
            for kind, idx, lim in touched_rows(P, top_k, E, 256, al, gate_up, BM):
                assert 0 <= idx < lim, f"{name} gate_up={gate_up} BM={BM}: {kind} row {idx} outside [0, {lim})"


def _decode_tile(L, gm, m_real, n_tiles):
    """Band decode of a logical tile (restates the kernel's integer arithmetic)."""
    band_tiles = gm * n_tiles
    band = L // band_tiles
    in_band = L - band * band_tiles
    gm_b = min(gm, m_real - band * gm)
    n_t = in_band // gm_b
    return band * gm + (in_band - n_t * gm_b), n_t


def _assigned_tiles(m_real, n_tiles, grid, gm):
    """Every (row tile, panel) that the workgroups of a launch process, in kernel order."""
    T = m_real * n_tiles
    per_xcd = grid >> 3
    out = []
    for bid in range(grid):
        xcd, slot = bid & 7, bid >> 3
        l_hi = T * (xcd + 1) // 8
        L = T * xcd // 8 + slot
        while slot < per_xcd and L < l_hi:
            out.append(_decode_tile(L, gm, m_real, n_tiles))
            L += per_xcd
    return out


@pytest.mark.parametrize("m_real,n_tiles,grid,gm", [
    (37, 112, 256, 8), (37, 16, 672, 8), (1, 1, 8, 8), (5, 3, 256, 8), (351, 8, 256, 8),
    (64, 11, 256, 16), (9, 7, 16, 4), (200, 1, 256, 8), (3, 200, 24, 2)])
def test_persistent_assignment_covers_each_tile_once(m_real, n_tiles, grid, gm):
    """The workgroups of a launch (persistent or one per tile) process every (row tile, column
    panel) of the real tile grid exactly once."""
    got = _assigned_tiles(m_real, n_tiles, grid, gm)
    assert len(got) == m_real * n_tiles
    assert sorted(got) == [(m, n) for m in range(m_real) for n in range(n_tiles)]


def _split_tail_segments(T, nk, grid, min_stages=8):
    """Segments (tile, k_begin, k_end, pos, pieces, slot of piece 0, slot stride) of a launch with
    a workspace (restates the kernel's integer arithmetic)."""
    per_xcd = grid >> 3
    Tw = T
    rest = T % grid
    if rest > 0 and min(per_xcd // ((rest + 7) // 8), nk // min_stages) >= 2:
        Tw = T // grid * grid
    tail = T - Tw
    out = []
    for bid in range(grid):
        xcd, slot = bid & 7, bid >> 3
        pos = xcd * per_xcd + slot
        l_hi = Tw * (xcd + 1) // 8
        L = Tw * xcd // 8 + slot
        while slot < per_xcd and L < l_hi:
            out.append((L, 0, nk, pos, 1, None, None))
            L += per_xcd
        if tail > 0:
            a_x = tail * xcd // 8
            n_x = tail * (xcd + 1) // 8 - a_x
            if n_x > 0:
                s_x = max(1, min(per_xcd // n_x, nk // min_stages))
                if slot < s_x * n_x:
                    u, j = slot % n_x, slot // n_x
                    out.append((Tw + a_x + u, j * nk // s_x, (j + 1) * nk // s_x, pos, s_x,
                                xcd * per_xcd + u, n_x))
    return out, Tw


@pytest.mark.parametrize("T,nk,grid", [
    (592, 224, 256), (4032, 64, 256), (299, 45, 256), (276, 25, 256), (272, 17, 256), (128, 17, 256),
    (80, 16, 256), (192, 34, 256), (1, 300, 256), (257, 8, 256), (384, 40, 256), (255, 100, 256),
    (17, 64, 16), (0, 10, 256)])
def test_split_tail_covers_each_stage_once(T, nk, grid):
    """With a workspace, the whole-tile rounds and the tail pieces cover every (tile, K stage)
    exactly once; the pieces of a tile share one piece count and sit on slots piece0 + j*stride,
    all inside the grid's partial slots; tail tile counters stay below the grid size."""
    segs, Tw = _split_tail_segments(T, nk, grid)
    cover = np.zeros((T, nk), np.int32)
    pieces = {}
    for L, kb, ke, pos, s, first, stride in segs:
        assert 0 <= L < T and 0 <= kb < ke <= nk and 0 <= pos < grid
        cover[L, kb:ke] += 1
        if s > 1:
            assert L - Tw < grid and ke - kb >= 8
            pieces.setdefault(L, []).append((kb, pos, s, first, stride))
    assert (cover == 1).all()
    for L, ps in pieces.items():
        ps.sort()
        s, first, stride = ps[0][2:]
        assert len(ps) == s and all(p[2:] == (s, first, stride) for p in ps)
        assert [p[1] for p in ps] == [first + j * stride for j in range(s)]
    # each workgroup runs whole tiles first, then at most one piece
    per_pos = {}
    for seg in segs:
        per_pos.setdefault(seg[3], []).append(seg)
    for lst in per_pos.values():
        assert sum(1 for x in lst if x[4] > 1 or x[0] >= Tw) <= 1


def test_expert_of_row_tile_binary_search():
    """Largest expert whose first row tile is <= m_t, with empty experts in between (the kernel's
    binary search over the inclusive tile scan): the expert found owns tile m_t, and it is the
    count of experts with tb[e] <= m_t, minus one."""
    rng = np.random.default_rng(5)
    cases = [[0, 3, 0, 0, 2, 0, 1, 0]]
    cases += [list(rng.integers(0, 3, size=E) * (rng.random(E) < 0.6)) for E in (1, 7, 64, 65, 200, 256)]
    for nt in cases:
        E = len(nt)
        tb = np.concatenate([[0], np.cumsum(nt)])
        for m_t in range(int(tb[-1])):
            a, b = 0, E - 1
            while a < b:
                mid = (a + b + 1) >> 1
                if tb[mid] <= m_t:
                    a = mid
                else:
                    b = mid - 1
            assert tb[a] <= m_t < tb[a + 1] and nt[a] > 0
            assert a == int(np.sum(tb[:E] <= m_t)) - 1
