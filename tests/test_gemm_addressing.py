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
