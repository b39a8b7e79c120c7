"""moe_align_noalloc (the static-table form of moe_align, for callers that cannot allocate) gives
the same alignment as moe_align with a workspace: bit-exact on every output array, on two calls
in a row with the second smaller, so a table left over from the first call cannot leak into the
second.  Both calls go through the C ABI."""
import numpy as np
import pytest

from moe_synth import MoeConfig, make_router_logits
from _util import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import mixture_experts_routed_route_amd as m
    m.lib()
    return torch.device("cuda:0")


def _arrays(r, P):
    return {"counts": r.counts.cpu().numpy(), "offsets": r.offsets.cpu().numpy(),
            "sorted_ids": r.sorted_ids.cpu().numpy(), "expert_ids": r.expert_ids.cpu().numpy(),
            "total": r.total_padded.cpu().numpy(), "inv": r.inv_sorted.cpu().numpy()[:P]}


# the first call uses 128 chunks (of 512 pairs) x 128 experts of the table, the second 12 chunks x
# 64 experts; the last case fits one workgroup (the table is not used at all)
CASES = [
    (MoeConfig("big", T=8192, H=8, I=8, E=128, top_k=8, block_size=64, logits="zipf", seed=41),
     MoeConfig("small", T=1000, H=8, I=8, E=64, top_k=6, block_size=16, seed=42)),
    (MoeConfig("mid", T=3000, H=8, I=8, E=256, top_k=4, block_size=32, seed=43),
     MoeConfig("one_chunk", T=16, H=8, I=8, E=64, top_k=6, block_size=16, seed=44)),
]


@pytest.mark.parametrize("first,second", CASES, ids=["big_then_small", "mid_then_one_chunk"])
def test_align_noalloc_matches_align(dev, first, second):
    import torch
    import mixture_experts_routed_route_amd as m
    for cfg in (first, second):
        print(f"align_noalloc {cfg.name}: P={cfg.P} E={cfg.E} bs={cfg.block_size}", flush=True)
        ids, _ = m.moe_route(to_dev(make_router_logits(cfg)), cfg.top_k)
        ref = m.moe_align(ids, cfg.E, cfg.block_size)
        got = m.Routing.allocate(cfg.P, cfg.top_k, cfg.E, cfg.block_size, dev)
        for t in (got.counts, got.offsets, got.sorted_ids, got.expert_ids, got.total_padded, got.inv_sorted):
            t.fill_(-7)   # every output must be written
        m.moe_align_noalloc(ids, cfg.E, cfg.block_size, got)
        torch.cuda.synchronize()
        a, b = _arrays(ref, cfg.P), _arrays(got, cfg.P)
        for k in a:
            assert np.array_equal(a[k], b[k]), f"{cfg.name}: {k} differs"


def test_align_noalloc_refuses_oversized_table(dev):
    import torch
    import mixture_experts_routed_route_amd as m
    from mixture_experts_routed_route_amd._lib import MOE_EUNSUPPORTED
    # 2^18 cells / 256 experts = 1024 chunks of 512 pairs; one pair more needs 1025 chunks
    P = 1024 * 512 + 1
    ids = torch.zeros(P, dtype=torch.int32, device=dev)
    r = m.Routing.allocate(P, 1, 256, 16, dev)
    with pytest.raises(m.MoeError) as ei:
        m.moe_align_noalloc(ids, 256, 16, r)
    assert ei.value.status == MOE_EUNSUPPORTED and "static table" in str(ei.value)
