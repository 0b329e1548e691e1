"""GPU parity of the router fused with the plan (nvfp4_moe_route) against the fp64 oracle.

The router is the step before the plan ("router" among the fused MoE parts of the "[Kernel][SM70]
Improve Qwen3.8 no-MTP concurrency" page, "Scope and related PRs"). Selections are comparisons
only, so the ids must equal the oracle's bit for bit, ties, signed zeros, NaN and infinities
included; the weights are an FP32 softmax and must match the oracle's fp64 value within
1e-6 + 1e-5*|w| with the same NaN pattern. The plan written with them must equal the oracle's plan
of those ids. Cases cover the fused one-launch path (M*topk <= 1024 and E <= 1024, one to several
tokens per wave), the separate router kernel with the small and with the chunked plan, E not a
multiple of 64, topk = E and the 8192-token prefill size.
"""
import numpy as np
import pytest
import torch

import gemm_nvfp4_amd as G
from synth import inputs as S

pytestmark = pytest.mark.gpu

CASES = [  # M, E, topk, logits kind
    (1, 512, 10, "normal"), (16, 512, 10, "normal"), (64, 512, 10, "ties"), (5, 100, 7, "ties"),
    (3, 8, 8, "special"), (2, 1, 1, "normal"), (9, 1024, 32, "special"), (7, 2048, 5, "normal"),
    (300, 4096, 4, "special"), (8192, 512, 10, "normal"), (1000, 33, 1, "ties"),
]


def _check_weights(got, ref):
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    f = ~np.isnan(ref)
    assert np.all(np.abs(got[f] - ref[f]) <= 1e-6 + 1e-5 * np.abs(ref[f])), np.max(np.abs(got[f] - ref[f]))


@pytest.mark.parametrize("M,E,topk,kind", CASES)
def test_route_matches_oracle(orc, M, E, topk, kind):
    x = S.router_logits(S.rng_for(S.WORKLOAD_IDS["route"], 10, M * 7919 + E), M, E, kind)
    ref_ids, ref_w = orc.route(x, topk)
    ids, w, plan = G.nvfp4_moe_route(torch.from_numpy(x).cuda(), topk)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    _check_weights(w.cpu().numpy().astype(np.float64), ref_w)
    pl = orc.plan(ref_ids, E, 16)
    got = G.plan_fields(plan, M, topk, E)
    for key in ("n_valid", "n_active", "n_bad", "n_tiles"):
        assert got[key] == pl[key], key
    for key in ("counts", "offsets", "active", "tile_expert", "tile_row0", "sorted_pair", "pos_of_pair"):
        assert np.array_equal(got[key], pl[key]), key


def test_route_plan_equals_plan_of_its_ids():
    """The fused launch leaves the same plan as nvfp4_moe_plan on the ids it wrote."""
    M, E, topk = 16, 512, 10
    x = S.router_logits(S.rng_for(S.WORKLOAD_IDS["route"], 11, 0), M, E)
    ids, _, plan = G.nvfp4_moe_route(torch.from_numpy(x).cuda(), topk)
    plan2 = G.nvfp4_moe_plan(ids, E)
    torch.cuda.synchronize()
    a, b = G.plan_fields(plan, M, topk, E), G.plan_fields(plan2, M, topk, E)
    for key in ("counts", "offsets", "active", "tile_expert", "tile_row0", "tile_base", "tile_rows", "sorted_pair",
                "pos_of_pair", "pair_expert"):
        assert np.array_equal(a[key], b[key]), key
    assert np.array_equal(a["hdr"][:8], b["hdr"][:8])  # words 8..15 are reserved
    for t, n in enumerate(a["tile_rows"]):  # tile_pair is defined for rows < tile_rows only
        assert np.array_equal(a["tile_pair"][t, :n], b["tile_pair"][t, :n]), t


def test_route_batch_invariance():
    """A token's ids and weights do not depend on the other tokens (bitwise)."""
    M, E, topk = 40, 512, 10
    x = torch.from_numpy(S.router_logits(S.rng_for(S.WORKLOAD_IDS["route"], 12, 0), M, E)).cuda()
    ids, w, _ = G.nvfp4_moe_route(x, topk)
    for t in (0, 17, 39):
        i1, w1, _ = G.nvfp4_moe_route(x[t:t + 1].contiguous(), topk)
        assert torch.equal(i1[0], ids[t]) and torch.equal(w1[0].view(torch.int32), w[t].view(torch.int32))


def test_route_rejects_topk_above_e():
    x = torch.zeros((2, 4), dtype=torch.float32, device="cuda")
    with pytest.raises(G.NVFP4Error):
        G.nvfp4_moe_route(x, 5)
