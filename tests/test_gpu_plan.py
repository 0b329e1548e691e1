"""GPU parity: the routing plan must equal the oracle's plan bit-exactly (integer work).

The plan is a stable counting sort by expert, so it is unique. It is checked on the decode
(single-block) path, on the prefill (chunked) path and on both sides of the 1024-pair switch
between them. Inputs include -1 and out-of-range ids, repeated ids, E = 1, topk = 32 and 4096
experts.
"""
import numpy as np
import pytest
import torch

import gemm_nvfp4_amd as G
from synth import inputs as S

pytestmark = pytest.mark.gpu


def _ids(M, topk, E, kind, seed):
    rng = S.rng_for(3, 0, seed)
    if kind == "random_invalid":
        return rng.integers(-3, E + 3, size=(M, topk)).astype(np.int32)
    if kind == "all_invalid":
        return np.full((M, topk), -1, np.int32)
    return S.ROUTINGS[kind](rng, M, topk, E)


CASES = [
    (1, 2, 8, "uniform"), (16, 10, 512, "uniform"), (1, 10, 512, "zipf"), (16, 10, 512, "zipf"),
    (16, 10, 512, "singleton"), (16, 10, 512, "shared"), (16, 10, 512, "repeat_invalid"),
    (7, 10, 512, "repeat_invalid"), (37, 7, 100, "random_invalid"), (5, 3, 1, "random_invalid"),
    (4, 4, 16, "all_invalid"), (3, 32, 4096, "uniform"), (102, 10, 512, "uniform"),   # 1020 pairs: small path
    (103, 10, 512, "uniform"), (205, 10, 512, "random_invalid"), (2049, 1, 64, "uniform"),  # large path
    (8192, 10, 512, "uniform"), (600, 8, 4096, "zipf"),
]


@pytest.mark.parametrize("M,topk,E,kind", CASES)
def test_plan_bit_exact(orc, M, topk, E, kind):
    ids = _ids(M, topk, E, kind, seed=M * 131 + topk)
    ref = orc.plan(ids, E, 16)
    d_ids = torch.from_numpy(ids).cuda()
    plan = torch.full((G.nvfp4_moe_plan_bytes(M, topk, E) // 4,), -99, dtype=torch.int32, device="cuda")
    G.nvfp4_moe_plan(d_ids, E, plan=plan)
    torch.cuda.synchronize()
    got = G.plan_fields(plan, M, topk, E)
    for key in ("n_valid", "n_active", "n_bad", "n_tiles"):
        assert got[key] == ref[key], key
    for key in ("counts", "offsets", "active", "tile_expert", "tile_row0", "sorted_pair", "pos_of_pair"):
        assert np.array_equal(got[key], ref[key]), key
    assert list(got["hdr"][4:8]) == [M, topk, E, 16]
    _check_tile_descriptors(got, ref)
    # pair_expert: the routed id of every placed pair, -1 for skipped ones
    want = np.where(ref["pos_of_pair"] >= 0, ids.reshape(-1), -1)
    assert np.array_equal(got["pair_expert"], want)


def _check_tile_descriptors(got, ref):
    """tile_base / tile_rows / tile_pair restate the oracle's tiles and sorted order (header doc)."""
    e, r0 = ref["tile_expert"], ref["tile_row0"]
    base = ref["offsets"][e] + r0
    rows = np.minimum(16, ref["counts"][e] - r0)
    assert np.array_equal(got["tile_base"], base)
    assert np.array_equal(got["tile_rows"], rows)
    for t in range(len(e)):
        assert np.array_equal(got["tile_pair"][t, :rows[t]], ref["sorted_pair"][base[t]:base[t] + rows[t]]), t


def test_plan_rebuild_overwrites_stale_plan(orc):
    """A plan buffer reused for a second routing holds exactly the second plan."""
    M, topk, E = 16, 10, 512
    plan = torch.empty((G.nvfp4_moe_plan_bytes(M, topk, E) // 4,), dtype=torch.int32, device="cuda")
    for kind in ("shared", "uniform"):
        ids = _ids(M, topk, E, kind, seed=5)
        G.nvfp4_moe_plan(torch.from_numpy(ids).cuda(), E, plan=plan)
        torch.cuda.synchronize()
        got, ref = G.plan_fields(plan, M, topk, E), orc.plan(ids, E, 16)
        assert np.array_equal(got["sorted_pair"], ref["sorted_pair"])
        assert np.array_equal(got["pos_of_pair"], ref["pos_of_pair"])
        assert np.array_equal(got["active"], ref["active"])
