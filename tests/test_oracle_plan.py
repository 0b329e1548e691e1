"""Pins for the oracle's routing plan (stable counting sort of (token, slot) pairs by expert).

The reference is numpy's stable argsort (a library routine) together with the plan's invariants.
The check is brute force over every tiny routing, including -1 and out-of-range ids. The pages
call it one integer plan that W13 and W2 reuse ("[Kernel][SM70] Improve Qwen3.8 no-MTP
concurrency", "Scope and related PRs").
"""
import itertools

import numpy as np
import pytest


def numpy_plan(ids, E, BM):
    flat = ids.reshape(-1)
    P = flat.size
    valid = (flat >= 0) & (flat < E)
    keys = np.where(valid, flat, E)  # invalid pairs sort last and are dropped
    order = np.argsort(keys, kind="stable")
    nv = int(valid.sum())
    sorted_pair = order[:nv].astype(np.int32)
    counts = np.bincount(flat[valid], minlength=E).astype(np.int32) if nv else np.zeros(E, np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    pos = np.full(P, -1, np.int32)
    pos[sorted_pair] = np.arange(nv, dtype=np.int32)
    active = np.nonzero(counts)[0].astype(np.int32)
    # Row tiles from counts alone: ceil(count / BM) tiles per active expert, numbered from each
    # expert's first tile (np.repeat and a cumulative sum, not a walk over the rows).
    per = -(-counts[active] // BM)
    te = np.repeat(active, per).astype(np.int32)
    first = np.repeat(np.cumsum(per) - per, per)
    tr = (BM * (np.arange(int(per.sum())) - first)).astype(np.int32)
    n_bad = int(((flat != -1) & ~valid).sum())
    return dict(counts=counts, offsets=offsets, sorted_pair=sorted_pair, pos_of_pair=pos, active=active,
                tile_expert=te, tile_row0=tr, n_valid=nv, n_active=len(active), n_bad=n_bad, n_tiles=len(te))


def check_tiles_partition(pl, E, BM):
    """The row tiles cover every expert's bucket rows exactly once, in (expert, first row) order,
    each with 1..BM rows, and their number is the sum of ceil(count / BM) over the experts."""
    te, tr, counts, offs = pl["tile_expert"], pl["tile_row0"], pl["counts"], pl["offsets"]
    assert pl["n_tiles"] == sum(-(-int(c) // BM) for c in counts)
    cover = np.zeros(pl["n_valid"], np.int64)
    for e, r0 in zip(te.tolist(), tr.tolist()):
        assert 0 <= e < E and 0 <= r0 < counts[e]
        rows = min(BM, int(counts[e]) - r0)
        assert 1 <= rows <= BM
        cover[offs[e] + r0: offs[e] + r0 + rows] += 1
    assert np.all(cover == 1)
    keys = list(zip(te.tolist(), tr.tolist()))
    assert keys == sorted(keys) and len(set(keys)) == len(keys)


def check_invariants(pl, ids, E):
    flat = ids.reshape(-1)
    assert pl["counts"].sum() == pl["n_valid"]
    assert np.all(np.diff(pl["offsets"]) >= 0) and pl["offsets"][0] == 0 and pl["offsets"][E] == pl["n_valid"]
    sp = pl["sorted_pair"]
    assert sorted(sp.tolist()) == sorted(np.nonzero((flat >= 0) & (flat < E))[0].tolist())
    for j, p in enumerate(sp):
        assert pl["pos_of_pair"][p] == j
        e = flat[p]
        assert pl["offsets"][e] <= j < pl["offsets"][e + 1]
    for e in range(E):  # stable: ascending p inside a bucket
        b = sp[pl["offsets"][e]:pl["offsets"][e + 1]]
        assert np.all(np.diff(b) > 0)


def compare(pl, ref):
    for key in ("counts", "offsets", "sorted_pair", "pos_of_pair", "active", "tile_expert", "tile_row0"):
        assert np.array_equal(pl[key], ref[key]), key
    for key in ("n_valid", "n_active", "n_bad", "n_tiles"):
        assert pl[key] == ref[key], key


def test_plan_brute_force_tiny(orc):
    n = 0
    for E in (1, 2, 3):
        alphabet = [-2, -1] + list(range(E)) + [E]
        for M in (0, 1, 2, 3):
            for topk in (1, 2):
                for combo in itertools.product(alphabet, repeat=M * topk):
                    ids = np.array(combo, np.int32).reshape(M, topk)
                    for BM in (1, 2):
                        pl = orc.plan(ids, E, BM)
                        compare(pl, numpy_plan(ids, E, BM))
                        check_invariants(pl, ids, E)
                        check_tiles_partition(pl, E, BM)
                        n += 1
    assert n > 10000


@pytest.mark.parametrize("seed", range(6))
def test_plan_random_against_numpy(orc, seed):
    rng = np.random.default_rng(seed)
    M, topk, E = int(rng.integers(1, 300)), int(rng.integers(1, 12)), int(rng.integers(1, 600))
    ids = rng.integers(-3, E + 3, size=(M, topk)).astype(np.int32)
    pl = orc.plan(ids, E, 16)
    compare(pl, numpy_plan(ids, E, 16))
    check_invariants(pl, ids, E)
    check_tiles_partition(pl, E, 16)


def test_plan_prefill_size(orc):
    from synth import inputs as S
    rng = S.rng_for(4, 0, 1000)
    ids = S.routing_uniform(rng, 8192, 10, 512)
    pl = orc.plan(ids, 512, 16)
    compare(pl, numpy_plan(ids, 512, 16))
    check_tiles_partition(pl, 512, 16)
    assert pl["n_valid"] == 81920 and pl["n_bad"] == 0
