"""Pins for the oracle's router (top-k expert selection and the softmax of the selected logits).

The pages name the router among the fused MoE parts ("[Kernel][SM70] Improve Qwen3.8 no-MTP
concurrency", "Scope and related PRs") and print no formula; the reading (largest logits first,
ties by expert id, NaN last, softmax over the selection) is pinned against library routines:
numpy's stable argsort and scipy's softmax, plus hand cases and invariants.
"""
import numpy as np
import pytest
from scipy.special import softmax

from synth import inputs as S


def _argsort_desc_stable(x):
    # Stable argsort of -x: larger first, equal values (+0 == -0) in ascending index order.
    return np.argsort(-x, axis=1, kind="stable")


@pytest.mark.parametrize("m,e,topk", [(7, 512, 10), (5, 100, 7), (3, 8, 8), (4, 1, 1), (2, 4096, 32)])
def test_route_matches_argsort_and_softmax(orc, m, e, topk):
    x = S.router_logits(S.rng_for(S.WORKLOAD_IDS["route"], 0, m * 1000 + e), m, e)
    ids, w = orc.route(x, topk)
    ref = _argsort_desc_stable(x.astype(np.float64))[:, :topk]
    assert np.array_equal(ids, ref)
    for t in range(m):
        np.testing.assert_allclose(w[t], softmax(x[t, ids[t]].astype(np.float64)), rtol=1e-14, atol=0)


def test_route_ties_and_signed_zeros(orc):
    x = S.router_logits(S.rng_for(S.WORKLOAD_IDS["route"], 1, 0), 40, 33, kind="ties")
    assert np.any(np.signbit(x) & (x == 0)) and np.any(~np.signbit(x) & (x == 0))
    ids, w = orc.route(x, 12)
    assert np.array_equal(ids, _argsort_desc_stable(x.astype(np.float64))[:, :12])
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-14)


def test_route_hand_cases(orc):
    ids, w = orc.route(np.array([[1.0, 3.0, 2.0, 3.0]], np.float32), 2)
    assert ids.tolist() == [[1, 3]] and w.tolist() == [[0.5, 0.5]]  # tie: lower expert first
    ids, w = orc.route(np.array([[0.0, -0.0, 0.0]], np.float32), 3)
    assert ids.tolist() == [[0, 1, 2]]  # +0 and -0 are equal
    ids, w = orc.route(np.array([[np.log(3.0), 0.0, -5.0]], np.float32), 2)
    np.testing.assert_allclose(w, [[0.75, 0.25]], rtol=1e-7)  # exp(l0-l0) : exp(-log 3) = 3 : 1
    # NaN ranks below every number, -inf included; NaNs among themselves by index.
    ids, w = orc.route(np.array([[np.nan, -np.inf, np.nan, 2.0]], np.float32), 4)
    assert ids.tolist() == [[3, 1, 0, 2]]
    assert np.all(np.isnan(w))  # a selected NaN makes the softmax NaN
    ids, w = orc.route(np.array([[np.nan, -np.inf, 1.0, 2.0]], np.float32), 2)
    assert ids.tolist() == [[3, 2]] and np.all(np.isfinite(w))
    ids, w = orc.route(np.array([[np.inf, 1.0]], np.float32), 2)
    assert ids.tolist() == [[0, 1]] and np.all(np.isnan(w))  # inf - inf = NaN, and NaN reaches the sum
    ids, w = orc.route(np.array([[-np.inf, -np.inf]], np.float32), 1)
    assert ids.tolist() == [[0]] and np.isnan(w[0, 0])


def test_route_special_values_brute_force(orc):
    x = S.router_logits(S.rng_for(S.WORKLOAD_IDS["route"], 2, 0), 30, 50, kind="special")
    ids, w = orc.route(x, 9)
    for t in range(x.shape[0]):
        # Python's sort with a key: not-NaN first, larger value first (-0 == +0), then index.
        order = sorted(range(x.shape[1]), key=lambda e: (bool(np.isnan(x[t, e])),
                                                         0.0 if np.isnan(x[t, e]) else -float(x[t, e]), e))
        assert ids[t].tolist() == order[:9]
        sel = x[t, ids[t]].astype(np.float64)
        if np.all(np.isfinite(sel)) or (np.all(~np.isnan(sel)) and sel[0] != np.inf and sel[0] != -np.inf):
            np.testing.assert_allclose(w[t], softmax(sel), rtol=1e-14, atol=1e-300)


def test_route_weights_ratio_invariant(orc):
    x = S.router_logits(S.rng_for(S.WORKLOAD_IDS["route"], 3, 0), 6, 64)
    ids, w = orc.route(x, 5)
    for t in range(6):
        l = x[t, ids[t]].astype(np.float64)
        np.testing.assert_allclose(w[t, 1:] / w[t, 0], np.exp(l[1:] - l[0]), rtol=1e-13)
        assert np.all(np.diff(l) <= 0) and abs(w[t].sum() - 1.0) < 1e-14
