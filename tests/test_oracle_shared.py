"""Pins for the oracle's shared expert and shared gate ("shared gate" among the fused MoE parts of
the "[Kernel][SM70] Improve Qwen3.8 no-MTP concurrency" page, "Scope and related PRs"; no formula is
printed, so the reading is the common one: out = routed + sigmoid(x . g) * shared MLP(x)).

Independent routes: scipy's expit of a numpy float64 dot product for the gate; the structural
identity that a shared expert equal to a routed one-expert MoE with slot weight sigma doubles as
a second slot; numpy for the whole combination on a tiny case.
"""
import numpy as np
from scipy.special import expit

from synth import inputs as S
from tests.test_oracle_gemm import dq_independent, silu


def test_shared_gate_matches_expit(orc):
    rng = S.rng_for(S.WORKLOAD_IDS["decode"], 70, 0)
    x = S.activations(rng, 9, 512)
    g = (rng.standard_normal(512) / np.sqrt(512)).astype(np.float16)
    ref = expit(x.astype(np.float64) @ g.astype(np.float64))
    np.testing.assert_allclose(orc.shared_gate(x, g), ref, rtol=1e-14, atol=1e-15)
    assert np.all(orc.shared_gate(np.zeros((2, 512), np.float16), g) == 0.5)


def test_moe_with_shared_matches_numpy(orc):
    sh = S.MoEShape(m=4, e=4, topk=2, k=128, i=32)
    case = S.moe_case(sh, workload="tiny", route_pattern=21)
    shared = S.shared_expert(S.rng_for(S.WORKLOAD_IDS["tiny"], 71, 0), sh.k, 48)
    out, ys, sg = orc.moe_with_shared(case, shared)
    x = case["x"].astype(np.float64)
    W13, W2 = dq_independent(*shared["w13"])[0], dq_independent(*shared["w2"])[0]
    ys_ref = (silu(x @ W13[:48].T) * (x @ W13[48:].T)) @ W2.T
    sg_ref = expit(x @ shared["g"].astype(np.float64))
    routed = orc.moe_token(case)
    np.testing.assert_allclose(ys, ys_ref, rtol=1e-10, atol=1e-10 * np.abs(ys_ref).max())
    np.testing.assert_allclose(out, routed + sg_ref[:, None] * ys_ref, rtol=1e-10, atol=1e-10 * np.abs(out).max())


def test_shared_expert_equals_an_extra_routed_slot(orc):
    """With E = 1 and the shared expert's weights as that expert's, the routed output with slot
    weight sigma equals the shared term (same sums, same order), bitwise in double."""
    sh = S.MoEShape(m=3, e=1, topk=1, k=128, i=32)
    shared = S.shared_expert(S.rng_for(S.WORKLOAD_IDS["tiny"], 72, 0), sh.k, sh.i)
    case = S.moe_case(sh, workload="tiny", route_pattern=22, weights=(shared["w13"], shared["w2"]))
    case["ids"] = np.zeros((3, 1), np.int32)
    _, ys, sg = orc.moe_with_shared(case, shared)
    case["topk_weights"] = sg.astype(np.float32)[:, None]
    routed = orc.moe_token(case)
    # fp32 weights: compare against sigma rounded to fp32 the same way
    assert np.array_equal(routed, sg.astype(np.float32).astype(np.float64)[:, None] * ys)
