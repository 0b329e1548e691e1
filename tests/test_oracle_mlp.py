"""Pins for the oracle's dense gated MLP (packed gate/up projection with SwiGLU, then the down
projection; "[SM70][Draft] Extend Qwen3.8 DFlash2 concurrency paths", "TP4-only NVFP4 verifier
follow-up").

Independent routes: numpy float64 matmuls of an independently decoded weight (hand E2M1 table
times torch's float8_e4m3fn cast), the two W13 layouts against each other, and the one-expert,
top-1 MoE oracle (itself pinned by exact rational arithmetic), which must agree bitwise.
"""
import numpy as np
import pytest

from synth import inputs as S
from tests.test_oracle_gemm import dq_independent, silu


def _case(m, k, i, n, seed, gscale=1.0):
    rng = S.rng_for(S.WORKLOAD_IDS["dense"], 40 + seed, 0)
    w13 = S.nvfp4_weights(rng, 1, 2 * i, k, gscale=gscale)
    w2 = S.nvfp4_weights(rng, 1, n, i, gscale=gscale)
    x = S.activations(rng, m, k)
    return x, w13, w2


@pytest.mark.parametrize("layout", [0, 1])
def test_gated_mlp_matches_numpy(orc, layout):
    x, w13, w2 = _case(6, 256, 48, 80, layout, gscale=0.37)
    W13, W2 = dq_independent(*w13)[0], dq_independent(*w2)[0]
    gate, up = (W13[0::2], W13[1::2]) if layout else (W13[:48], W13[48:])
    xd = x.astype(np.float64)
    h_ref = silu(xd @ gate.T) * (xd @ up.T)
    y_ref = h_ref @ W2.T
    h, y = orc.gated_mlp(x, w13, w2, layout)
    assert np.allclose(h, h_ref, rtol=1e-12, atol=1e-12 * np.abs(h_ref).max())
    assert np.allclose(y, y_ref, rtol=1e-11, atol=1e-11 * np.abs(y_ref).max())


def test_layouts_differ(orc):
    x, w13, w2 = _case(3, 128, 32, 64, 7)
    h0, _ = orc.gated_mlp(x, w13, w2, 0)
    h1, _ = orc.gated_mlp(x, w13, w2, 1)
    assert np.abs(h0 - h1).max() > 1e-3 * np.abs(h0).max()


def test_gated_mlp_is_one_expert_top1_moe_bitwise(orc):
    """A one-expert MoE with every token on slot 0 and weight 1 is the dense gated MLP, with the
    same sums in the same order, so the two oracle functions agree bit for bit."""
    sh = S.MoEShape(m=5, e=1, topk=1, k=256, i=64)
    case = S.moe_case(sh, workload="tiny", route_pattern=9)
    case["ids"] = np.zeros((sh.m, 1), np.int32)
    case["topk_weights"] = np.ones((sh.m, 1), np.float32)
    for layout in (0, 1):
        out, h_moe = orc.moe_token(case, layout=layout, want_h=True)
        h, y = orc.gated_mlp(case["x"], case["w13"], case["w2"], layout)
        assert np.array_equal(h, h_moe[:, 0, :])
        assert np.array_equal(y, out)
