"""Pins for the oracle's GEMM parts: dequantization, the dense projection and the grouped MoE.

Nothing here re-types the oracle's formulas. The checks use independent routes:
  - dequantization with a hand E2M1 table times torch's float8_e4m3fn cast;
  - numpy's float64 matmul (a library routine);
  - exact rational brute force (fractions.Fraction) on the tiny MoE shape;
  - an integer-exact case where every sum is an exact multiple of 0.5;
  - structural special cases: topk=1 reduces to a dense SwiGLU MLP, E=1 to dense GEMMs, zero
    codes give a zero output;
  - the grouped (plan-driven) form against the per-token loop, bitwise in double.
The method follows the "[Kernel][SM70] Improve Qwen3.8 no-MTP concurrency" page ("Scope and
related PRs"): W13 with SiLU(gate)*up, then W2 with a top-k-weighted reduction.
"""
import math
from fractions import Fraction as F

import numpy as np
import pytest
import torch

from synth import inputs as S

E2M1_HAND = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])


def dq_independent(codes, scales, gs):
    G, N, K2 = codes.shape
    nib = np.stack([codes & 15, codes >> 4], -1).reshape(G, N, 2 * K2)
    e4 = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return E2M1_HAND[nib] * np.repeat(e4, 16, axis=2) * gs.astype(np.float64)[:, None, None]


def silu(g):
    return g / (1.0 + np.exp(-g))


def test_dequant_matches_independent_decode(orc):
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 256, (3, 5, 32), dtype=np.uint8)
    scales = rng.integers(0, 256, (3, 5, 4), dtype=np.uint8)
    gs = np.array([1.0, 0.37, -2.5], np.float32)
    a, b = orc.dequant(codes, scales, gs), dq_independent(codes, scales, gs)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    assert np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])


def test_linear_matches_numpy_matmul(orc):
    rng = S.rng_for(1, 5, 0)
    w = S.nvfp4_weights(rng, 1, 96, 512, gscale=0.37)
    x = S.activations(rng, 7, 512)
    ref = x.astype(np.float64) @ dq_independent(*w)[0].T
    got = orc.linear(x, w)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_linear_integer_exact(orc):
    """Scales 0x38 (=1), global 1, x in {-1,0,1}: every partial sum is a multiple of 0.5, so the
    result is exact; brute force in Python integers (twice the value) must agree exactly."""
    rng = np.random.default_rng(11)
    N, K, M = 40, 256, 5
    codes = rng.integers(0, 256, (1, N, K // 2), dtype=np.uint8)
    scales = np.full((1, N, K // 16), 0x38, np.uint8)
    x = rng.integers(-1, 2, (M, K)).astype(np.float16)
    twice = [0, 1, 2, 3, 4, 6, 8, 12]  # 2 * E2M1 magnitude, integers
    got = orc.linear(x, (codes, scales, np.ones(1, np.float32)))
    for m in range(M):
        for n in range(N):
            acc = 0
            for k in range(K):
                byte = int(codes[0, n, k // 2])
                c = (byte >> 4) if k & 1 else (byte & 15)
                v = twice[c & 7] * (-1 if c & 8 else 1)
                acc += int(x[m, k]) * v
            assert got[m, n] == acc / 2


def _fraction_moe(case, layout):
    """Exact-rational MoE for one token: g, u and y, out exact; h = silu(g)*u in double."""
    sh = case["shape"]
    W13 = dq_independent(*case["w13"])
    W2 = dq_independent(*case["w2"])
    outs = []
    for t in range(sh.m):
        xt = [F(float(v)) for v in case["x"][t].astype(np.float64)]
        out = [F(0)] * sh.k
        for k in range(sh.topk):
            e = int(case["ids"][t, k])
            if e < 0 or e >= sh.e:
                continue
            h = []
            for i in range(sh.i):
                gr, ur = (2 * i, 2 * i + 1) if layout else (i, sh.i + i)
                g = sum(a * F(float(b)) for a, b in zip(xt, W13[e, gr]))
                u = sum(a * F(float(b)) for a, b in zip(xt, W13[e, ur]))
                gf, uf = float(g), float(u)
                h.append(F(gf / (1.0 + math.exp(-gf)) * uf))
            wk = F(float(case["topk_weights"][t, k]))
            for n in range(sh.k):
                y = sum(F(float(a)) * b for a, b in zip(W2[e, n], h))
                out[n] += wk * y
        outs.append([float(v) for v in out])
    return np.array(outs)


@pytest.mark.parametrize("layout", [0, 1])
def test_moe_tiny_exact_rational(orc, layout):
    case = S.moe_case(S.TINY, workload="tiny", gscale2=0.37)
    ref = _fraction_moe(case, layout)
    got = orc.moe_token(case, layout=layout)
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()
    # layouts really differ (the same bytes read as the other layout give another result)
    other = orc.moe_token(case, layout=1 - layout)
    assert np.abs(other - ref).max() > 1e-3 * np.abs(ref).max()


def test_moe_topk1_is_dense_swiglu_mlp(orc):
    sh = S.MoEShape(m=5, e=4, topk=1, k=128, i=64)
    case = S.moe_case(sh, workload="tiny", route_pattern=3)
    case["topk_weights"] = np.ones((sh.m, 1), np.float32)
    W13, W2 = dq_independent(*case["w13"]), dq_independent(*case["w2"])
    x = case["x"].astype(np.float64)
    ref = np.zeros((sh.m, sh.k))
    for t in range(sh.m):
        e = case["ids"][t, 0]
        g, u = W13[e, :sh.i] @ x[t], W13[e, sh.i:] @ x[t]
        ref[t] = W2[e] @ (silu(g) * u)
    got = orc.moe_token(case)
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-10 * np.abs(ref).max())


def test_moe_single_expert_is_dense_gemms(orc):
    sh = S.MoEShape(m=6, e=1, topk=1, k=128, i=32)
    case = S.moe_case(sh, workload="tiny", route_pattern=4)
    W13, W2 = dq_independent(*case["w13"]), dq_independent(*case["w2"])
    x = case["x"].astype(np.float64)
    G, U = x @ W13[0, :sh.i].T, x @ W13[0, sh.i:].T
    ref = (silu(G) * U) @ W2[0].T * case["topk_weights"].astype(np.float64)
    got = orc.moe_token(case)
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-10 * np.abs(ref).max())


def test_moe_zero_codes_give_zero(orc):
    case = S.moe_case(S.TINY, workload="tiny")
    c13, s13, g13 = case["w13"]
    case["w13"] = (np.zeros_like(c13), s13, g13)
    out = orc.moe_token(case)
    assert np.all(out == 0)


@pytest.mark.parametrize("routing", ["uniform", "zipf", "shared", "repeat_invalid"])
@pytest.mark.parametrize("layout", [0, 1])
def test_grouped_equals_per_token_bitwise(orc, routing, layout):
    sh = S.MoEShape(m=9, e=24, topk=4, k=128, i=64)
    case = S.moe_case(sh, routing=routing, workload="stress", route_pattern=2, gscale13=0.37)
    pl = orc.plan(case["ids"], sh.e)
    h, out = orc.moe_grouped(case, pl, layout=layout)
    out_t, h_t = orc.moe_token(case, layout=layout, want_h=True)
    assert np.array_equal(out, out_t)
    flat_pos = pl["pos_of_pair"]
    for p, j in enumerate(flat_pos):
        t, k = divmod(p, sh.topk)
        if j < 0:
            assert np.all(np.isnan(h_t[t, k]))
        else:
            assert np.array_equal(h[j], h_t[t, k])


def test_w2_reduce_matches_numpy(orc):
    sh = S.MoEShape(m=7, e=12, topk=3, k=96, i=64)
    case = S.moe_case(sh, routing="repeat_invalid", workload="stress", route_pattern=5, gscale2=0.37)
    pl = orc.plan(case["ids"], sh.e)
    rng = np.random.default_rng(1)
    h16 = rng.standard_normal((pl["n_valid"], sh.i)).astype(np.float16)
    W2 = dq_independent(*case["w2"])
    ref = np.zeros((sh.m, sh.k))
    for t in range(sh.m):
        for k in range(sh.topk):
            j = pl["pos_of_pair"][t * sh.topk + k]
            if j >= 0:
                e = case["ids"][t, k]
                ref[t] += float(case["topk_weights"][t, k]) * (W2[e] @ h16[j].astype(np.float64))
    got = orc.w2_reduce(h16, case, pl)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    assert np.all(got[sh.m - 1] == 0)  # the last token has no valid slot


def test_nan_scale_propagates_to_its_rows_only(orc):
    rng = S.rng_for(1, 9, 0)
    codes, scales, gs = S.nvfp4_weights(rng, 1, 8, 64)
    scales = scales.copy()
    scales[0, 3, 2] = 0x7F
    x = S.activations(rng, 2, 64)
    y = orc.linear(x, (codes, scales, gs))
    assert np.all(np.isnan(y[:, 3])) and not np.any(np.isnan(np.delete(y, 3, axis=1)))
