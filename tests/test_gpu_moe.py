"""GPU parity of the grouped MoE layer (plan -> W13+SwiGLU -> W2+reduce) against the fp64 oracle.

The workloads are those of the "[Kernel][SM70] Improve Qwen3.8 no-MTP concurrency" page with
synthetic weights: the tiny case, the 16-token / 512-expert / top-10 decode ("Latest grouped-MoE
screen") and the routing-stress sweep. The page's own test list ("Test Result") includes
poisoned buffers, all-singleton, repeated and invalid experts, exact grouped W2 against native W2,
and both W13 layouts. All of them are here, plus bitwise batch invariance, token-permutation
equivariance and plan reuse.
"""
import numpy as np
import pytest
import torch

import gemm_nvfp4_amd as G
from synth import inputs as S
from tests.parity import assert_rows_close, dev_moe, half_bits, run_moe, to_np64

pytestmark = pytest.mark.gpu


def _check_against_oracle(orc, case, layout, res, what):
    sh = case["shape"]
    pl = orc.plan(case["ids"], sh.e, 16)
    h_ref, out_ref = orc.moe_grouped(case, pl, layout=layout)
    nv = pl["n_valid"]
    assert_rows_close(to_np64(res["h"][:nv]), h_ref, f"{what} h")
    assert_rows_close(to_np64(res["out"]), out_ref, f"{what} out")
    # canary: rows of h past n_valid are never written (still the 0x7E00 poison)
    assert np.all(half_bits(res["h"][nv:]) == 0x7E00), f"{what}: h rows >= n_valid were written"
    return pl


@pytest.mark.parametrize("layout", [0, 1])
def test_moe_tiny(orc, layout):
    case = S.moe_case(S.TINY, workload="tiny")
    _check_against_oracle(orc, case, layout, run_moe(case, layout), f"tiny layout={layout}")


@pytest.mark.parametrize("layout", [0, 1])
def test_moe_decode_16_tokens(orc, layout):
    case = S.moe_case(S.DECODE, workload="decode")
    _check_against_oracle(orc, case, layout, run_moe(case, layout), f"decode layout={layout}")


_STRESS_W = {}


def _stress_case(m, routing, pattern=0):
    if "w" not in _STRESS_W:
        _STRESS_W["w"] = S.moe_case(S.DECODE, workload="stress")
    base = _STRESS_W["w"]
    sh = S.MoEShape(m=m, e=512, topk=10, k=2048, i=512)
    return S.moe_case(sh, routing=routing, workload="stress", route_pattern=pattern + 17 * m,
                      weights=(base["w13"], base["w2"]))


@pytest.mark.parametrize("routing", ["zipf", "singleton", "shared", "repeat_invalid"])
@pytest.mark.parametrize("m", [1, 2, 5, 16])
def test_moe_routing_stress(orc, m, routing):
    case = _stress_case(m, routing)
    _check_against_oracle(orc, case, 0, run_moe(case, 0), f"stress m={m} {routing}")


def test_moe_w2_alone_matches_oracle_on_device_h(orc):
    """Feed the GPU's own h to the oracle's W2 + reduction ('exact grouped W2 versus native W2')."""
    case = _stress_case(16, "zipf", pattern=3)
    res = run_moe(case, 0)
    pl = orc.plan(case["ids"], 512, 16)
    h16 = res["h"][: pl["n_valid"]].cpu().numpy()
    ref = orc.w2_reduce(h16, case, pl)
    assert_rows_close(to_np64(res["out"]), ref, "w2 alone", rel_l2=5e-4, max_abs_rms=5e-3)


def test_moe_nonunit_global_scales(orc):
    case = S.moe_case(S.TINY, workload="tiny", route_pattern=9, gscale13=0.37, gscale2=1.75)
    _check_against_oracle(orc, case, 1, run_moe(case, 1), "tiny global scales")


def test_moe_batch_invariance_bitwise():
    """Each token's output in a 16-token batch equals, bitwise, a 1-token call with its own routing row."""
    case = _stress_case(16, "zipf", pattern=5)
    res = run_moe(case, 0)
    d = res["dev"]
    for t in range(16):
        single = dict(case)
        single["shape"] = S.MoEShape(m=1, e=512, topk=10, k=2048, i=512)
        single["x"], single["ids"], single["topk_weights"] = case["x"][t:t + 1], case["ids"][t:t + 1], case["topk_weights"][t:t + 1]
        dd = {"x": d["x"][t:t + 1].contiguous(), "ids": d["ids"][t:t + 1].contiguous(),
              "tw": d["tw"][t:t + 1].contiguous(), "w13": d["w13"], "w2": d["w2"]}
        one = run_moe(single, 0, dev=dd)
        assert torch.equal(one["out"][0].view(torch.int16), res["out"][t].view(torch.int16)), f"token {t}"


def test_moe_token_permutation_equivariance():
    case = _stress_case(16, "repeat_invalid", pattern=6)
    res = run_moe(case, 0)
    perm = np.random.default_rng(0).permutation(16)
    pc = dict(case)
    pc["x"], pc["ids"], pc["topk_weights"] = case["x"][perm], case["ids"][perm], case["topk_weights"][perm]
    rp = run_moe(pc, 0)
    assert torch.equal(rp["out"].view(torch.int16), res["out"][torch.from_numpy(perm).cuda()].view(torch.int16))


def test_moe_plan_reuse_and_repeat_determinism():
    """W13 and W2 run twice on one plan give identical bits (the plan is only read)."""
    case = _stress_case(8, "shared", pattern=1)
    res = run_moe(case, 0)
    sh, d = case["shape"], res["dev"]
    h2 = torch.empty_like(res["h"])
    out2 = torch.empty_like(res["out"])
    G.nvfp4_moe_w13_swiglu(res["plan"], sh.m, sh.topk, sh.e, d["x"], d["w13"], 0, h=h2)
    G.nvfp4_moe_w2_reduce(res["plan"], sh.m, sh.topk, sh.e, h2, d["w2"], d["tw"], out=out2)
    torch.cuda.synchronize()
    nv = int(res["plan"][0].item())
    assert torch.equal(h2[:nv].view(torch.int16), res["h"][:nv].view(torch.int16))
    assert torch.equal(out2.view(torch.int16), res["out"].view(torch.int16))


def test_moe_all_slots_invalid_gives_zero():
    case = _stress_case(4, "uniform", pattern=2)
    case["ids"] = np.full_like(case["ids"], -1)
    res = run_moe(case, 0)
    o = half_bits(res["out"])
    assert np.all(o == 0)


@pytest.mark.parametrize("i", [384, 640])
def test_moe_token_major_and_expert_major_w2_agree(orc, i):
    """W2 + reduce runs token-major with the reduction fused when pairs rarely share an expert
    (P <= E/4), expert-major with an FP32 workspace otherwise. A 5-token batch (P = 70 > 16) takes
    the second path, each token alone (P = 14) the first: the outputs must match bitwise, and the
    batch must match the oracle. topk = 14 leaves the four waves uneven slot counts; I = 384 is a
    short single chunk, I = 640 needs two chunks."""
    sh = S.MoEShape(m=5, e=64, topk=14, k=256, i=i)
    case = S.moe_case(sh, routing="repeat_invalid", workload="stress", route_pattern=31 + i)
    res = run_moe(case, 0)
    _check_against_oracle(orc, case, 0, res, f"w2 paths i={i}")
    d = res["dev"]
    for t in range(sh.m):
        one = dict(case)
        one["shape"] = S.MoEShape(m=1, e=sh.e, topk=sh.topk, k=sh.k, i=sh.i)
        one["x"], one["ids"], one["topk_weights"] = case["x"][t:t + 1], case["ids"][t:t + 1], case["topk_weights"][t:t + 1]
        dd = {"x": d["x"][t:t + 1].contiguous(), "ids": d["ids"][t:t + 1].contiguous(),
              "tw": d["tw"][t:t + 1].contiguous(), "w13": d["w13"], "w2": d["w2"]}
        single = run_moe(one, 0, dev=dd)["out"][0]
        assert torch.equal(single.view(torch.int16), res["out"][t].view(torch.int16)), f"token {t}"


@pytest.mark.parametrize("m", [2, 9])
def test_moe_maximum_reduction_lengths(orc, m):
    """K = I = 2048, the largest reduction lengths the grouped GEMMs accept: W13 and W2 both split
    into four 512-element chunks. m = 2 (P = 8 <= E/4) runs W2 token-major, m = 9 (P = 36)
    expert-major with the four-way intra-block split; both must match the oracle and each token
    alone, bitwise."""
    sh = S.MoEShape(m=m, e=32, topk=4, k=2048, i=2048)
    case = S.moe_case(sh, routing="uniform", workload="stress", route_pattern=70 + m)
    res = run_moe(case, 0)
    _check_against_oracle(orc, case, 0, res, f"max K/I m={m}")
    d = res["dev"]
    for t in (0, m - 1):
        one = dict(case)
        one["shape"] = S.MoEShape(m=1, e=sh.e, topk=sh.topk, k=sh.k, i=sh.i)
        one["x"], one["ids"], one["topk_weights"] = case["x"][t:t + 1], case["ids"][t:t + 1], case["topk_weights"][t:t + 1]
        dd = {"x": d["x"][t:t + 1].contiguous(), "ids": d["ids"][t:t + 1].contiguous(),
              "tw": d["tw"][t:t + 1].contiguous(), "w13": d["w13"], "w2": d["w2"]}
        single = run_moe(one, 0, dev=dd)["out"][0]
        assert torch.equal(single.view(torch.int16), res["out"][t].view(torch.int16)), f"token {t}"


def test_moe_general_negative_subnormal_and_nan_scales(orc):
    """Block scales beyond powers of two: E4M3 bytes with mantissa bits, negative and subnormal
    ones (0x01..0x30 and their negatives). A NaN scale (0x7F) in one W2 row makes that output column
    NaN and nothing else; a NaN scale in a W13 gate row makes the token's whole output NaN (its h row
    feeds every W2 row). NaN propagates by IEEE rules, as in the oracle."""
    sb = np.array([b for b in range(0x01, 0x31)] + [0x80 | b for b in range(0x01, 0x31)], dtype=np.uint8)
    case = S.moe_case(S.TINY, workload="tiny", route_pattern=11, scale_bytes=sb)
    e0, e1 = int(case["ids"][0, 0]), int(case["ids"][0, 1])
    assert e0 != e1 and e0 >= 0 and e1 >= 0
    w2c, w2s, w2g = case["w2"]
    w2s = w2s.copy()
    w2s[e1, 5, 3] = 0x7F  # W2 row 5 of the second slot's expert
    case = dict(case, w2=(w2c, w2s, w2g))
    res = run_moe(case, 0)
    pl = orc.plan(case["ids"], S.TINY.e, 16)
    h_ref, out_ref = orc.moe_grouped(case, pl)
    out = to_np64(res["out"])
    assert np.isnan(out[0, 5]) and np.isnan(out_ref[0, 5])
    assert np.isfinite(np.delete(out[0], 5)).all()
    assert_rows_close(to_np64(res["h"][: pl["n_valid"]]), h_ref, "general scales h")
    assert_rows_close(out, out_ref, "general scales out (NaN column)")
    # NaN in a W13 gate row of the first slot's expert
    w13c, w13s, w13g = case["w13"]
    w13s = w13s.copy()
    w13s[e0, 7, 2] = 0x7F
    case2 = dict(case, w13=(w13c, w13s, w13g), w2=(w2c, case["w2"][1].copy(), w2g))
    case2["w2"][1][e1, 5, 3] = 0x08
    res2 = run_moe(case2, 0)
    h2_ref, out2_ref = orc.moe_grouped(case2, orc.plan(case2["ids"], S.TINY.e, 16))
    assert np.isnan(to_np64(res2["out"])).all() and np.isnan(out2_ref).all()
    assert_rows_close(to_np64(res2["h"][: pl["n_valid"]]), h2_ref, "NaN gate row h")
