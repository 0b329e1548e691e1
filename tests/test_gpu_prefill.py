"""GPU parity of the prefill (MFMA-tiled) regime of the grouped MoE against the fp64 oracle.

The workload is the 8192-token, top-10 W13/W2 route of the "[Perf][SM70] Optimize Qwen3.8 Flash
Next prefill" page ("SM70 QSA indexer hotspot update"), with synthetic weights. The library picks
its MFMA-tiled kernels once experts average at least 16 pairs (M*topk >= 16*E). Every regime uses
one reduction order. So besides matching the oracle, a token's output from a prefill-size batch
must be bitwise equal to the same token run alone, which goes through the streaming kernels.
"""
import numpy as np
import pytest
import torch

from synth import inputs as S
from tests.parity import assert_rows_close, assert_rows_close_all, dev_moe, half_bits, run_moe, to_np64

pytestmark = pytest.mark.gpu


def _single_token_out(case, d, t, layout):
    sh = case["shape"]
    one = dict(case)
    one["shape"] = S.MoEShape(m=1, e=sh.e, topk=sh.topk, k=sh.k, i=sh.i)
    one["x"], one["ids"], one["topk_weights"] = case["x"][t:t + 1], case["ids"][t:t + 1], case["topk_weights"][t:t + 1]
    dd = {"x": d["x"][t:t + 1].contiguous(), "ids": d["ids"][t:t + 1].contiguous(), "tw": d["tw"][t:t + 1].contiguous(),
          "w13": d["w13"], "w2": d["w2"]}
    return run_moe(one, layout, dev=dd)["out"][0]


@pytest.mark.parametrize("routing,layout", [("uniform", 0), ("zipf", 1)])
def test_prefill_medium_multi_pass(orc, routing, layout):
    """8 experts x 600 tokens x top-2: about 150 rows per expert, i.e. several 96-row passes."""
    sh = S.MoEShape(m=600, e=8, topk=2, k=512, i=128)
    case = S.moe_case(sh, routing=routing, workload="prefill", route_pattern=7, gscale13=0.37)
    res = run_moe(case, layout)
    pl = orc.plan(case["ids"], sh.e, 16)
    h_ref, out_ref = orc.moe_grouped(case, pl, layout=layout)
    assert_rows_close(to_np64(res["h"][: pl["n_valid"]]), h_ref, "prefill medium h")
    assert_rows_close(to_np64(res["out"]), out_ref, "prefill medium out")
    for t in (0, 1, 299, 599):
        single = _single_token_out(case, res["dev"], t, layout)
        assert torch.equal(single.view(torch.int16), res["out"][t].view(torch.int16)), f"token {t}"


def test_prefill_ragged_k_and_i(orc):
    """K = 640 (a 128-element tail chunk), I = 384 (a partial last block of i slices)."""
    sh = S.MoEShape(m=200, e=4, topk=3, k=640, i=384)
    case = S.moe_case(sh, routing="repeat_invalid", workload="prefill", route_pattern=8)
    res = run_moe(case, 0)
    pl = orc.plan(case["ids"], sh.e, 16)
    h_ref, out_ref = orc.moe_grouped(case, pl)
    assert_rows_close(to_np64(res["h"][: pl["n_valid"]]), h_ref, "prefill ragged h")
    assert_rows_close(to_np64(res["out"]), out_ref, "prefill ragged out")
    assert np.all(half_bits(res["h"][pl["n_valid"]:]) == 0x7E00)
    for t in (0, 57, 199):
        single = _single_token_out(case, res["dev"], t, 0)
        assert torch.equal(single.view(torch.int16), res["out"][t].view(torch.int16)), f"token {t}"


def test_prefill_8192_tokens_full(orc):
    """Full prefill size, compared whole: the plan must be bit-exact, and every one of the 8192
    output rows and of the 81,920 h rows (every expert's bucket rows, all passes of every expert's
    MFMA tiles) must match the grouped fp64 oracle under the tolerance rule. A few tokens are also
    run alone and must be bitwise equal to their rows of the batch."""
    case = S.moe_case(S.PREFILL, workload="prefill")
    res = run_moe(case, 0)
    import gemm_nvfp4_amd as G
    got = G.plan_fields(res["plan"], S.PREFILL.m, S.PREFILL.topk, S.PREFILL.e)
    pl = orc.plan(case["ids"], S.PREFILL.e, 16)
    assert np.array_equal(got["sorted_pair"], pl["sorted_pair"])
    assert np.array_equal(got["pos_of_pair"], pl["pos_of_pair"])
    h = to_np64(res["h"][: pl["n_valid"]])
    out = to_np64(res["out"])
    h_ref, out_ref = orc.moe_grouped(case, pl)
    print(f"prefill 8192: h worst rel-L2 / max-abs-RMS {assert_rows_close_all(h, h_ref, 'prefill h')}; "
          f"out {assert_rows_close_all(out, out_ref, 'prefill out')}", flush=True)
    tokens = np.random.default_rng(4).choice(S.PREFILL.m, size=6, replace=False)
    for t in tokens:
        single = _single_token_out(case, res["dev"], int(t), 0)
        assert torch.equal(single.view(torch.int16), res["out"][int(t)].view(torch.int16)), f"token {t}"


@pytest.mark.parametrize("i", [640, 1024])
def test_prefill_multi_chunk_w2(orc, i):
    """I > 512: W2 reduces over several chunks and runs the multi-chunk prefill kernel (passes of up
    to 80 rows, chunk sums in order); I = 640 ends in a 128-element chunk. About 150 rows per
    expert: two passes each."""
    sh = S.MoEShape(m=300, e=4, topk=2, k=256, i=i)
    case = S.moe_case(sh, routing="uniform", workload="prefill", route_pattern=40 + i)
    res = run_moe(case, 0)
    pl = orc.plan(case["ids"], sh.e, 16)
    h_ref, out_ref = orc.moe_grouped(case, pl)
    assert_rows_close(to_np64(res["h"][: pl["n_valid"]]), h_ref, f"prefill I={i} h")
    assert_rows_close(to_np64(res["out"]), out_ref, f"prefill I={i} out")
    for t in (0, 149, 299):
        single = _single_token_out(case, res["dev"], t, 0)
        assert torch.equal(single.view(torch.int16), res["out"][t].view(torch.int16)), f"token {t}"
