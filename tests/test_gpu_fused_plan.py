"""GPU tests of nvfp4_moe_plan_w13_swiglu: the routing plan built inside the W13 launch.

The call must give exactly what nvfp4_moe_plan followed by nvfp4_moe_w13_swiglu gives (the plan is
the integer plan that W13 and W2 share, "[Kernel][SM70] Improve Qwen3.8 no-MTP concurrency",
"Scope and related PRs"): the whole plan buffer word for word (both start from the same poison, so
words neither writes stay equal too), h bitwise and the layer output bitwise, and the oracle's
results within the tolerance rule. Cases: the tiny layer, the routing-stress cases around the
one-launch limit of 256 pairs (25 tokens: 250 pairs, one launch; 26: 260 pairs, plan and W13
launched separately), and ids outside [-1, E), which are skipped and counted.
"""
import numpy as np
import pytest
import torch

from synth import inputs as S
from tests.parity import assert_rows_close, dev_moe, half_bits, run_moe, to_np64

pytestmark = pytest.mark.gpu

_W = {}


def _case(m, routing, pattern=0):
    if "w" not in _W:
        _W["w"] = S.moe_case(S.DECODE, workload="stress")
    base = _W["w"]
    sh = S.MoEShape(m=m, e=512, topk=10, k=2048, i=512)
    return S.moe_case(sh, routing=routing, workload="stress", route_pattern=pattern + 31 * m,
                      weights=(base["w13"], base["w2"]))


def _dev(case):
    """Device tensors of a stress case, with the 512-expert weights uploaded once."""
    if "dev" not in _W:
        _W["dev"] = dev_moe(case)
    d = dict(_W["dev"])
    small = dev_moe(dict(case, w13=S.moe_case(S.TINY, workload="tiny")["w13"],
                         w2=S.moe_case(S.TINY, workload="tiny")["w2"]))
    d.update(x=small["x"], ids=small["ids"], tw=small["tw"])
    return d


def _assert_same(a, b, what):
    assert torch.equal(a["plan"], b["plan"]), f"{what}: plan buffers differ"
    assert np.array_equal(half_bits(a["h"]), half_bits(b["h"])), f"{what}: h differs"
    assert np.array_equal(half_bits(a["out"]), half_bits(b["out"])), f"{what}: out differs"


@pytest.mark.parametrize("layout", [0, 1])
def test_fused_plan_tiny(orc, layout):
    case = S.moe_case(S.TINY, workload="tiny", route_pattern=5)
    fused, sep = run_moe(case, layout, fused=True), run_moe(case, layout)
    _assert_same(fused, sep, f"tiny layout={layout}")
    pl = orc.plan(case["ids"], S.TINY.e, 16)
    h_ref, out_ref = orc.moe_grouped(case, pl, layout=layout)
    assert_rows_close(to_np64(fused["h"][: pl["n_valid"]]), h_ref, "fused tiny h")
    assert_rows_close(to_np64(fused["out"]), out_ref, "fused tiny out")


@pytest.mark.parametrize("routing", ["uniform", "zipf", "singleton", "shared", "repeat_invalid"])
@pytest.mark.parametrize("m", [1, 5, 16, 25, 26])
def test_fused_plan_equals_separate_calls(m, routing):
    case = _case(m, routing)
    d = _dev(case)
    _assert_same(run_moe(case, 0, dev=d, fused=True), run_moe(case, 0, dev=d), f"m={m} {routing}")


@pytest.mark.parametrize("m,routing", [(16, "uniform"), (25, "repeat_invalid")])
def test_fused_plan_matches_oracle(orc, m, routing):
    case = _case(m, routing, pattern=7)
    res = run_moe(case, 0, dev=_dev(case), fused=True)
    pl = orc.plan(case["ids"], 512, 16)
    h_ref, out_ref = orc.moe_grouped(case, pl)
    nv = pl["n_valid"]
    assert_rows_close(to_np64(res["h"][:nv]), h_ref, f"fused m={m} h")
    assert_rows_close(to_np64(res["out"]), out_ref, f"fused m={m} out")
    assert np.all(half_bits(res["h"][nv:]) == 0x7E00), "h rows >= n_valid were written"


def test_fused_plan_skips_and_counts_bad_ids():
    case = _case(12, "uniform", pattern=3)
    ids = case["ids"].copy()
    ids[0, 3] = 512        # == E
    ids[4, 0] = 9999
    ids[7, 9] = -7
    ids[11, 2] = -1        # skipped, not counted
    case = dict(case, ids=ids)
    d = _dev(case)
    fused, sep = run_moe(case, 0, dev=d, fused=True), run_moe(case, 0, dev=d)
    _assert_same(fused, sep, "bad ids")
    assert int(fused["plan"][2].item()) == 3, "status word: three ids outside [-1, E)"
