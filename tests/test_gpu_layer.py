"""GPU checks of the whole-layer call (nvfp4_moe_layer): one library call that enqueues the plan,
grouped W13 + SwiGLU and grouped W2 + the slot-order reduction (the grouped-MoE complete call timed on
the "[Kernel][SM70] Improve Qwen3.8 no-MTP concurrency" page, "Latest grouped-MoE screen").

Its output, and the plan and h it leaves in the workspace, must be bitwise those of the separate
calls (nvfp4_moe_plan_w13_swiglu, then nvfp4_moe_w2_reduce) in every regime: the pair-major path
(1, 4 and 12 tokens: W13 straight from the ids with h in pair order, token-major W2 on that h),
the plan built inside W13 with expert-major W2 and the reduction launch (16 and 40 tokens), the
separate plan launch (30 tokens: 300 pairs), and the MFMA-tiled prefill kernels (1024 tokens). The
16-token case is also compared with the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import gemm_nvfp4_amd as G
from synth import inputs as S
from tests.parity import assert_rows_close, dev_moe, run_moe, to_np64

pytestmark = pytest.mark.gpu

_W = {}


def _case(m, routing="uniform", pattern=0):
    if "w" not in _W:
        _W["w"] = S.moe_case(S.DECODE, workload="decode", weight_set=3)
    base = _W["w"]
    sh = S.MoEShape(m=m, e=512, topk=10, k=2048, i=512)
    case = S.moe_case(sh, routing=routing, workload="decode", weight_set=3, route_pattern=100 + m + pattern,
                      weights=(base["w13"], base["w2"]))
    if "dev" not in _W:
        _W["dev"] = dev_moe(case)
    d = dict(_W["dev"])
    d.update(x=torch.from_numpy(case["x"]).cuda(),
             ids=torch.from_numpy(np.ascontiguousarray(case["ids"], np.int32)).cuda(),
             tw=torch.from_numpy(np.ascontiguousarray(case["topk_weights"], np.float32)).cuda())
    return case, d


@pytest.mark.parametrize("m,routing", [(1, "uniform"), (4, "repeat_invalid"), (12, "zipf"), (16, "uniform"),
                                       (30, "zipf"), (40, "repeat_invalid"), (1024, "uniform")])
def test_layer_call_equals_separate_calls(m, routing):
    case, d = _case(m, routing)
    sep = run_moe(case, 0, dev=d, fused=True)
    ws_bytes = G.nvfp4_moe_layer_workspace_bytes(m, 10, 512, 2048, 512)
    ws = torch.full((ws_bytes,), 0xEE, dtype=torch.uint8, device="cuda")
    out = torch.full((m, 2048), float("nan"), dtype=torch.float16, device="cuda")
    G.nvfp4_moe_layer(d["ids"], 512, d["x"], d["w13"], d["w2"], d["tw"], out=out, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), sep["out"].view(torch.int16)), f"out, m={m}"
    h_off, _ = G.layer_workspace_parts(m, 10, 512, 512)
    got = G.plan_fields(ws[:h_off].view(torch.int32), m, 10, 512)
    ref = G.plan_fields(sep["plan"], m, 10, 512)
    for name in ("sorted_pair", "pos_of_pair", "counts", "offsets", "active", "tile_base", "tile_rows"):
        assert np.array_equal(got[name], ref[name]), f"plan {name}, m={m}"
    nv = ref["n_valid"]
    h = ws[h_off:h_off + m * 10 * 512 * 2].view(torch.float16).view(m * 10, 512)
    if G.layer_h_pair_order(m, 10, 512):  # pair-major path: row p is pair p's h
        pos = torch.from_numpy(ref["pos_of_pair"].astype(np.int64)).cuda()
        valid = pos >= 0
        assert int(valid.sum()) == nv
        assert torch.equal(h[valid].view(torch.int16), sep["h"][pos[valid]].view(torch.int16)), f"h, m={m}"
    else:
        assert torch.equal(h[:nv].view(torch.int16), sep["h"][:nv].view(torch.int16)), f"h, m={m}"


def _layer(d, m):
    ws = torch.empty((G.nvfp4_moe_layer_workspace_bytes(m, 10, 512, 2048, 512),), dtype=torch.uint8, device="cuda")
    out = torch.full((m, 2048), float("nan"), dtype=torch.float16, device="cuda")
    G.nvfp4_moe_layer(d["ids"], 512, d["x"], d["w13"], d["w2"], d["tw"], out=out, ws=ws)
    return out


@pytest.mark.parametrize("m,routing", [(2, "zipf"), (3, "uniform"), (8, "repeat_invalid")])
def test_layer_small_batch_equals_tokens_alone(m, routing):
    """Each token of a small batch equals, bitwise, the layer on that token alone. One token runs
    the token-major W2 with one slot chain per wave (12-wave blocks), three tokens and more with
    three chains per wave (4-wave blocks), so this also pins the two block shapes to each other."""
    case, d = _case(m, routing, pattern=7)
    out = _layer(d, m)
    for t in range(m):
        dt = dict(d)
        dt.update(x=d["x"][t:t + 1].contiguous(), ids=d["ids"][t:t + 1].contiguous(), tw=d["tw"][t:t + 1].contiguous())
        one = _layer(dt, 1)
        torch.cuda.synchronize()
        assert torch.equal(one[0].view(torch.int16), out[t].view(torch.int16)), f"m={m} token {t}"


@pytest.mark.parametrize("m,routing", [(4, "repeat_invalid"), (16, "uniform")])
def test_layer_call_against_oracle(orc, m, routing):
    case, d = _case(m, routing)
    out = G.nvfp4_moe_layer(d["ids"], 512, d["x"], d["w13"], d["w2"], d["tw"])
    torch.cuda.synchronize()
    pl = orc.plan(case["ids"], 512, 16)
    _, out_ref = orc.moe_grouped(case, pl)
    assert_rows_close(to_np64(out), out_ref, "layer call out")


def test_layer_object_reuses_its_workspace():
    """MoELayer runs nvfp4_moe_layer on one workspace; its plan and h views hold the call's plan and
    h, and repeated calls on new inputs equal fresh calls bitwise."""
    case, d = _case(16)
    layer = G.MoELayer(16, 10, d["w13"], d["w2"])
    for p in range(3):
        c2, d2 = _case(16, pattern=10 + p)
        got = layer(d2["x"], d2["ids"], d2["tw"]).clone()
        ref = G.nvfp4_moe_layer(d2["ids"], 512, d2["x"], d2["w13"], d2["w2"], d2["tw"])
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
        f = G.plan_fields(layer.plan, 16, 10, 512)
        assert f["n_valid"] == int(((c2["ids"] >= 0) & (c2["ids"] < 512)).sum())


def test_layer_workspace_reused_across_shapes():
    """One workspace sized for the largest call serves calls of other token counts in turn, in every
    regime of the decode layer (token-major W2 at 1 token, expert-major at 16 to 64): each output
    equals that of a fresh workspace."""
    sizes = (40, 16, 64, 1, 24)
    need = max(G.nvfp4_moe_layer_workspace_bytes(m, 10, 512, 2048, 512) for m in sizes)
    ws = torch.full((need,), 0xEE, dtype=torch.uint8, device="cuda")
    for m in sizes:
        case, d = _case(m, pattern=7)
        got = G.nvfp4_moe_layer(d["ids"], 512, d["x"], d["w13"], d["w2"], d["tw"], ws=ws).clone()
        ref = G.nvfp4_moe_layer(d["ids"], 512, d["x"], d["w13"], d["w2"], d["tw"])
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"m={m}"
