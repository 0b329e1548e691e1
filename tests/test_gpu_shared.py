"""GPU parity of the shared expert and shared gate against the fp64 oracle ("shared gate" among
the fused MoE parts of the "[Kernel][SM70] Improve Qwen3.8 no-MTP concurrency" page, "Scope and
related PRs"; reading: out = routed + sigmoid(x . g) * shared MLP(x), the shared term added after
the routed slots, one fp16 rounding).

Covers the shared expert's FP32 output and gate, the MoE output with the shared term in all three
W2 regimes (token-major, expert-major streaming, MFMA-tiled prefill), batch invariance, and that a
zero shared term leaves the routed output bitwise unchanged.
"""
import numpy as np
import pytest
import torch

import gemm_nvfp4_amd as G
from synth import inputs as S
from tests.parity import assert_rows_close, dev_moe, run_moe, to_np64

pytestmark = pytest.mark.gpu


def _shared_dev(shared):
    return (G.NVFP4Tensor.from_numpy(shared["w13"]), G.NVFP4Tensor.from_numpy(shared["w2"]),
            torch.from_numpy(shared["g"]).cuda())


def _run(case, shared, d=None):
    sh = case["shape"]
    res = run_moe(case, dev=d)  # plan, h (W13) and the routed-only output
    d = res["dev"]
    w13s, w2s, g = _shared_dev(shared)
    ys, sg, _ = G.nvfp4_moe_shared_expert(d["x"], w13s, w2s, g)
    out = G.nvfp4_moe_w2_reduce_shared(res["plan"], sh.m, sh.topk, sh.e, res["h"], d["w2"], d["tw"], ys, sg)
    torch.cuda.synchronize()
    return out, ys, sg, res


def test_shared_expert_outputs(orc):
    rng = S.rng_for(S.WORKLOAD_IDS["decode"], 50, 0)
    shared = S.shared_expert(rng, 2048, 512)
    x = S.activations(rng, 16, 2048)
    w13s, w2s, g = _shared_dev(shared)
    ys, sg, _ = G.nvfp4_moe_shared_expert(torch.from_numpy(x).cuda(), w13s, w2s, g)
    torch.cuda.synchronize()
    _, ys_ref = orc.gated_mlp(x, shared["w13"], shared["w2"])
    sg_ref = orc.shared_gate(x, shared["g"])
    assert_rows_close(ys.cpu().numpy().astype(np.float64), ys_ref, "shared y")
    assert np.all(np.abs(sg.cpu().numpy() - sg_ref) <= 1e-6 + 1e-5 * sg_ref)


def test_shared_gate_unaligned_gate_vector(orc):
    """A gate vector that is only 2-byte aligned takes the element-wise gate kernel (16-byte
    aligned ones take the vector loads); both match the oracle."""
    rng = S.rng_for(S.WORKLOAD_IDS["decode"], 52, 0)
    shared = S.shared_expert(rng, 2048, 256)
    x = S.activations(rng, 7, 2048)
    w13s, w2s, g = _shared_dev(shared)
    buf = torch.zeros(2048 + 8, dtype=torch.float16, device="cuda")
    g_odd = buf[1:2049]
    g_odd.copy_(g)
    assert g_odd.data_ptr() % 16 == 2
    xd = torch.from_numpy(x).cuda()
    _, sg_vec, _ = G.nvfp4_moe_shared_expert(xd, w13s, w2s, g)
    _, sg_el, _ = G.nvfp4_moe_shared_expert(xd, w13s, w2s, g_odd)
    torch.cuda.synchronize()
    sg_ref = orc.shared_gate(x, shared["g"])
    for sg in (sg_vec, sg_el):
        assert np.all(np.abs(sg.cpu().numpy() - sg_ref) <= 1e-6 + 1e-5 * sg_ref)


@pytest.mark.parametrize("shape,routing", [
    (S.MoEShape(m=5, e=512, topk=10, k=2048, i=512), "uniform"),      # token-major W2 (P <= E/4)
    (S.DECODE, "uniform"),                                             # expert-major streaming W2
    (S.MoEShape(m=600, e=8, topk=2, k=512, i=128), "repeat_invalid"),  # MFMA-tiled prefill W2
])
def test_moe_with_shared_matches_oracle(orc, shape, routing):
    case = S.moe_case(shape, routing=routing, route_pattern=31)
    shared = S.shared_expert(S.rng_for(S.WORKLOAD_IDS["decode"], 51, shape.m), shape.k, 256)
    out, _, _, _ = _run(case, shared)
    tokens = None if shape.m <= 16 else np.arange(0, shape.m, 37, dtype=np.int32)
    ref, _, _ = orc.moe_with_shared(case, shared, tokens=tokens)
    got = to_np64(out) if tokens is None else to_np64(out)[tokens]
    assert_rows_close(got, ref, f"moe+shared m={shape.m}")


def test_moe_with_shared_batch_invariance():
    case = S.moe_case(S.DECODE, route_pattern=32)
    shared = S.shared_expert(S.rng_for(S.WORKLOAD_IDS["decode"], 52, 0), S.DECODE.k, 256)
    out, _, _, res = _run(case, shared)
    for t in (0, 7, 15):
        one = dict(case)
        one["shape"] = S.MoEShape(m=1, e=S.DECODE.e, topk=S.DECODE.topk, k=S.DECODE.k, i=S.DECODE.i)
        one["x"], one["ids"], one["topk_weights"] = case["x"][t:t + 1], case["ids"][t:t + 1], case["topk_weights"][t:t + 1]
        o1, _, _, _ = _run(one, shared)
        assert torch.equal(o1[0].view(torch.int16), out[t].view(torch.int16)), t


def test_zero_shared_term_is_the_routed_output():
    case = S.moe_case(S.DECODE, route_pattern=33)
    res = run_moe(case)
    sh = S.DECODE
    zeros_y = torch.zeros((sh.m, sh.k), dtype=torch.float32, device="cuda")
    zeros_s = torch.zeros((sh.m,), dtype=torch.float32, device="cuda")
    d = res["dev"]
    out = G.nvfp4_moe_w2_reduce_shared(res["plan"], sh.m, sh.topk, sh.e, res["h"], d["w2"], d["tw"], zeros_y, zeros_s)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), res["out"].view(torch.int16))


def _run_fused(case, shared, layout=0, res=None):
    """The shared expert inside the routed W13 and W2 launches (nvfp4_moe_*_with_shared), on the
    same plan and device inputs as `res` (a run_moe result)."""
    sh = case["shape"]
    res = run_moe(case, layout) if res is None else res
    d = res["dev"]
    w13s, w2s, g = _shared_dev(shared)
    h, hs, sg = G.nvfp4_moe_w13_swiglu_with_shared(res["plan"], sh.m, sh.topk, sh.e, d["x"], d["w13"], w13s, g,
                                                   layout=layout)
    out = G.nvfp4_moe_w2_reduce_with_shared(res["plan"], sh.m, sh.topk, sh.e, h, d["w2"], d["tw"], hs, w2s, sg)
    torch.cuda.synchronize()
    return h, hs, sg, out, res


@pytest.mark.parametrize("shape,routing,i_shared,layout", [
    (S.MoEShape(m=5, e=512, topk=10, k=2048, i=512), "uniform", 512, 0),      # token-major W2: shared slot
    (S.DECODE, "uniform", 512, 0),                                             # expert-major: shared tiles
    (S.MoEShape(m=17, e=64, topk=4, k=256, i=128), "zipf", 128, 1),           # two shared tiles, 17 tokens
    (S.MoEShape(m=2, e=32, topk=4, k=2048, i=2048), "uniform", 2048, 0),      # four chunks, token-major
    (S.MoEShape(m=9, e=32, topk=4, k=2048, i=2048), "repeat_invalid", 2048, 0),  # four chunks, expert-major
    (S.DECODE, "uniform", 256, 0),                                             # shared I != I: own launches
    (S.MoEShape(m=600, e=8, topk=2, k=512, i=128), "repeat_invalid", 128, 0),  # prefill: own launches
])
def test_fused_shared_equals_separate_launches(shape, routing, i_shared, layout):
    """The one-launch forms give bitwise the separate launches' h, shared h, gate and output (and
    fall back to those launches where they do not apply)."""
    case = S.moe_case(shape, routing=routing, route_pattern=61, weights=None)
    shared = S.shared_expert(S.rng_for(S.WORKLOAD_IDS["decode"], 53, shape.m), shape.k, i_shared)
    h, hs, sg, out, res = _run_fused(case, shared, layout)
    d = res["dev"]
    w13s, w2s, g = _shared_dev(shared)
    ys_ref, sg_ref, hs_ref = G.nvfp4_moe_shared_expert(d["x"], w13s, w2s, g, layout=layout)
    out_ref = G.nvfp4_moe_w2_reduce_shared(res["plan"], shape.m, shape.topk, shape.e, res["h"], d["w2"], d["tw"],
                                           ys_ref, sg_ref)
    torch.cuda.synchronize()
    nv = int(G.plan_fields(res["plan"], shape.m, shape.topk, shape.e)["n_valid"])
    assert torch.equal(h[:nv].view(torch.int16), res["h"][:nv].view(torch.int16))
    assert torch.equal(hs.view(torch.int16), hs_ref.view(torch.int16))
    assert torch.equal(sg.view(torch.int32), sg_ref.view(torch.int32))
    assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16))


def test_fused_shared_matches_oracle(orc):
    case = S.moe_case(S.DECODE, route_pattern=62)
    shared = S.shared_expert(S.rng_for(S.WORKLOAD_IDS["decode"], 54, 0), S.DECODE.k, S.DECODE.i)
    _, _, sg, out, _ = _run_fused(case, shared)
    ref, _, _ = orc.moe_with_shared(case, shared)
    assert_rows_close(to_np64(out), ref, "fused moe+shared")
    sg_ref = orc.shared_gate(case["x"], shared["g"])
    assert np.all(np.abs(sg.cpu().numpy() - sg_ref) <= 1e-6 + 1e-5 * sg_ref)


@pytest.mark.parametrize("shape,routing,i_shared,layout", [
    (S.MoEShape(m=5, e=512, topk=10, k=2048, i=512), "uniform", 512, 0),      # one launch
    (S.DECODE, "repeat_invalid", 512, 1),                                      # one launch, bad ids
    (S.MoEShape(m=17, e=64, topk=4, k=256, i=128), "zipf", 128, 0),           # two shared tiles, one launch
    (S.MoEShape(m=26, e=512, topk=10, k=2048, i=512), "uniform", 512, 0),     # 260 pairs: plan launched first
    (S.DECODE, "uniform", 256, 0),                                             # shared I != I: own launches
])
def test_plan_in_shared_w13_launch_equals_separate_calls(shape, routing, i_shared, layout):
    """nvfp4_moe_plan_w13_swiglu_with_shared gives the plan buffer word for word and h, shared h and
    the gates bitwise as nvfp4_moe_plan followed by nvfp4_moe_w13_swiglu_with_shared."""
    case = S.moe_case(shape, routing=routing, route_pattern=67, weights=None)
    shared = S.shared_expert(S.rng_for(S.WORKLOAD_IDS["decode"], 59, shape.m), shape.k, i_shared)
    d = dev_moe(case)
    w13s, _, g = _shared_dev(shared)
    words = max(G.nvfp4_moe_plan_bytes(shape.m, shape.topk, shape.e), 4) // 4
    plan_a = torch.full((words,), -1, dtype=torch.int32, device="cuda")
    plan_b = plan_a.clone()
    _, h_a, hs_a, sg_a = G.nvfp4_moe_plan_w13_swiglu_with_shared(d["ids"], shape.e, d["x"], d["w13"], w13s, g,
                                                                layout=layout, plan=plan_a)
    G.nvfp4_moe_plan(d["ids"], shape.e, plan=plan_b)
    h_b, hs_b, sg_b = G.nvfp4_moe_w13_swiglu_with_shared(plan_b, shape.m, shape.topk, shape.e, d["x"], d["w13"],
                                                         w13s, g, layout=layout)
    torch.cuda.synchronize()
    assert torch.equal(plan_a, plan_b)
    nv = int(G.plan_fields(plan_b, shape.m, shape.topk, shape.e)["n_valid"])
    assert torch.equal(h_a[:nv].view(torch.int16), h_b[:nv].view(torch.int16))
    assert torch.equal(hs_a.view(torch.int16), hs_b.view(torch.int16))
    assert torch.equal(sg_a.view(torch.int32), sg_b.view(torch.int32))
