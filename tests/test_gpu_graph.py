"""HIP-graph replays of the MoE layer: every entry point only enqueues work (no allocation, no
host synchronisation, no memset node), so a captured layer must give, on every replay, bitwise the
result of the same calls run eagerly, also when other calls have overwritten the layer's plan, h
and workspace buffers between replays. Covered: the decode layer with the plan built in the W13
launch (1 and 16 tokens), the layer with a shared expert in the routed launches, and a prefill-size
layer (plan in four launches, MFMA kernels)."""
import pytest
import torch

import gemm_nvfp4_amd as G
from synth import inputs as S
from tests.parity import dev_moe

pytestmark = pytest.mark.gpu

_W = {}


def _weights():
    if "d" not in _W:
        _W["d"] = dev_moe(S.moe_case(S.DECODE, workload="stress"))
    return _W["d"]


def _routes(m, n, seed, e=512):
    out = []
    for p in range(n):
        c = S.moe_case(S.MoEShape(m=m, e=e, topk=10, k=2048, i=512), routing="uniform", workload="stress",
                       route_pattern=seed + p, weights=(None, None))
        out.append((torch.from_numpy(c["x"]).cuda(), torch.from_numpy(c["ids"].astype("int32")).cuda(),
                    torch.from_numpy(c["topk_weights"]).cuda()))
    return out


def _check_replays(run_calls, n_outs, disturb):
    """run_calls(outs) enqueues the calls and copies each call's output into outs[i]."""
    eager = [None] * n_outs
    run_calls(eager)
    torch.cuda.synchronize()
    eager = [t.clone() for t in eager]
    outs = [torch.empty_like(t) for t in eager]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_calls(outs)
    for rep in range(3):
        for t in outs:
            t.zero_()
        disturb()  # eager calls that overwrite the layer's buffers
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(n_outs):
            assert torch.equal(outs[i].view(torch.int16), eager[i].view(torch.int16)), f"replay {rep}, call {i}"
    del g


@pytest.mark.parametrize("m", [1, 16])
def test_decode_layer_graph_replays(m):
    d = _weights()
    layer = G.MoELayer(m, 10, d["w13"], d["w2"])
    routes = _routes(m, 3, 700 + m)
    other = _routes(m, 1, 900 + m)[0]

    def run_calls(outs):
        for i, (x, ids, tw) in enumerate(routes):
            out = layer(x, ids, tw)
            if outs[i] is None:
                outs[i] = out.clone()
            else:
                outs[i].copy_(out)

    _check_replays(run_calls, len(routes), lambda: layer(*other))


def test_shared_expert_layer_graph_replays():
    d = _weights()
    m, I = 16, 512
    sh = S.shared_expert(S.rng_for(S.WORKLOAD_IDS["decode"], 71, m), 2048, I)
    w13s, w2s = G.NVFP4Tensor.from_numpy(sh["w13"]), G.NVFP4Tensor.from_numpy(sh["w2"])
    gate = torch.from_numpy(sh["g"]).cuda()
    routes = _routes(m, 2, 800)
    plan = torch.empty(G.nvfp4_moe_plan_bytes(m, 10, 512) // 4, dtype=torch.int32, device="cuda")
    h = torch.empty((m * 10, I), dtype=torch.float16, device="cuda")
    hs = torch.empty((m, I), dtype=torch.float16, device="cuda")
    sg = torch.empty((m,), dtype=torch.float32, device="cuda")
    ys = torch.empty((m, 2048), dtype=torch.float32, device="cuda")
    ws = torch.empty(G.nvfp4_moe_w2_workspace_bytes(m, 10, 2048), dtype=torch.uint8, device="cuda")
    out = torch.empty((m, 2048), dtype=torch.float16, device="cuda")

    def layer(x, ids, tw):
        G.nvfp4_moe_plan_w13_swiglu_with_shared(ids, 512, x, d["w13"], w13s, gate, plan=plan, h=h, shared_h=hs,
                                                shared_sigma=sg)
        G.nvfp4_moe_w2_reduce_with_shared(plan, m, 10, 512, h, d["w2"], tw, hs, w2s, sg, shared_y=ys, out=out, ws=ws)
        return out

    def run_calls(outs):
        for i, r in enumerate(routes):
            o = layer(*r)
            if outs[i] is None:
                outs[i] = o.clone()
            else:
                outs[i].copy_(o)

    other = _routes(m, 1, 950)[0]
    _check_replays(run_calls, len(routes), lambda: layer(*other))


def test_prefill_layer_graph_replays():
    d = _weights()
    m = 1024  # 10240 pairs over 512 experts: 20 per expert, the MFMA regime, plan in four launches
    layer = G.MoELayer(m, 10, d["w13"], d["w2"])
    routes = _routes(m, 2, 600)

    def run_calls(outs):
        for i, r in enumerate(routes):
            o = layer(*r)
            if outs[i] is None:
                outs[i] = o.clone()
            else:
                outs[i].copy_(o)

    _check_replays(run_calls, len(routes), lambda: layer(*routes[1]))


@pytest.mark.parametrize("m", [1, 16, 1024])
def test_graph_replay_with_new_routing_and_activations(m):
    """A captured layer reads its inputs from the captured buffers: after new ids, routing weights
    and activations are copied into them in place, a replay gives bitwise the eager result for the
    new inputs (decode with the plan in W13, and the prefill regime)."""
    d = _weights()
    layer = G.MoELayer(m, 10, d["w13"], d["w2"])
    routes = _routes(m, 4, 500 + m)
    x, ids, tw = (t.clone() for t in routes[0])
    out = torch.empty((m, 2048), dtype=torch.float16, device="cuda")
    layer(x, ids, tw)  # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out.copy_(layer(x, ids, tw))
    for i in range(1, 4):
        xn, idn, twn = routes[i]
        ref = layer(xn, idn, twn).clone()  # eager, on the new inputs
        x.copy_(xn)
        ids.copy_(idn)
        tw.copy_(twn)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay with routes[{i}]"
    del g
