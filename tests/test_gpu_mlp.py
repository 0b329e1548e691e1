"""GPU parity of the dense NVFP4 gated MLP: the packed gate/up projection with SwiGLU fused
(nvfp4_linear_swiglu), then the down projection (nvfp4_linear) on its h ("[SM70][Draft] Extend
Qwen3.8 DFlash2 concurrency paths", "TP4-only NVFP4 verifier follow-up": gate/up and down of the
packed MLP weights, M <= 32).

The MLP shard has hidden size 5120 and 2176 intermediate columns: its packed gate/up weight is the
4352 x 5120 projection of the dense workload. h and the MLP output are checked against the fp64
oracle by the per-row tolerance rule; batches must be bitwise equal to single rows; and h must
equal the grouped W13 of a one-expert top-1 MoE bitwise (one arithmetic for both).
"""
import numpy as np
import pytest
import torch

import gemm_nvfp4_amd as G
from synth import inputs as S
from tests.parity import assert_rows_close, dev_moe, to_np64

pytestmark = pytest.mark.gpu

K, I, N = S.DENSE_K, S.DENSE_N // 2, S.DENSE_K


def _weights(seed, k=K, i=I, n=N, gscale=1.0):
    rng = S.rng_for(S.WORKLOAD_IDS["dense"], 60 + seed, 0)
    return S.nvfp4_weights(rng, 1, 2 * i, k, gscale=gscale), S.nvfp4_weights(rng, 1, n, i, gscale=gscale)


@pytest.mark.parametrize("M", [1, 8, 16, 17, 32])
def test_gated_mlp_matches_oracle(orc, M):
    w13, w2 = _weights(0)
    x = S.activations(S.rng_for(S.WORKLOAD_IDS["dense"], 61, M), M, K)
    h = G.nvfp4_linear_swiglu(torch.from_numpy(x).cuda(), G.NVFP4Tensor.from_numpy(w13))
    y = G.nvfp4_linear(h, G.NVFP4Tensor.from_numpy(w2))
    torch.cuda.synchronize()
    h_ref, y_ref = orc.gated_mlp(x, w13, w2)
    assert_rows_close(to_np64(h), h_ref, f"mlp h M={M}")
    assert_rows_close(to_np64(y), y_ref, f"mlp y M={M}")


def test_gated_interleaved_layout_and_global_scale(orc):
    w13, w2 = _weights(1, k=640, i=96, n=128, gscale=0.37)
    x = S.activations(S.rng_for(S.WORKLOAD_IDS["dense"], 62, 0), 5, 640)
    for layout in (0, 1):
        h = G.nvfp4_linear_swiglu(torch.from_numpy(x).cuda(), G.NVFP4Tensor.from_numpy(w13), layout=layout)
        torch.cuda.synchronize()
        h_ref, _ = orc.gated_mlp(x, w13, w2, layout)
        assert_rows_close(to_np64(h), h_ref, f"mlp h layout={layout}")


def test_gated_batch_invariance():
    w13, _ = _weights(2)
    x = torch.from_numpy(S.activations(S.rng_for(S.WORKLOAD_IDS["dense"], 63, 0), 32, K)).cuda()
    W = G.NVFP4Tensor.from_numpy(w13)
    h = G.nvfp4_linear_swiglu(x, W)
    for m in (0, 9, 31):
        h1 = G.nvfp4_linear_swiglu(x[m:m + 1].contiguous(), W)
        assert torch.equal(h1[0].view(torch.int16), h[m].view(torch.int16)), m
    h8 = torch.cat([G.nvfp4_linear_swiglu(x[r:r + 8].contiguous(), W) for r in range(0, 32, 8)])
    assert torch.equal(h8.view(torch.int16), h.view(torch.int16))


@pytest.mark.parametrize("M", [8, 32])
def test_gated_equals_one_expert_moe_w13_bitwise(M):
    """Streaming (M=8) and MFMA-tiled (M=32) MoE regimes both reproduce the dense gated form."""
    sh = S.MoEShape(m=M, e=1, topk=1, k=2048, i=512)
    case = S.moe_case(sh, workload="tiny", route_pattern=M)
    case["ids"] = np.zeros((M, 1), np.int32)
    d = dev_moe(case)
    for layout in (0, 1):
        plan = G.nvfp4_moe_plan(d["ids"], 1)
        h_moe = G.nvfp4_moe_w13_swiglu(plan, M, 1, 1, d["x"], d["w13"], layout=layout)
        h = G.nvfp4_linear_swiglu(d["x"], G.NVFP4Tensor.from_numpy(case["w13"]), layout=layout)
        torch.cuda.synchronize()
        assert torch.equal(h.view(torch.int16), h_moe.view(torch.int16)), layout


def test_gated_zero_rows():
    w13, _ = _weights(3, k=256, i=32, n=64)
    h = G.nvfp4_linear_swiglu(torch.zeros((0, 256), dtype=torch.float16, device="cuda"), G.NVFP4Tensor.from_numpy(w13))
    assert h.shape == (0, 32)


@pytest.mark.parametrize("M,layout", [(16, 0), (33, 1), (12, 1)])
def test_gated_split_k_bitwise_equals_one_launch(M, layout):
    """nvfp4_linear_swiglu_ws folds the gate and up partials with the one-launch epilogue: h is
    bitwise the same, in both layouts (33 rows take two staging passes)."""
    w13, _ = _weights(3)
    x = torch.from_numpy(S.activations(S.rng_for(S.WORKLOAD_IDS["dense"], 64, M), M, K)).cuda()
    wt = G.NVFP4Tensor.from_numpy(w13)
    ws = torch.full((G.nvfp4_linear_ws_bytes(M, 2 * I, K),), 0xFF, dtype=torch.uint8, device="cuda")
    one = G.nvfp4_linear_swiglu(x, wt, layout)
    split = G.nvfp4_linear_swiglu_ws(x, wt, layout, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), split.view(torch.int16))
