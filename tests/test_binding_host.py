"""The Python binding's own checks, on the CPU: every wrapper compares the tensors it is given with
the sizes the library will read and write, and raises before calling the library (whose W13/W2 calls
take no plan size, so a short buffer would otherwise be read out of bounds). CPU tensors are used on
purpose: the shape checks run before the device checks, which would reject them next."""
import pytest
import torch

import gemm_nvfp4_amd as G
from gemm_nvfp4_amd._lib import NVFP4Tensor


def _w(groups, rows, k):
    return NVFP4Tensor(torch.zeros((groups, rows, k // 2), dtype=torch.uint8),
                       torch.zeros((groups, rows, k // 16), dtype=torch.uint8), torch.ones(groups))


def _f16(*shape):
    return torch.zeros(shape, dtype=torch.float16)


E, K, I, M, TOPK = 8, 256, 128, 4, 2
W13, W2 = _w(E, 2 * I, K), _w(E, K, I)


def _plan(m=M, topk=TOPK):
    return torch.zeros(G.nvfp4_moe_plan_bytes(m, topk, E) // 4, dtype=torch.int32)


def _raises_shape(fn, what):
    with pytest.raises(ValueError, match=what):
        fn()


def test_w13_checks():
    ids = torch.zeros((M, TOPK), dtype=torch.int32)
    _raises_shape(lambda: G.nvfp4_moe_w13_swiglu(_plan(), M, TOPK, E, _f16(M, K + 128), W13), "x must have shape")
    _raises_shape(lambda: G.nvfp4_moe_w13_swiglu(_plan()[:-64], M, TOPK, E, _f16(M, K), W13), "plan holds")
    _raises_shape(lambda: G.nvfp4_moe_w13_swiglu(_plan(), M, TOPK, E, _f16(M, K), W13, h=_f16(M * TOPK - 1, I)),
                  "h must have shape")
    _raises_shape(lambda: G.nvfp4_moe_plan_w13_swiglu(ids, E, _f16(M + 1, K), W13), "x must have shape")
    _raises_shape(lambda: G.nvfp4_moe_plan_w13_swiglu(ids, E, _f16(M, K), W13, h=_f16(M * TOPK, I // 2)),
                  "h must have shape")


def test_w2_checks():
    h, tw = _f16(M * TOPK, I), torch.zeros((M, TOPK))
    _raises_shape(lambda: G.nvfp4_moe_w2_reduce(_plan()[:8], M, TOPK, E, h, W2, tw), "plan holds")
    _raises_shape(lambda: G.nvfp4_moe_w2_reduce(_plan(), M, TOPK, E, _f16(M * TOPK, I + 128), W2, tw),
                  "h must have shape")
    _raises_shape(lambda: G.nvfp4_moe_w2_reduce(_plan(), M, TOPK, E, h, W2, torch.zeros((M, TOPK + 1))),
                  "topk_weights must have shape")
    _raises_shape(lambda: G.nvfp4_moe_w2_reduce(_plan(), M, TOPK, E, h, W2, tw, out=_f16(M, K - 16)),
                  "out must have shape")


def test_dense_and_shared_checks():
    w = _w(1, 64, 256)
    _raises_shape(lambda: G.nvfp4_linear(_f16(3, 384), w), "x must have shape")
    _raises_shape(lambda: G.nvfp4_linear(_f16(3, 256), w, y=_f16(3, 48)), "y must have shape")
    _raises_shape(lambda: G.nvfp4_linear_swiglu(_f16(3, 256), w, h=_f16(3, 64)), "h must have shape")
    _raises_shape(lambda: G.nvfp4_linear_ws(_f16(3, 256), w, ws=torch.zeros(64, dtype=torch.uint8)), "ws holds")
    _raises_shape(lambda: G.nvfp4_linear_swiglu_ws(_f16(3, 256), w, ws=torch.zeros(64, dtype=torch.uint8)), "ws holds")
    s13, s2 = _w(1, 2 * I, K), _w(1, K, I)
    _raises_shape(lambda: G.nvfp4_moe_shared_expert(_f16(M, K), s13, s2, _f16(K + 8)), "gate must have shape")
    _raises_shape(lambda: G.nvfp4_moe_shared_expert(_f16(M, K), s13, s2, _f16(K), h=_f16(M, I + 16)),
                  "h must have shape")


def test_layer_checks():
    ids, tw = torch.zeros((M, TOPK), dtype=torch.int32), torch.zeros((M, TOPK))
    _raises_shape(lambda: G.nvfp4_moe_layer(ids, E, _f16(M, K), W13, W2, tw, ws=torch.zeros(64, dtype=torch.uint8)),
                  "ws holds")
    _raises_shape(lambda: G.nvfp4_moe_layer(ids, E, _f16(M, K + 128), W13, W2, tw), "x must have shape")
    layer = G.MoELayer(M, TOPK, W13, W2, device="cpu")
    h_off, w2_off = G.layer_workspace_parts(M, TOPK, E, I)
    assert layer.plan.numel() * 4 == h_off and layer.h.shape == (M * TOPK, I)
    assert layer.ws.numel() == G.nvfp4_moe_w2_workspace_bytes(M, TOPK, K)
    with pytest.raises(ValueError, match="override must have the layer's shape"):
        layer(_f16(M, K), ids, tw, w13=_w(E, 2 * I, 2 * K))
    with pytest.raises(ValueError, match="override must have the layer's shape"):
        layer(_f16(M, K), ids, tw, w2=_w(E + 1, K, I))
    _raises_shape(lambda: layer(_f16(M, K), torch.zeros((M + 1, TOPK), dtype=torch.int32), tw),
                  "topk_ids must have shape")
    with pytest.raises(ValueError, match="w2 must be"):
        G.MoELayer(M, TOPK, W13, _w(E, K, 2 * I), device="cpu")
