"""The no-allocation layer call (nvfp4_moe_layer_noalloc) against the workspace-taking call it is a
variant of (nvfp4_moe_layer), through the C ABI: consecutive calls on the library's static device
scratch array, each smaller than the one before, must give bitwise the workspace call's output
(the same kernels on the same arguments). A shape whose workspace exceeds the array is refused
before anything is enqueued, and its output buffer stays untouched."""
import numpy as np
import pytest
import torch

import gemm_nvfp4_amd as G
from synth import inputs as S

pytestmark = pytest.mark.gpu


def _inputs(sh, routing, pattern, w):
    case = S.moe_case(sh, routing=routing, workload="decode", weight_set=5, route_pattern=pattern,
                      weights=(w["w13"], w["w2"]))
    return (torch.from_numpy(np.ascontiguousarray(case["ids"], np.int32)).cuda(), torch.from_numpy(case["x"]).cuda(),
            torch.from_numpy(np.ascontiguousarray(case["topk_weights"], np.float32)).cuda())


@pytest.mark.parametrize("shape", ["decode", "prefill_regime"])
def test_noalloc_layer_equals_workspace_layer(shape):
    if shape == "decode":  # 512 experts: expert-major W2 with the reduction (40, 16 tokens), token-major (1)
        e, k, i, topk, ms = 512, 2048, 512, 10, (40, 16, 1)
    else:  # 8 experts: the MFMA-tiled prefill kernels (at least 16 pairs per expert), then smaller
        e, k, i, topk, ms = 8, 256, 128, 2, (200, 64, 3)
    base = S.moe_case(S.MoEShape(m=1, e=e, topk=topk, k=k, i=i), workload="decode", weight_set=5)
    w13, w2 = G.NVFP4Tensor.from_numpy(base["w13"]), G.NVFP4Tensor.from_numpy(base["w2"])
    for n, m in enumerate(ms):
        sh = S.MoEShape(m=m, e=e, topk=topk, k=k, i=i)
        assert G.nvfp4_moe_layer_workspace_bytes(m, topk, e, k, i) <= G.NOALLOC_SCRATCH_BYTES
        ids, x, tw = _inputs(sh, "zipf" if n == 1 else "uniform", 300 + m, base)
        ref = G.nvfp4_moe_layer(ids, e, x, w13, w2, tw)
        out = torch.full((m, k), float("nan"), dtype=torch.float16, device="cuda")
        G.nvfp4_moe_layer_noalloc(ids, e, x, w13, w2, tw, out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"{shape}: call {n} (M={m})"


def test_noalloc_layer_refuses_shapes_beyond_its_array():
    e, k, i, topk, m = 512, 2048, 512, 10, 128  # about 10.6 MiB of workspace > 8 MiB
    assert G.nvfp4_moe_layer_workspace_bytes(m, topk, e, k, i) > G.NOALLOC_SCRATCH_BYTES
    base = S.moe_case(S.MoEShape(m=1, e=e, topk=topk, k=k, i=i), workload="decode", weight_set=5)
    w13, w2 = G.NVFP4Tensor.from_numpy(base["w13"]), G.NVFP4Tensor.from_numpy(base["w2"])
    ids, x, tw = _inputs(S.MoEShape(m=m, e=e, topk=topk, k=k, i=i), "uniform", 7, base)
    out = torch.full((m, k), 7.0, dtype=torch.float16, device="cuda")
    with pytest.raises(G.NVFP4Error) as err:
        G.nvfp4_moe_layer_noalloc(ids, e, x, w13, w2, tw, out)
    assert err.value.status == 4  # NVFP4_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
