"""gemm_nvfp4_amd: NVFP4 weight-only MoE and dense-projection kernels for MI355X (gfx950).

The compute lives in libnvfp4moe.so (HIP, C ABI in include/nvfp4moe.h); this package is its thin
Python binding. Entry points carry the C names.
"""
from ._lib import (  # noqa: F401
    FP8ChannelTensor,
    MoELayer,
    NVFP4Error,
    NVFP4Tensor,
    header_functions,
    layer_workspace_parts,
    layer_h_pair_order,
    lib,
    nvfp4_abi_version,
    nvfp4_linear,
    nvfp4_linear_fp8,
    nvfp4_linear_swiglu,
    nvfp4_moe_layer,
    NOALLOC_SCRATCH_BYTES,
    nvfp4_moe_layer_noalloc,
    nvfp4_moe_layer_workspace_bytes,
    nvfp4_moe_plan,
    nvfp4_moe_plan_bytes,
    nvfp4_moe_plan_w13_swiglu,
    nvfp4_moe_plan_w13_swiglu_with_shared,
    nvfp4_moe_route,
    nvfp4_moe_shared_expert,
    nvfp4_moe_w13_swiglu,
    nvfp4_moe_w2_reduce,
    nvfp4_moe_w2_reduce_shared,
    nvfp4_moe_w13_swiglu_with_shared,
    nvfp4_moe_w2_reduce_with_shared,
    nvfp4_moe_w2_workspace_bytes,
    nvfp4_status_str,
    plan_fields,
)
