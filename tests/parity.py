"""Helpers for the GPU parity tests: move seeded cases to the device, run the library, and
compare with the oracle under the acceptance rule.

Acceptance rule for floating-point outputs, per output row, in float64:
  ||gpu - ref||_2 / ||ref||_2 <= 1e-3   and   max |gpu - ref| <= 1e-2 * RMS(ref).
  A reference row that is all zero must come back as exactly +0.
  Non-finite reference values must match the GPU's NaN / +-inf pattern. The finite remainder is
  checked as above.
Error budget: the fp16 rounding of h and of the output (each at most 2^-11 relative, about 2.8e-4
RMS) plus FP32 accumulation (about sqrt(K)*2^-24). Together that is about 4e-4 RMS relative,
inside the 1e-3 bound.
"""
from __future__ import annotations

import numpy as np
import torch

REL_L2 = 1e-3
MAX_ABS_RMS = 1e-2


def assert_rows_close(gpu: np.ndarray, ref: np.ndarray, what: str = "", rel_l2: float = REL_L2,
                      max_abs_rms: float = MAX_ABS_RMS):
    gpu = np.asarray(gpu, dtype=np.float64).reshape(ref.shape[0], -1)
    ref = np.asarray(ref, dtype=np.float64).reshape(ref.shape[0], -1)
    for r in range(ref.shape[0]):
        g, f = gpu[r], ref[r]
        fin = np.isfinite(f)
        if not fin.all():
            assert np.array_equal(np.isnan(g), np.isnan(f)), f"{what} row {r}: NaN pattern differs"
            inf = np.isinf(f)
            assert np.array_equal(g[inf], f[inf]), f"{what} row {r}: inf pattern differs"
            g, f = g[fin], f[fin]
            if f.size == 0:
                continue
        if not np.any(f):
            assert np.all(g == 0) and not np.any(np.signbit(g)), f"{what} row {r}: expected exact +0"
            continue
        assert np.all(np.isfinite(g)), f"{what} row {r}: unexpected non-finite output"
        err = g - f
        rms = np.sqrt(np.mean(f * f))
        rl2 = np.linalg.norm(err) / np.linalg.norm(f)
        mab = np.abs(err).max()
        assert rl2 <= rel_l2, f"{what} row {r}: rel-L2 {rl2:.3e} > {rel_l2}"
        assert mab <= max_abs_rms * rms, f"{what} row {r}: max-abs {mab:.3e} > {max_abs_rms}*RMS {rms:.3e}"


def assert_rows_close_all(gpu: np.ndarray, ref: np.ndarray, what: str = "", rel_l2: float = REL_L2,
                          max_abs_rms: float = MAX_ABS_RMS):
    """assert_rows_close for many rows at once (the same rule, vectorised over rows). Rows with a
    non-finite or all-zero reference go through the per-row form."""
    gpu = np.asarray(gpu, dtype=np.float64).reshape(ref.shape[0], -1)
    ref = np.asarray(ref, dtype=np.float64).reshape(ref.shape[0], -1)
    special = ~np.isfinite(ref).all(axis=1) | ~np.any(ref, axis=1)
    for r in np.nonzero(special)[0]:
        assert_rows_close(gpu[r][None], ref[r][None], f"{what} row {r}", rel_l2, max_abs_rms)
    g, f = gpu[~special], ref[~special]
    rows = np.nonzero(~special)[0]
    assert np.isfinite(g).all(), f"{what}: unexpected non-finite output in row {rows[~np.isfinite(g).all(axis=1)][0]}"
    err = g - f
    rl2 = np.linalg.norm(err, axis=1) / np.linalg.norm(f, axis=1)
    mab = np.abs(err).max(axis=1) / np.sqrt(np.mean(f * f, axis=1))
    bad = np.nonzero((rl2 > rel_l2) | (mab > max_abs_rms))[0]
    assert bad.size == 0, (f"{what}: {bad.size} rows fail, first row {rows[bad[0]]}: rel-L2 {rl2[bad[0]]:.3e}, "
                           f"max-abs/RMS {mab[bad[0]]:.3e}")
    return float(rl2.max()), float(mab.max())


def half_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def to_np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def dev_moe(case, device="cuda"):
    """Device tensors of a synth.inputs.moe_case."""
    from gemm_nvfp4_amd import NVFP4Tensor
    return {
        "x": torch.from_numpy(case["x"]).to(device),
        "ids": torch.from_numpy(np.ascontiguousarray(case["ids"], dtype=np.int32)).to(device),
        "tw": torch.from_numpy(np.ascontiguousarray(case["topk_weights"], dtype=np.float32)).to(device),
        "w13": NVFP4Tensor.from_numpy(case["w13"], device),
        "w2": NVFP4Tensor.from_numpy(case["w2"], device),
    }


def run_moe(case, layout=0, dev=None, poison=True, fused=False):
    """plan -> W13 -> W2 on the GPU (fused: plan and W13 through nvfp4_moe_plan_w13_swiglu). Buffers
    are poisoned first (0x7E00 = fp16 NaN, 0xFFFF words) so that every element that must be written
    is seen to be written. Returns a dict of device tensors."""
    import gemm_nvfp4_amd as G
    sh = case["shape"]
    d = dev or dev_moe(case)
    P = sh.m * sh.topk
    plan = torch.full((max(G.nvfp4_moe_plan_bytes(sh.m, sh.topk, sh.e), 4) // 4,), -1, dtype=torch.int32,
                      device="cuda")
    h = torch.empty((P, sh.i), dtype=torch.float16, device="cuda")
    out = torch.empty((sh.m, sh.k), dtype=torch.float16, device="cuda")
    ws = torch.empty(max(G.nvfp4_moe_w2_workspace_bytes(sh.m, sh.topk, sh.k), 4), dtype=torch.uint8, device="cuda")
    if poison:
        h.view(torch.int16).fill_(0x7E00)
        out.view(torch.int16).fill_(0x7E00)
        ws.fill_(0xFF)
    if fused:
        G.nvfp4_moe_plan_w13_swiglu(d["ids"], sh.e, d["x"], d["w13"], layout, plan=plan, h=h)
    else:
        G.nvfp4_moe_plan(d["ids"], sh.e, plan=plan)
        G.nvfp4_moe_w13_swiglu(plan, sh.m, sh.topk, sh.e, d["x"], d["w13"], layout, h=h)
    G.nvfp4_moe_w2_reduce(plan, sh.m, sh.topk, sh.e, h, d["w2"], d["tw"], out=out, ws=ws)
    torch.cuda.synchronize()
    return {"plan": plan, "h": h, "out": out, "ws": ws, "dev": d}
