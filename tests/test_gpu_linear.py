"""GPU parity of the dense NVFP4 projection against the fp64 oracle.

Covers the 4352 x 5120 projection at M = 1..32, an integer-exact case (bitwise), batch
invariance, and the split-K form (nvfp4_linear_ws) bitwise against the one-launch form. A batch must be bitwise equal to single-row calls and to concatenated 8-row calls
(the verifier check on the "[SM70][Draft] Extend Qwen3.8 DFlash2 concurrency paths" page). It
also covers ragged K and M, a non-unit global scale, NaN propagation and M = 0.
"""
import numpy as np
import pytest
import torch

import gemm_nvfp4_amd as G
from synth import inputs as S
from tests.parity import assert_rows_close, to_np64

pytestmark = pytest.mark.gpu


def _run(x, w):
    y = G.nvfp4_linear(torch.from_numpy(x).cuda(), G.NVFP4Tensor.from_numpy(w))
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("M", S.DENSE_MS)
def test_linear_dense_projection(orc, M):
    case = S.dense_case(M)
    y = _run(case["x"], case["w"])
    ref = orc.linear(case["x"], case["w"])
    assert_rows_close(to_np64(y), ref, f"linear M={M}")


@pytest.mark.parametrize("N,K,M", [(64, 640, 19), (32, 128, 1), (48, 384, 33), (16, 1536, 50)])
def test_linear_integer_exact(orc, N, K, M):
    """Scale bytes 0x38 (=1.0), global 1, x in {-1,0,1}: every partial sum is a multiple of 0.5 and
    every |y| < 1024, so FP32 accumulation and the fp16 output are exact and the GPU must equal
    the oracle bitwise."""
    rng = np.random.default_rng(N * K + M)
    codes = rng.integers(0, 256, (1, N, K // 2), dtype=np.uint8)
    scales = np.full((1, N, K // 16), 0x38, np.uint8)
    x = rng.integers(-1, 2, (M, K)).astype(np.float16)
    w = (codes, scales, np.ones(1, np.float32))
    ref = orc.linear(x, w)
    assert np.abs(ref).max() < 1024
    got = to_np64(_run(x, w))
    assert np.array_equal(got, ref)


def test_linear_batch_invariance():
    case = S.dense_case(32, weight_set=1)
    w = G.NVFP4Tensor.from_numpy(case["w"])
    x = torch.from_numpy(case["x"]).cuda()
    full = G.nvfp4_linear(x, w)
    singles = torch.cat([G.nvfp4_linear(x[m:m + 1].contiguous(), w) for m in range(32)])
    eights = torch.cat([G.nvfp4_linear(x[m:m + 8].contiguous(), w) for m in range(0, 32, 8)])
    torch.cuda.synchronize()
    assert torch.equal(full.view(torch.int16), singles.view(torch.int16))
    assert torch.equal(full.view(torch.int16), eights.view(torch.int16))


def test_linear_global_scale_and_ragged(orc):
    rng = S.rng_for(1, 7, 0)
    w = S.nvfp4_weights(rng, 1, 96, 1152, gscale=0.37)  # 1152 = 2 chunks of 512 + one of 128
    x = S.activations(rng, 45, 1152)
    assert_rows_close(to_np64(_run(x, w)), orc.linear(x, w), "linear ragged")


def test_linear_nan_scale_and_general_scales(orc):
    rng = S.rng_for(1, 8, 0)
    codes, _, gs = S.nvfp4_weights(rng, 1, 32, 512)
    scales = rng.integers(0, 0x60, (1, 32, 32), dtype=np.uint8)   # finite E4M3 bytes up to 2^5
    scales[0, :, ::2] |= 0x80                                       # and negative ones
    scales[0, 5, 7] = 0x7F                                          # one NaN scale in row 5
    x = S.activations(rng, 3, 512)
    y = to_np64(_run(x, (codes, scales, gs)))
    ref = orc.linear(x, (codes, scales, gs))
    assert np.all(np.isnan(y[:, 5]))
    keep = [c for c in range(32) if c != 5]
    assert_rows_close(y[:, keep], ref[:, keep], "linear general scales")


def test_linear_m0_is_noop():
    case = S.dense_case(1)
    w = G.NVFP4Tensor.from_numpy(case["w"])
    y = G.nvfp4_linear(torch.empty((0, S.DENSE_K), dtype=torch.float16, device="cuda"), w)
    torch.cuda.synchronize()
    assert y.shape == (0, S.DENSE_N)


@pytest.mark.parametrize("K", [16896, 32768])
def test_linear_long_reduction(orc, K):
    """Past K = 16384 the projection takes at most one weight tile per wave, so the chunk partials
    fit in the CU's 160 KiB of LDS (with two tiles, 33 or more chunks would need more); the reduction
    order is the same either way."""
    case = S.dense_case(3, n=64, k=K, weight_set=K)
    y = _run(case["x"], case["w"])
    assert_rows_close(to_np64(y), orc.linear(case["x"], case["w"]), f"linear K={K}")


def _poisoned_ws(M, N, K):
    """A split-K workspace filled with NaN bytes: the call must overwrite every partial it reads."""
    return torch.full((max(G.nvfp4_linear_ws_bytes(M, N, K), 16),), 0xFF, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("N,K,M", [(4352, 5120, 10), (4352, 5120, 16), (4352, 5120, 32), (256, 2176, 45),
                                   (64, 640, 80), (96, 1152, 70), (4352, 5120, 4), (64, 640, 33)])
def test_linear_split_k_bitwise_equals_one_launch(N, K, M):
    """nvfp4_linear_ws (per-chunk partials in a workspace, then their sum in chunk order) equals
    nvfp4_linear bitwise: past 32 rows it stages x in passes (45, 70, 80), 2176, 1152 and 640 end
    in a short chunk. Where each block's copy of x is small (M = 4, and 33 rows of 640) the call runs
    the one-launch kernel instead."""
    case = S.dense_case(M, n=N, k=K, weight_set=N + K)
    w = G.NVFP4Tensor.from_numpy(case["w"])
    x = torch.from_numpy(case["x"]).cuda()
    one = G.nvfp4_linear(x, w)
    split = G.nvfp4_linear_ws(x, w, ws=_poisoned_ws(M, N, K))
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), split.view(torch.int16))


def test_linear_split_k_matches_oracle_and_batch_invariance(orc):
    case = S.dense_case(32, weight_set=5)
    w = G.NVFP4Tensor.from_numpy(case["w"])
    x = torch.from_numpy(case["x"]).cuda()
    ws = _poisoned_ws(32, S.DENSE_N, S.DENSE_K)
    full = G.nvfp4_linear_ws(x, w, ws=ws)
    halves = torch.cat([G.nvfp4_linear_ws(x[m:m + 16].contiguous(), w, ws=ws) for m in (0, 16)])
    torch.cuda.synchronize()
    assert torch.equal(full.view(torch.int16), halves.view(torch.int16))
    assert_rows_close(to_np64(full), orc.linear(case["x"], case["w"]), "linear split-K M=32")
