"""GPU parity of the channel-FP8 ("QPN8") dense projection against the fp64 oracle ("[SM70][Draft]
Extend Qwen3.8 DFlash2 concurrency paths", "Follow-up: exact channel-FP8 QPN8 concurrency paths and
endpoint evidence": exact paths through M = 32, bitwise equal to concatenated 8-row calls).

Covers the 4352 x 5120 projection at M = 1..32 (per-row tolerance rule), an integer-exact case
(bitwise), batch invariance (single rows and 8-row concatenations), ragged K and an odd number of
16-row tiles, NaN bytes, and M = 0.
"""
import numpy as np
import pytest
import torch

import gemm_nvfp4_amd as G
from synth import inputs as S
from tests.parity import assert_rows_close, to_np64

pytestmark = pytest.mark.gpu


def _w(seed, n=S.DENSE_N, k=S.DENSE_K):
    return S.fp8_channel_weights(S.rng_for(S.WORKLOAD_IDS["dense"], 90 + seed, 0), n, k)


@pytest.mark.parametrize("M", S.DENSE_MS)
def test_fp8_projection_matches_oracle(orc, M):
    w = _w(0)
    x = S.activations(S.rng_for(S.WORKLOAD_IDS["dense"], 91, M), M, S.DENSE_K)
    y = G.nvfp4_linear_fp8(torch.from_numpy(x).cuda(), G.FP8ChannelTensor.from_numpy(w))
    torch.cuda.synchronize()
    assert_rows_close(to_np64(y), orc.linear_fp8(x, *w), f"fp8 M={M}")


@pytest.mark.parametrize("N,K,M", [(48, 640, 19), (64, 128, 1), (32, 1536, 40)])
def test_fp8_integer_exact(orc, N, K, M):
    """Bytes of the integers -4..4, scale 1, x in {-1,0,1}, |y| < 1024: exact, so bitwise."""
    ints = np.array([0xC8, 0xC4, 0xC0, 0xB8, 0x00, 0x38, 0x40, 0x44, 0x48], np.uint8)  # -4..4
    rng = np.random.default_rng(N + K + M)
    while True:
        codes = ints[rng.integers(0, 9, size=(N, K))]
        x = rng.integers(-1, 2, size=(M, K)).astype(np.float16)
        ref = orc.linear_fp8(x, codes, np.ones(N, np.float32))
        if np.abs(ref).max() < 1024:
            break
    y = G.nvfp4_linear_fp8(torch.from_numpy(x).cuda(), G.FP8ChannelTensor.from_numpy((codes, np.ones(N, np.float32))))
    torch.cuda.synchronize()
    assert np.array_equal(to_np64(y), ref)


def test_fp8_batch_invariance():
    w = G.FP8ChannelTensor.from_numpy(_w(1))
    x = torch.from_numpy(S.activations(S.rng_for(S.WORKLOAD_IDS["dense"], 92, 0), 32, S.DENSE_K)).cuda()
    y = G.nvfp4_linear_fp8(x, w)
    for m in (0, 13, 31):
        y1 = G.nvfp4_linear_fp8(x[m:m + 1].contiguous(), w)
        assert torch.equal(y1[0].view(torch.int16), y[m].view(torch.int16)), m
    y8 = torch.cat([G.nvfp4_linear_fp8(x[r:r + 8].contiguous(), w) for r in range(0, 32, 8)])
    assert torch.equal(y8.view(torch.int16), y.view(torch.int16))


def test_fp8_nan_byte_and_ragged(orc):
    codes, scale = _w(2, n=48, k=384)
    codes[7, 100] = 0x7F  # NaN in output column 7
    x = S.activations(S.rng_for(S.WORKLOAD_IDS["dense"], 93, 0), 5, 384)
    y = G.nvfp4_linear_fp8(torch.from_numpy(x).cuda(), G.FP8ChannelTensor.from_numpy((codes, scale)))
    torch.cuda.synchronize()
    got, ref = to_np64(y), orc.linear_fp8(x, codes, scale)
    assert np.all(np.isnan(got[:, 7])) and np.all(np.isnan(ref[:, 7]))
    keep = [c for c in range(48) if c != 7]
    assert_rows_close(got[:, keep], ref[:, keep], "fp8 ragged")


def test_fp8_m0_is_noop():
    w = G.FP8ChannelTensor.from_numpy(_w(3, n=32, k=128))
    y = G.nvfp4_linear_fp8(torch.zeros((0, 128), dtype=torch.float16, device="cuda"), w)
    assert y.shape == (0, 32)
