"""Pins for the oracle's channel-FP8 ("QPN8") dense projection ("[SM70][Draft] Extend Qwen3.8
DFlash2 concurrency paths", "Follow-up: exact channel-FP8 QPN8 concurrency paths and endpoint
evidence"): E4M3FN weight bytes with one FP32 scale per output channel.

Independent routes: torch's float8_e4m3fn cast (a library routine) times the channel scale, then a
numpy float64 matmul; an integer-exact case checked in Python integers; NaN bytes and zero scales.
"""
import numpy as np
import torch

from synth import inputs as S


def dq(codes, scale):
    e4 = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return e4 * scale.astype(np.float64)[:, None]


def test_fp8_linear_matches_numpy(orc):
    rng = S.rng_for(S.WORKLOAD_IDS["dense"], 80, 0)
    codes, scale = S.fp8_channel_weights(rng, 96, 640)
    x = S.activations(rng, 7, 640)
    ref = x.astype(np.float64) @ dq(codes, scale).T
    got = orc.linear_fp8(x, codes, scale)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_fp8_linear_integer_exact(orc):
    """Bytes of the integers -4..4 in E4M3FN, scale 1, x in {-1, 0, 1}: exact in integers."""
    ints = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48, -1: 0xB8, -2: 0xC0, -3: 0xC4, -4: 0xC8}
    rng = np.random.default_rng(5)
    N, K, M = 24, 256, 3
    iv = rng.integers(-4, 5, size=(N, K))
    codes = np.vectorize(ints.get)(iv).astype(np.uint8)
    xi = rng.integers(-1, 2, size=(M, K))
    got = orc.linear_fp8(xi.astype(np.float16), codes, np.ones(N, np.float32))
    ref = [[sum(int(a) * int(b) for a, b in zip(xi[m], iv[n])) for n in range(N)] for m in range(M)]
    assert np.array_equal(got, np.array(ref, dtype=np.float64))


def test_fp8_nan_byte_and_zero_scale(orc):
    rng = S.rng_for(S.WORKLOAD_IDS["dense"], 81, 0)
    codes, scale = S.fp8_channel_weights(rng, 4, 128)
    codes[1, 5] = 0x7F  # NaN poisons column 1 only
    scale[2] = 0.0       # a zero channel gives zeros (no NaN bytes in it)
    x = S.activations(rng, 3, 128)
    y = orc.linear_fp8(x, codes, scale)
    assert np.all(np.isnan(y[:, 1])) and np.all(np.isfinite(y[:, [0, 2, 3]]))
    assert np.all(y[:, 2] == 0.0)
