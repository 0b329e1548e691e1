"""Pins for the oracle's number formats (E2M1, E4M3FN, binary16) and SiLU.

Each check uses something other than the oracle: hand values from the formats' definitions
(tests/golden/e4m3_e2m1_values.txt), torch's float8_e4m3fn cast, numpy's float16 conversion,
and scipy's expit. The "[Kernel][SM70] Improve Qwen3.8 no-MTP concurrency" page, "Test Plan",
asks for native E4M3 encoding, subnormal, signed-zero and NaN tests.
"""
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_e2m1_values.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        fmt, byte, val = line.split()
        rows.append((fmt, int(byte, 16), float(val)))
    return rows


def _same(a, b):
    if math.isnan(b):
        return math.isnan(a)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


@pytest.mark.parametrize("fmt,byte,val", _golden())
def test_golden_decode_values(orc, fmt, byte, val):
    got = orc.e2m1(byte) if fmt == "e2m1" else orc.e4m3(byte)
    assert _same(got, val), (fmt, hex(byte), got, val)


def test_e4m3_all_bytes_match_torch_float8(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        assert _same(orc.e4m3(b), float(ref[b])), hex(b)


def test_e2m1_closed_form_properties(orc):
    mags = [orc.e2m1(c) for c in range(8)]
    assert mags == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(8):  # sign bit only flips the sign
        assert _same(orc.e2m1(c | 8), -mags[c])


def test_half_decode_all_patterns_match_numpy(orc):
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.half(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_half_encode_matches_numpy_rne(orc):
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.standard_normal(4000) * 10.0 ** rng.integers(-9, 6, 4000),
        rng.uniform(-1, 1, 2000) * 2.0 ** -14,          # subnormal range
        np.array([65504.0, 65519.99, 65520.0, 70000.0, -65520.0, 1e-9, -0.0, 0.0,
                  1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11,      # ties: to even (down, then up)
                  2.0 ** -25, 3 * 2.0 ** -25, 2.0 ** -24 * 1023.5, math.inf, -math.inf]),
    ])
    for v in vals:
        ref = int(np.array([v], dtype=np.float64).astype(np.float16).view(np.uint16)[0])
        assert orc.to_half(float(v)) == ref, (v, hex(ref))
    assert orc.to_half(math.nan) & 0x7C00 == 0x7C00 and orc.to_half(math.nan) & 0x3FF


def test_e2m1_times_e4m3_exact_in_fp16(orc):
    """Every finite e2m1*e4m3 product is exactly representable in binary16 (a closed-form fact the
    device decode relies on): at most 6 significant bits, magnitude in [2^-10, 2688]."""
    for c in range(16):
        for b in range(256):
            s = orc.e4m3(b)
            if math.isnan(s):
                continue
            p = orc.e2m1(c) * s
            assert float(np.float16(p)) == p, (c, hex(b), p)


def test_silu_identities_and_library(orc):
    from scipy.special import expit
    assert orc.silu(0.0) == 0.0
    for g in np.linspace(-30, 30, 601):
        assert abs((orc.silu(g) - orc.silu(-g)) - g) <= 1e-12 * max(1.0, abs(g))
        assert abs(orc.silu(g) - g * expit(g)) <= 1e-14 * max(1.0, abs(g))
    assert orc.silu(-800.0) == 0.0  # exp overflow gives g/inf = -0
