"""Pins for the oracle's storage-format roundings (bfloat16 and IEEE binary16,
round-to-nearest-even), checked against torch's and numpy's own casts, and
against hand-worked tie and overflow cases."""
import numpy as np
import pytest
import torch


def _torch_bf16_bits(vals_f32):
    t = torch.from_numpy(np.asarray(vals_f32, np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(3000).astype(np.float32),
        (rng.standard_normal(500) * 1e-38).astype(np.float32),      # subnormal range
        (rng.standard_normal(500) * 1e37).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.4e38], np.float32),
    ])
    # exact midpoints between neighbouring bf16 values (ties -> even)
    mids = (rng.integers(0x0080, 0x7f00, 400).astype(np.uint32) << 16) | 0x8000
    vals = np.concatenate([vals, mids.view(np.float32)])
    expect = _torch_bf16_bits(vals)
    got = np.array([orc.bf16_bits(float(v)) for v in vals], np.uint16)
    assert np.array_equal(got, expect)


def test_bf16_hand_cases(orc):
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1.0 (0x3f80)
    assert orc.bf16_bits(1.0 + 2.0 ** -8) == 0x3F80
    # 1 + 3 * 2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even) -> 0x3f82
    assert orc.bf16_bits(1.0 + 3 * 2.0 ** -8) == 0x3F82
    # just above the midpoint rounds up (single rounding from double)
    assert orc.bf16_bits(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    assert orc.bf16_bits(-2.0) == 0xC000
    assert orc.bf16_bits(float("inf")) == 0x7F80


def test_f16_rounding_matches_numpy(orc):
    rng = np.random.default_rng(2)
    vals = np.concatenate([
        rng.standard_normal(3000),
        rng.standard_normal(500) * 1e-6,        # subnormal range of binary16
        rng.standard_normal(500) * 3e4,
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 2.0 ** -24,
                  2.0 ** -25, 2.0 ** -25 + 2.0 ** -40, 6e-8]),
    ])
    expect = vals.astype(np.float16).view(np.uint16)
    got = np.array([orc.f16_bits(float(v)) for v in vals], np.uint16)
    assert np.array_equal(got, expect)


def test_f16_hand_cases(orc):
    assert orc.f16_bits(1.0) == 0x3C00
    assert orc.f16_bits(1.0 + 2.0 ** -11) == 0x3C00          # tie -> even
    assert orc.f16_bits(1.0 + 3 * 2.0 ** -11) == 0x3C02      # tie -> even (up)
    assert orc.f16_bits(65504.0) == 0x7BFF
    assert orc.f16_bits(65520.0) == 0x7C00                   # overflow to inf
    assert orc.f16_bits(2.0 ** -24) == 0x0001                # smallest subnormal
    assert orc.f16_bits(2.0 ** -25) == 0x0000                # tie -> even (zero)
    assert orc.f16_bits(-(2.0 ** -14)) == 0x8400             # smallest normal


def test_decode_all_patterns(orc):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f16 = pats.view(np.float16).astype(np.float64)
    bf = (pats.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    step = 97  # a spread sample of every exponent / sign
    for p in range(0, 65536, step):
        if np.isfinite(f16[p]):
            assert orc.f16_value(p) == f16[p]
        if np.isfinite(bf[p]):
            assert orc.bf16_value(p) == bf[p]
