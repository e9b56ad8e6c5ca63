"""Pins for the oracle's exact rounding helpers (CPU only)."""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import floats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split()
                out[k] = v
    return out


def test_precision_table_2p3():
    """The page's worked example: 2.3 stored in fp32 / fp16 / bf16 / int8."""
    g = _golden("precision_2p3.txt")
    f32 = floats.fraction_to_f32(Fraction(23, 10))
    assert repr(float(f32)).startswith(g["fp32"][:14])
    # fp16: library conversion from the exact decimal (single rounding)
    assert float(np.float16(Fraction(23, 10).__float__())) == float(g["fp16"])
    bf = floats.f32_to_bf16_bits(np.array([f32], dtype=np.float32))
    assert float(floats.bf16_bits_to_f32(bf)[0]) == float(g["bf16"])
    assert int(2.3) == int(g["int8"])  # the page's int8 value truncates


def test_fraction_to_f32_matches_single_rounding_from_binary64():
    """For a rational that is exactly a binary64 value, RN to binary32 is the
    library's float64 -> float32 conversion (one rounding)."""
    g = np.random.default_rng(7)
    vals = np.concatenate([
        g.standard_normal(2000),
        g.standard_normal(500) * 1e-39,      # subnormal binary32 range
        g.standard_normal(500) * 1e-44,
        np.ldexp(1.0 + np.arange(64) / 2.0 ** 24, -130),  # exact half-way points
        np.ldexp(1.0 + (2 * np.arange(64) + 1) / 2.0 ** 25, 3),
    ])
    for v in vals:
        got = floats.fraction_to_f32(Fraction(float(v)))
        want = np.float32(v)
        assert got.view(np.uint32) == want.view(np.uint32), v


def test_bf16_rne_matches_torch():
    g = np.random.default_rng(11)
    bits = g.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # keep values whose bf16 rounding stays finite
    x = x[np.abs(x) < np.float32(3.38e38)]
    # add exact ties and subnormals
    ties = (np.arange(0, 4096, dtype=np.uint32) << np.uint32(16)) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(np.float32), np.float32([0.0, -0.0, 1e-45, -1e-45, 2.3])])
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = floats.f32_to_bf16_bits(x)
    np.testing.assert_array_equal(got, want)


def test_bf16_widen_is_exact():
    b = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    f = floats.bf16_bits_to_f32(b)
    fin = np.isfinite(f)
    back = floats.f32_to_bf16_bits(f[fin])
    np.testing.assert_array_equal(back, b[fin])
