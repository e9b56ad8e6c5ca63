"""Pins for the oracle's double quantization, dequantization, matmul and
storage arithmetic (CPU only)."""

import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import blockwise as bw, codebook, dequant, double_quant as dq, floats, matmul, memory

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split()
                out[k] = float(v)
    return out


# ---------------------------------------------------------------- tree sum / mean

def test_tree_sum_exact_cases_equal_fsum():
    g = np.random.default_rng(2)
    for n in (1, 2, 3, 5, 255, 256, 257, 1000):
        v = g.integers(0, 1000, n).astype(np.float64)
        assert dq.tree_sum_f64(v) == math.fsum(v)


def test_tree_sum_uses_pairwise_order():
    # sequential left-to-right gives 2^53 (each +1 is lost); the pairwise tree
    # adds the two ones first and keeps them
    v = np.array([2.0 ** 53, 0.0, 1.0, 1.0])
    assert dq.tree_sum_f64(v) == 2.0 ** 53 + 2.0
    seq = 0.0
    for x in v:
        seq += x
    assert seq == 2.0 ** 53
    # zero padding to the next power of two: [2^53, 1, 1] -> [2^53, 1, 1, 0]
    assert dq.tree_sum_f64(np.array([2.0 ** 53, 1.0, 1.0])) == 2.0 ** 53


def test_mean_is_fp64_sum_over_count_then_fp32():
    a = np.float32([1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0])
    assert dq.mean_f32(a) == np.float32(4.0)
    a = np.float32([1.0, 1.0, 2.0])
    assert dq.mean_f32(a) == floats.fraction_to_f32(Fraction(4, 3))


def _half_even(x: Fraction) -> int:
    fl = x.numerator // x.denominator
    rem = x - fl
    if rem != Fraction(1, 2):
        return fl + (1 if rem > Fraction(1, 2) else 0)
    return fl + (fl % 2)


def test_mean_keeps_the_sum_bits_beyond_fp32():
    """The sum 1 + 2^-24 needs 25 significant bits: kept in fp64 and divided by
    nb = 5 in fp64, the mean rounds once to fp32 and lands one ulp above 0.2.
    Rounding the sum to fp32 first (a tie, to even: 1.0) or summing in fp32
    gives fp32(0.2), so a mean divided in fp32 fails here."""
    a = np.float32([1.0, 2.0 ** -24, 0.0, 0.0, 0.0])
    exact = (Fraction(1) + Fraction(1, 2 ** 24)) / 5
    want = floats.fraction_to_f32(Fraction(float(exact)))     # fp64 quotient, then fp32
    got = dq.mean_f32(a)
    assert got == want and got.view(np.uint32) == np.float32(0.2).view(np.uint32) + 1
    # the same value as one rounding of the exact quotient (no double rounding here)
    assert want == floats.fraction_to_f32(exact)
    # the readings this case rules out
    seq32 = np.float32(0.0)
    for v in a:
        seq32 = np.float32(seq32 + v)
    assert np.float32(seq32 / np.float32(a.size)) != got
    assert np.float32(np.float32(1.0 + 2.0 ** -24) / np.float32(5.0)) != got


# ---------------------------------------------------------------- double quant

def test_hand_worked_double_quant():
    """absmax [1, 2, 3, 4]: mean 2.5, centred [-1.5, -0.5, 0.5, 1.5], block max 1.5,
    q = rint(127 * c / 1.5) = [-127, -42, 42, 127] (127/3 = 42.33)."""
    q, sigma, mu = dq.double_quant(np.float32([1, 2, 3, 4]))
    assert mu == np.float32(2.5)
    assert q.tolist() == [-127, -42, 42, 127]
    assert sigma.tolist() == [np.float32(1.5) / np.float32(127)]


def test_double_quant_ties_round_half_even():
    """absmax = 200 + [127, -127, .5, -.5, 2.5, -2.5, 1.5, -1.5]: the mean is 200
    exactly, the block maximum |c| is 127 and RN(RN(c/127)*127) gives back
    +-0.5, +-2.5, +-1.5, which are ties.  Half-even rounding sends them to
    0, 0, 2, -2, 2, -2; half-away-from-zero (floor(x + 1/2) for positives, C
    roundf) would give 1, -1, 3, -3, 2, -2."""
    offs = [127.0, -127.0, 0.5, -0.5, 2.5, -2.5, 1.5, -1.5]
    a = np.float32(200.0) + np.float32(offs)
    q, sigma, mu = dq.double_quant(a)
    assert mu == np.float32(200.0)
    s = Fraction(127)
    want, scaled = [], []
    for j in range(a.size):
        c = floats.fraction_to_f32(Fraction(float(a[j])) - Fraction(float(mu)))
        ratio = floats.fraction_to_f32(Fraction(float(c)) / s)
        u = Fraction(float(floats.fraction_to_f32(Fraction(float(ratio)) * 127)))
        scaled.append(u)
        want.append(_half_even(u))
    assert scaled[2:] == [Fraction(v) for v in offs[2:]]      # the ties are reached exactly
    assert want == [127, -127, 0, 0, 2, -2, 2, -2]
    assert q.tolist() == want
    assert sigma.tolist() == [np.float32(1.0)]
    # the rule this case rules out
    away = [int(np.sign(float(u))) * int(np.floor(abs(float(u)) + 0.5)) for u in scaled]
    assert away != want


def test_constant_absmax_round_trips_exactly():
    a = np.full(1000, np.float32(0.0173), dtype=np.float32)
    q, sigma, mu = dq.double_quant(a)
    assert mu == a[0] and not q.any() and not sigma.any()
    np.testing.assert_array_equal(dq.reconstruct_absmax(q, sigma, mu), a)


def test_double_quant_extremes_range_and_error_bound():
    g = np.random.default_rng(4)
    a = np.abs(g.standard_normal(256 * 7 + 13)).astype(np.float32) * np.float32(0.03)
    q, sigma, mu = dq.double_quant(a)
    assert q.min() >= -127 and q.max() <= 127
    c = (a - mu).astype(np.float32)
    for d in range(sigma.size):
        blk = slice(d * 256, (d + 1) * 256)
        j = int(np.argmax(np.abs(c[blk])))
        assert abs(int(q[blk][j])) == 127
    rec = dq.reconstruct_absmax(q, sigma, mu)
    sig = np.repeat(sigma, 256)[: a.size].astype(np.float64)
    err = np.abs(rec.astype(np.float64) - a.astype(np.float64))
    ulp = np.spacing(np.abs(a)).astype(np.float64)
    assert np.all(err <= sig / 2 + 4 * ulp + sig * 1e-6)


def test_double_quant_zero_block():
    a = np.float32([0.5] * 256 + [0.25] * 256)
    q, sigma, mu = dq.double_quant(a)
    assert mu == np.float32(0.375)
    assert q[:256].tolist() == [127] * 256 and q[256:].tolist() == [-127] * 256


# ---------------------------------------------------------------- dequant

def test_dequant_hand_worked_and_signed_zero():
    l = codebook.nf4_levels()
    packed = bw.pack(np.uint8([15, 0, 7, 8]))
    y = dequant.dequantize_f32(packed, 4, 2, l, np.float32([2.0, 0.0]))
    assert y[0] == 2.0 and y[1] == -2.0
    assert y[2] == 0.0 and np.signbit(y[2])     # negative level times zero absmax
    assert y[3] == 0.0 and not np.signbit(y[3])
    yb = dequant.dequantize_bf16_bits(packed, 4, 2, l, np.float32([2.0, 0.0]))
    assert yb.tolist() == [0x4000, 0xC000, 0x8000, 0x0000]


def test_dequant_through_double_quant_uses_two_roundings():
    q = np.int8([100, -3])
    sigma = np.float32([np.float32(0.1) / np.float32(127)])
    mu = np.float32(0.0371)
    got = dq.reconstruct_absmax(q, sigma, mu)
    for j in range(2):
        prod = floats.fraction_to_f32(Fraction(int(q[j])) * Fraction(float(sigma[0])))
        want = floats.fraction_to_f32(Fraction(float(prod)) + Fraction(float(mu)))
        assert got[j] == want


# ---------------------------------------------------------------- matmul

def test_qlora_forward_matches_exact_rationals_non_square():
    g = np.random.default_rng(6)
    M, N, K, r = 3, 5, 7, 2
    X = g.standard_normal((M, K)).astype(np.float32)
    W = g.standard_normal((N, K)).astype(np.float32)
    A = g.standard_normal((K, r)).astype(np.float32)
    B = g.standard_normal((r, N)).astype(np.float32)
    got = matmul.qlora_forward_f64(X, W, A, B, 2.0)
    want = matmul.qlora_forward_exact(X, W, A, B, 2)
    for m in range(M):
        for n in range(N):
            assert abs(got[m, n] - float(want[m][n])) <= 1e-12 * (1 + abs(float(want[m][n])))
    base = matmul.qlora_forward_f64(X, W)
    want0 = matmul.qlora_forward_exact(X, W)
    assert np.allclose(base, np.array(want0, dtype=np.float64), rtol=1e-13, atol=1e-13)


def test_lora_only_when_base_is_zero():
    g = np.random.default_rng(8)
    X = g.standard_normal((4, 6))
    A = g.standard_normal((6, 2))
    B = g.standard_normal((2, 3))
    Y = matmul.qlora_forward_f64(X, np.zeros((3, 6)), A, B, 2.0)
    assert np.allclose(Y, 2.0 * (X @ A) @ B)


def test_tolerance_metrics():
    ref = np.array([[1.0, -2.0], [3.0, 4.0]])
    assert matmul.rel_frobenius(ref, ref) == 0.0
    assert matmul.max_rel_to_peak(ref + np.array([[0.0, 0.0], [0.0, 0.4]]), ref) == pytest.approx(0.1)


# ---------------------------------------------------------------- memory / counts

def test_pages_memory_figures():
    g = _golden("memory_figures.txt")
    n70 = int(g["params_70b"])
    assert n70 * 2 / 1e9 == g["gb_fp16_70b"]
    assert n70 * 0.5 / 1e9 == g["gb_4bit_70b"]
    n13 = int(g["params_13b"])
    assert n13 * 2 / 1e9 == g["gb_fp16_13b"]
    assert n13 * 0.5 / 1e9 == g["gb_4bit_13b"]
    # codes plus NF4 + double-quant overhead for 70e9 params
    assert abs(memory.state_bytes(n70) / 1e9 - 70e9 * 4.126953125 / 8 / 1e9) < 1e-6


def test_double_quant_bits_per_param():
    g = _golden("memory_figures.txt")
    plain = memory.bits_per_param(64, nested=False)
    nested = memory.bits_per_param(64, nested=True)
    assert plain == Fraction(9, 2)
    assert float(nested) == 4.126953125
    assert round(float(plain - nested), 2) == g["dq_saving_bits"]
    assert float(plain - 4) == g["overhead_bits_before_dq"]
    assert round(float(nested - 4), 2) == g["overhead_bits_after_dq"]


def test_state_bytes_equals_oracle_output_sizes():
    g = np.random.default_rng(12)
    for n in (1, 63, 64, 65, 1000, 16384 + 7, 256 * 64 * 3 + 1):
        x = g.standard_normal(n).astype(np.float32)
        packed, a = bw.quantize_blockwise(x, 64, codebook.nf4_levels())
        q, sigma, mu = dq.double_quant(a)
        assert memory.state_bytes(n, 64, True) == packed.nbytes + q.nbytes + sigma.nbytes + 4
        assert memory.state_bytes(n, 64, False) == packed.nbytes + a.nbytes


def test_lora_parameter_count_and_scale():
    g = _golden("memory_figures.txt")
    d, r = int(g["row_width_example"]), int(g["lora_rank"])
    assert d * d == g["lora_full_params"]
    assert d * r + r * d == g["lora_r16_params"]
    assert d * d // (2 * d * r) == g["lora_ratio"]
    assert bw.num_blocks(d, 64) == g["blocks_per_row_example"]
    assert 32 / 16 == 2.0   # lora_alpha / r of the page's PEFT example
