"""Exact rounding helpers for the oracle (test infrastructure only).

* ``fraction_to_f32`` rounds an exact rational to the nearest IEEE binary32
  value, ties to even, subnormals kept.  It is the "RN_fp32" used when a level
  table is defined from exact or high-precision quantities.
* ``f32_to_bf16_bits`` is round-to-nearest-even from binary32 to bfloat16,
  written out from its definition (keep the upper 16 bits, look at the 16
  dropped bits, go up if they exceed half, stay if below, go to the even
  neighbour on a tie).  The precision table of "LLM 相關知識" (section
  精度 (Precision), the 2.3 example) fixes bf16(2.3) = 2.296875, which the tests
  check.
"""

from fractions import Fraction

import numpy as np

F32_MIN_EXP = -126      # exponent of the smallest normal binary32
F32_MANT_BITS = 23      # stored fraction bits of binary32
F32_SUBNORMAL_QUANTUM = Fraction(1, 2 ** 149)


def _floor_log2(q: Fraction) -> int:
    """floor(log2(q)) for a positive rational, exactly."""
    e = q.numerator.bit_length() - q.denominator.bit_length()
    # now 2**(e-1) < q < 2**(e+1); fix up to 2**e <= q < 2**(e+1)
    if e >= 0:
        if q < Fraction(2 ** e):
            e -= 1
    else:
        if q < Fraction(1, 2 ** (-e)):
            e -= 1
    return e


def _round_half_even(q: Fraction) -> int:
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def fraction_to_f32(q) -> np.float32:
    """Round an exact rational (Fraction, int, or exactly-converted float) to
    binary32 with round-to-nearest-even.  Finite results only."""
    q = Fraction(q)
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = _floor_log2(a)
    if e < F32_MIN_EXP:
        quantum = F32_SUBNORMAL_QUANTUM
    else:
        quantum = Fraction(2) ** (e - F32_MANT_BITS)
    m = _round_half_even(a / quantum)
    val = m * quantum  # exactly representable in binary32 (and binary64)
    out = np.float32(float(val))
    if not np.isfinite(out):
        raise OverflowError("value does not fit binary32")
    assert Fraction(float(out)) == val
    return np.float32(sign * out)


def f32_to_bf16_bits(x) -> np.ndarray:
    """binary32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    Inputs are finite (NaN/Inf are outside the contract of every caller)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    bits = x.view(np.uint32).astype(np.uint64)
    kept = bits >> np.uint64(16)            # truncated bf16 pattern
    dropped = bits & np.uint64(0xFFFF)      # the 16 bits that are thrown away
    half = np.uint64(0x8000)
    go_up = (dropped > half) | ((dropped == half) & ((kept & np.uint64(1)) == np.uint64(1)))
    # adding one to the pattern steps to the next bf16 away from zero in magnitude
    # (carries into the exponent are the correct next binade)
    out = kept + go_up.astype(np.uint64)
    return out.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """bfloat16 bit patterns -> binary32 (exact)."""
    b = np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f32_bits(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
