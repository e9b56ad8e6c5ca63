"""Level tables (step a1) — oracle, test infrastructure only.

NF4 ("篇2-bitsandbytes-具体观-算法与实现剖析", §2.2 QLoRA / NF4, 【原理】 ①):
the standard normal CDF is cut into 16 slabs of equal probability, each slab
is represented by its midpoint, so every level carries the same probability
mass; the weights are normalised to [-1, 1] before the lookup.

Reading taken here (the page leaves it open): "midpoint" is the probability
midpoint of slab i, (2i+1)/32, because the value midpoint of the two end slabs
is infinite.  The quantiles are divided by the largest one so the table spans
exactly [-1, 1].  The result is symmetric and has no exact-zero level.

    q_i = Phi^-1((2i+1)/32),  i = 0..15        (mpmath, 50 significant digits)
    l_i = RN_fp32(q_i / q_15)

FP4 (same page, §2.2 【代码】: a generic floating-point table builder with
exponent_bits=2, precision_bits=1, signed, 4 bits; "Tim Dettmers 如何用
bitsandbytes 與 QLoRA 降低 LLM 訓練門檻？", section "NF4 不是一般四位元浮點格式",
contrasts NF4 with an IEEE-style FP4): code c = s<<3 | e<<1 | m, with IEEE
subnormals at e = 0, normalised by the largest magnitude.  The exponent bias
cancels in the normalisation.  The table is kept in code order, so it is not
sorted and holds both +0 (code 0) and -0 (code 8).
"""

from fractions import Fraction

import mpmath
import numpy as np

from .floats import fraction_to_f32

NF4 = 0
FP4 = 1


def _mpf_to_fraction(v) -> Fraction:
    sign, man, exp, _ = mpmath.mpf(v)._mpf_   # value = (-1)^sign * man * 2^exp, exactly
    f = Fraction(int(man)) * (Fraction(2) ** int(exp))
    return -f if sign else f


def nf4_quantiles(dps: int = 50):
    """q_i = Phi^-1((2i+1)/32) as mpmath numbers."""
    with mpmath.workdps(dps):
        return [mpmath.sqrt(2) * mpmath.erfinv(mpmath.mpf(2 * i + 1) / 16 - 1) for i in range(16)]


def nf4_levels() -> np.ndarray:
    with mpmath.workdps(50):
        q = nf4_quantiles(50)
        ratios = [q[i] / q[15] for i in range(16)]
        fr = [_mpf_to_fraction(r) for r in ratios]
    return np.array([fraction_to_f32(f) for f in fr], dtype=np.float32)


def fp_table_exact(exponent_bits: int = 2, precision_bits: int = 1, signed: bool = True):
    """Exact rational values of an IEEE-style minifloat, in code order,
    normalised by the largest magnitude.  Returns a list of (sign, Fraction)."""
    bias = 2 ** (exponent_bits - 1) - 1
    total = (1 if signed else 0) + exponent_bits + precision_bits
    out = []
    for c in range(2 ** total):
        s = (c >> (exponent_bits + precision_bits)) & 1 if signed else 0
        e = (c >> precision_bits) & (2 ** exponent_bits - 1)
        m = c & (2 ** precision_bits - 1)
        frac = Fraction(m, 2 ** precision_bits)
        if e == 0:  # subnormal: 0.m * 2^(1-bias)
            mag = frac * Fraction(2) ** (1 - bias)
        else:       # normal: 1.m * 2^(e-bias)
            mag = (1 + frac) * Fraction(2) ** (e - bias)
        out.append((s, mag))
    top = max(mag for _, mag in out)
    return [(s, mag / top) for s, mag in out]


def fp4_levels() -> np.ndarray:
    vals = []
    for s, mag in fp_table_exact(2, 1, True):
        v = fraction_to_f32(mag)
        vals.append(-v if s else v)  # keeps -0.0 for code 8
    return np.array(vals, dtype=np.float32)


def levels(kind: int) -> np.ndarray:
    if kind == NF4:
        return nf4_levels()
    if kind == FP4:
        return fp4_levels()
    raise ValueError(f"unknown codebook kind {kind}")
