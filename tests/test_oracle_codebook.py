"""Pins for the oracle's level tables (CPU only).

NF4 is pinned by the property the page defines it by — equal probability mass
per level — checked with an independent normal CDF (math.erf), and by a second
inverse-normal implementation (the standard library's).  FP4 is pinned by the
E2M1 magnitudes of the IEEE-style minifloat with 2 exponent and 1 mantissa bit.
"""

import math
import statistics
from fractions import Fraction

import numpy as np

from oracle import codebook


def _phi(z: float) -> float:
    return 0.5 * (1.0 + math.erf(z / math.sqrt(2.0)))


def test_nf4_equal_probability_mass():
    l = codebook.nf4_levels().astype(np.float64)
    q15 = float(codebook.nf4_quantiles()[15])
    assert abs(_phi(q15) - 31 / 32) < 1e-15
    for i in range(16):
        # level i is the probability midpoint of slab [i/16, (i+1)/16]
        assert abs(_phi(l[i] * q15) - (2 * i + 1) / 32) < 2e-7, i
    # equal mass between consecutive slab midpoints
    masses = np.diff([_phi(v * q15) for v in l])
    assert np.allclose(masses, 1 / 16, atol=3e-7)


def test_nf4_shape_invariants():
    l = codebook.nf4_levels()
    assert l.dtype == np.float32 and l.shape == (16,)
    assert l[0] == np.float32(-1.0) and l[15] == np.float32(1.0)
    assert np.all(np.diff(l) > 0)
    np.testing.assert_array_equal(l[::-1].view(np.uint32) ^ np.uint32(0x80000000), l.view(np.uint32))
    assert not np.any(l == 0)  # the equal-mass construction has no zero level
    assert abs(float(l[8]) - 0.0420954) < 1e-6
    assert abs(float(l[14]) - 0.7075688) < 1e-6


def test_nf4_matches_second_inverse_normal():
    nd = statistics.NormalDist()
    q = [nd.inv_cdf((2 * i + 1) / 32) for i in range(16)]
    alt = np.array([np.float32(v / q[15]) for v in q], dtype=np.float32)
    np.testing.assert_array_equal(alt.view(np.uint32), codebook.nf4_levels().view(np.uint32))


def test_fp4_is_e2m1_normalised():
    l = codebook.fp4_levels()
    e2m1 = [0, 0.5, 1, 1.5, 2, 3, 4, 6]   # E2M1 magnitudes, code order
    for c in range(8):
        assert l[c] == np.float32(e2m1[c] / 6)
        assert l[c + 8] == -np.float32(e2m1[c] / 6)
    assert np.signbit(l[8]) and l[8] == 0
    assert l[7] == 1 and l[15] == -1
    assert len(set(float(v) for v in l)) == 15
    exact = codebook.fp_table_exact(2, 1, True)
    assert [m for _, m in exact[:8]] == [Fraction(k, 12) for k in (0, 1, 2, 3, 4, 6, 8, 12)]
