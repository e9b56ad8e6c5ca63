"""Pins for the oracle's 8-bit blockwise quantization with the dynamic map (CPU).

The pages describe the map by its properties (256 non-uniform levels, dense near
zero and sparse in the tails, maximising the code entropy; signed and unsigned
variants) and the blocking by figure 2-3 of "篇2-bitsandbytes-具体观-算法与实现剖析"
(blocks of 2048, a local absmax each, 8-bit codes).  Each pin below checks one of
those properties, or the exact definition on small inputs, by a route that does
not reuse the oracle's own arithmetic."""

import statistics
from fractions import Fraction

import numpy as np

from oracle import blockwise as obw, blockwise8 as o8
from oracle.floats import fraction_to_f32

PHI = statistics.NormalDist()


def test_signed_map_equal_mass_symmetric_and_dense_at_zero():
    lv = o8.dynamic_map(True)
    q255 = PHI.inv_cdf(511 / 512)
    for i in (0, 1, 64, 127, 128, 200, 254, 255):
        assert abs(PHI.cdf(float(lv[i]) * q255) - (2 * i + 1) / 512) < 1e-6
    assert lv[0] == -1.0 and lv[255] == 1.0
    assert np.all(np.diff(lv.astype(np.float64)) > 0)
    assert np.array_equal(lv[::-1].view(np.uint32), (-lv).view(np.uint32))      # antisymmetric, bitwise
    gaps = np.diff(lv.astype(np.float64))
    assert np.all(np.diff(gaps[127:]) > 0) and np.all(np.diff(gaps[:128]) < 0)  # sparser away from 0
    assert 0 not in lv                                                          # no exact-zero level


def test_unsigned_map_half_normal_mass_and_dense_at_zero():
    lv = o8.dynamic_map(False)
    q = PHI.inv_cdf(0.5 + 511 / 1024)
    for i in (0, 1, 100, 254, 255):
        assert abs(PHI.cdf(float(lv[i]) * q) - (0.5 + (2 * i + 1) / 1024)) < 1e-6
    assert lv[255] == 1.0 and lv[0] > 0
    gaps = np.diff(lv.astype(np.float64))
    assert np.all(gaps > 0) and np.all(np.diff(gaps) > 0)


def test_signed_map_codes_of_normal_data_are_near_uniform():
    """Equal mass per level: standard normal data scaled by q_255 fills the 256
    codes about equally (maximum entropy), apart from the clipped tails."""
    lv = o8.dynamic_map(True)
    z = np.random.default_rng(5).standard_normal(2_000_000)
    t = (z / PHI.inv_cdf(511 / 512)).astype(np.float32)
    t = np.clip(t, -1, 1)
    counts = np.bincount(obw.nearest_code(t, lv), minlength=256)
    expect = z.size / 256
    inner = counts[2:-2]
    assert np.max(np.abs(inner - expect)) < 6 * np.sqrt(expect)
    H = -np.sum((counts / z.size) * np.log2(np.maximum(counts, 1) / z.size))
    assert H > 7.99


def test_quantize8_matches_bruteforce_and_blocks():
    """Tiny inputs against the exact definition: flattened blocks (the last
    partial), fp32 absmax, IEEE division, exact nearest level with ties to the
    lower index (t = 0 lies exactly on the middle threshold of the signed map)."""
    g = np.random.default_rng(7)
    for signed in (True, False):
        lv = o8.dynamic_map(signed)
        x = (g.standard_t(3, size=300) * 1e-3).astype(np.float32)
        if not signed:
            x = np.abs(x)
        x[5:9] = 0.0
        x[256:] = 0.0                                   # an all-zero last block (B = 64 below)
        B = 64
        codes, a = o8.quantize_blockwise8(x, B, lv)
        assert a.size == 5 and a[-1] == 0.0
        for j in range(a.size):
            blk = x[j * B:(j + 1) * B]
            assert a[j] == np.max(np.abs(blk))
            aj = Fraction(float(a[j]))
            for k, xv in enumerate(blk):
                tv = np.float32(0.0) if aj == 0 else fraction_to_f32(Fraction(float(xv)) / aj)
                assert codes[j * B + k] == obw.nearest_code_bruteforce([tv], lv)[0]
    lv = o8.dynamic_map(True)
    codes, _ = o8.quantize_blockwise8(np.zeros(10, np.float32), 2048, lv)
    assert np.all(codes == 127)                          # tie at 0 goes to the lower index


def test_on_grid_values_round_trip_exactly():
    lv = o8.dynamic_map(True)
    a = np.float32(0.37)
    x = (lv * a).astype(np.float32)                      # RN(l_i * a), contains +-a
    codes, am = o8.quantize_blockwise8(x, 256, lv)
    assert am[0] == a
    assert np.array_equal(codes, np.arange(256))
    y = o8.dequantize_blockwise8(codes, am, 256, 256, lv)
    assert np.array_equal(y.view(np.uint32), x.view(np.uint32))


def test_error_within_half_the_widest_gap():
    lv = o8.dynamic_map(True)
    x = (np.random.default_rng(9).standard_normal(8192) * 1e-2).astype(np.float32)
    codes, a = o8.quantize_blockwise8(x, 2048, lv)
    y = o8.dequantize_blockwise8(codes, a, x.size, 2048, lv)
    half_gap = np.max(np.diff(lv.astype(np.float64))) / 2
    aa = np.repeat(a.astype(np.float64), 2048)
    assert np.all(np.abs(y.astype(np.float64) - x) <= aa * half_gap * (1 + 1e-6) + 1e-12)


def test_state_memory_of_the_page():
    """Figure 2-3's page: Adam keeps m and v in fp32, 8 GB for 1 B parameters;
    the 8-bit states take one byte per element plus an fp32 absmax per 2048."""
    n = 10 ** 9
    assert 2 * 4 * n == 8 * 10 ** 9
    assert o8.state_bytes8(n) == n + 4 * ((n + 2047) // 2048)
    assert 2 * o8.state_bytes8(n) < 2.01e9
