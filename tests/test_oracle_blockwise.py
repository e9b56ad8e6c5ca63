"""Pins for the oracle's blockwise quantization (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import blockwise as bw, codebook, dequant, floats


def _neighbours(v: np.float32, k: int = 4):
    """All binary32 values within k ulp of v (inclusive)."""
    out = []
    cur = np.float32(v)
    for _ in range(k):
        cur = np.nextafter(cur, np.float32(-np.inf), dtype=np.float32)
    for _ in range(2 * k + 1):
        out.append(cur)
        cur = np.nextafter(cur, np.float32(np.inf), dtype=np.float32)
    return out


@pytest.mark.parametrize("kind", [codebook.NF4, codebook.FP4])
def test_nearest_code_matches_bruteforce_near_every_midpoint(kind):
    l = codebook.levels(kind)
    u = sorted(set(float(v) for v in l))
    probes = []
    for a, b in zip(u[:-1], u[1:]):
        mid = (Fraction(a) + Fraction(b)) / 2
        probes += _neighbours(floats.fraction_to_f32(mid))
    for v in l:
        probes += _neighbours(v, 2)
    probes += [np.float32(0.0), np.float32(-0.0), np.float32(1e-45), np.float32(-1e-45),
               np.float32(1.0), np.float32(-1.0)]
    g = np.random.default_rng(3)
    probes += list(g.uniform(-1, 1, 500).astype(np.float32))
    t = np.array(probes, dtype=np.float32)
    t = t[np.abs(t) <= 1]
    assert list(bw.nearest_code(t, l)) == bw.nearest_code_bruteforce(t, l)


def test_nf4_zero_and_ties():
    l = codebook.nf4_levels()
    # +0 and -0 are at equal distance from l_7 and l_8: the lower index wins
    assert list(bw.nearest_code(np.float32([0.0, -0.0]), l)) == [7, 7]
    # the smallest positive subnormal is nearer to l_8
    assert bw.nearest_code(np.float32([1e-45]), l)[0] == 8


def test_fp4_ties_go_to_smaller_code_not_smaller_value():
    l = codebook.fp4_levels()
    # -1/24 is equidistant from -1/12 (code 9) and 0 (codes 0 and 8): code 0 wins
    t = np.float32(-1.0 / 24.0)
    assert bw.nearest_code_bruteforce([t], l) == list(bw.nearest_code(np.array([t]), l))
    assert bw.nearest_code(np.float32([0.0, -0.0]), l).tolist() == [0, 0]


def test_hand_worked_nf4_block():
    """A block of 8 worked by hand from the NF4 levels
    (-1, -.7076, -.5422, -.4168, -.3109, -.2159, -.1273, -.0421, +mirror)."""
    x = np.float32([1.0, -1.0, 0.5, -0.5, 0.25, 0.0, 0.1, -0.3])
    packed, a = bw.quantize_blockwise(x, 8, codebook.nf4_levels())
    assert a.tolist() == [1.0]
    assert bw.unpack(packed, 8).tolist() == [15, 0, 13, 2, 10, 7, 9, 4]
    assert packed.tolist() == [0xF0, 0xD2, 0xA7, 0x94]


def test_absmax_bruteforce_and_partial_block():
    g = np.random.default_rng(5)
    x = g.standard_normal(203).astype(np.float32)
    for B in (8, 64, 128):
        got = bw.absmax(x, B)
        want = [max(abs(float(v)) for v in x[i:i + B]) for i in range(0, x.size, B)]
        assert got.tolist() == [np.float32(w) for w in want]
        assert got.size == -(-x.size // B)


def test_normalize_is_correctly_rounded_division():
    g = np.random.default_rng(9)
    x = np.concatenate([g.standard_normal(300), g.standard_normal(50) * 1e-40]).astype(np.float32)
    x[:64] = 0.0                                  # one zero block at B=64
    a = bw.absmax(x, 64)
    t = bw.normalize(x, a, 64)
    for k in range(x.size):
        aj = a[k // 64]
        if aj == 0:
            assert t[k] == 0 and not np.signbit(t[k])
            continue
        want = floats.fraction_to_f32(Fraction(float(x[k])) / Fraction(float(aj)))
        assert t[k].view(np.uint32) == want.view(np.uint32)
    assert np.all(np.abs(t) <= 1)


def test_pack_high_nibble_first_and_odd_tail():
    assert bw.pack(np.uint8([1, 2, 3])).tolist() == [0x12, 0x30]
    c = np.random.default_rng(1).integers(0, 16, 101).astype(np.uint8)
    assert bw.unpack(bw.pack(c), 101).tolist() == c.tolist()
    assert bw.pack(c).size == 51


@pytest.mark.parametrize("kind", [codebook.NF4, codebook.FP4])
def test_exact_round_trip_on_grid_fp32(kind):
    """A block holding +-a and values already on the grid l_i * a returns the
    same codes and the same fp32 values after dequantization."""
    l = codebook.levels(kind)
    g = np.random.default_rng(kind + 20)
    B = 64
    blocks = []
    want_codes = []
    for _ in range(40):
        a = np.float32(abs(g.standard_normal()) * 0.05 + 1e-3)
        codes = g.integers(0, 16, B).astype(np.uint8)
        codes[0] = 15 if kind == codebook.NF4 else 7   # +a  (level +1)
        if kind == codebook.FP4:
            codes[codes == 8] = 0     # -0 is never produced: use code 0 instead
        x = (l[codes] * a).astype(np.float32)
        blocks.append(x)
        want_codes.append(codes)
    x = np.concatenate(blocks)
    packed, amax = bw.quantize_blockwise(x, B, l)
    assert bw.unpack(packed, x.size).tolist() == np.concatenate(want_codes).tolist()
    y = dequant.dequantize_f32(packed, x.size, B, l, amax)
    np.testing.assert_array_equal(y.view(np.uint32), x.view(np.uint32))


def test_exact_round_trip_on_grid_bf16():
    """bf16 input already on the grid: x = RNE_bf16(RN(l_i * a)) with a a bf16
    value.  The bf16 rounding moves x by far less than half a level spacing, so
    the codes are i again and the bf16 dequantized output is x bitwise."""
    l = codebook.nf4_levels()
    g = np.random.default_rng(31)
    B = 64
    xs, cs = [], []
    for _ in range(40):
        a_bits = floats.f32_to_bf16_bits(np.float32([abs(g.standard_normal()) * 0.05 + 1e-3]))
        a = floats.bf16_bits_to_f32(a_bits)[0]
        codes = g.integers(0, 16, B).astype(np.uint8)
        codes[0] = 15
        xs.append(floats.bf16_bits_to_f32(floats.f32_to_bf16_bits((l[codes] * a).astype(np.float32))))
        cs.append(codes)
    x = np.concatenate(xs)
    packed, amax = bw.quantize_blockwise(x, B, l)
    assert bw.unpack(packed, x.size).tolist() == np.concatenate(cs).tolist()
    yb = dequant.dequantize_bf16_bits(packed, x.size, B, l, amax)
    np.testing.assert_array_equal(yb, floats.f32_to_bf16_bits(x))


def test_block_counts_match_pages_and_edge_shape():
    # a 4096-wide row at blocksize 64 is 64 blocks
    assert bw.num_blocks(4096, 64) == 64
    n = 3000 * 4099
    assert [bw.num_blocks(n, B) for B in (64, 128, 256)] == [192141, 96071, 48036]
    assert [n - (bw.num_blocks(n, B) - 1) * B for B in (64, 128, 256)] == [40, 40, 40]
