"""GPU parity of quantize, double quantization and dequantization against the
CPU oracle: bit-exact codes, absmax, q8 / scale / mean and dequantized values."""

import numpy as np
import pytest
import torch

import bit_blockwise_weight_amd as qk
import workloads
from oracle import blockwise as obw, codebook as ocb, dequant as odq, double_quant as odd, floats as ofl
from tests.gpu_common import (assert_bits_equal, bf16_bits_to_f32, dev_bf16, dev_f16, dev_f32, host,
                              require_gpu, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _levels(kind):
    return ocb.levels(kind)


def _run_quant(x_dev, B, kind):
    lv = torch.from_numpy(_levels(kind))
    codes, absmax = qk.qk_quantize_blockwise(x_dev, B, lv)
    torch.cuda.synchronize()
    return host(codes), host(absmax)


def _check_quant(x_f32, x_dev, B, kind, what):
    codes, absmax = _run_quant(x_dev, B, kind)
    want_codes, want_absmax = obw.quantize_blockwise(x_f32, B, _levels(kind))
    assert_bits_equal(absmax, want_absmax, f"{what} absmax")
    assert_bits_equal(codes, want_codes, f"{what} codes")
    return codes, absmax


def test_single_1024_quantize_dq_dequant():
    say("case: single_1024 NF4 B=64 + DQ")
    W, _ = workloads.single_1024()
    xf = bf16_bits_to_f32(W).reshape(-1)
    xd = dev_bf16(W)
    codes, absmax = _check_quant(xf, xd, 64, ocb.NF4, "single_1024")
    q8, scale, mean = qk.qk_double_quant(dev_f32(absmax))
    torch.cuda.synchronize()
    oq, osig, omu = odd.double_quant(absmax)
    assert_bits_equal(host(mean), np.float32([omu]), "mean")
    assert_bits_equal(host(scale), osig, "dq scale")
    assert_bits_equal(host(q8), oq, "q8")
    lv = _levels(ocb.NF4)
    st = qk.qk_state_init(qk.NF4, lv, 1024, 1024, 64, dev_u8(codes), None, q8, scale, mean)
    for dt in (torch.bfloat16, torch.float32):
        y = host(qk.qk_dequantize(st, dt))
        a_eff = odd.reconstruct_absmax(oq, osig, omu)
        want = odq.dequantize_f32(codes, xf.size, 64, lv, a_eff)
        if dt == torch.bfloat16:
            want = ofl.f32_to_bf16_bits(want)
        assert_bits_equal(y, want, f"dequant {dt}")


def test_double_quant_ties_and_wide_mean_sum():
    """The absmax arrays that pin the oracle's double quantization: ties of
    RN(RN(c/s)*127) at +-0.5, +-2.5, +-1.5 (half-even: 0, 0, 2, -2, 2, -2) and a
    mean whose fp64 sum 1 + 2^-24 needs 25 bits (one fp32 ulp above 0.2).  Each
    is also repeated past one DQ block and past one tree-partial chunk."""
    ties = np.float32(200.0) + np.float32([127.0, -127.0, 0.5, -0.5, 2.5, -2.5, 1.5, -1.5])
    wide = np.float32([1.0, 2.0 ** -24, 0.0, 0.0, 0.0])
    for name, a in (("ties", ties), ("wide-sum mean", wide), ("ties x 700", np.tile(ties, 700)),
                    ("ties x 1200", np.tile(ties, 1200))):
        say(f"case: double quant {name}, nb={a.size}")
        q8, scale, mean = qk.qk_double_quant(dev_f32(a))
        torch.cuda.synchronize()
        oq, osig, omu = odd.double_quant(a)
        assert_bits_equal(host(mean), np.float32([omu]), f"{name} mean")
        assert_bits_equal(host(scale), osig, f"{name} scale")
        assert_bits_equal(host(q8), oq, f"{name} q8")
    assert oq[:8].tolist() == [127, -127, 0, 0, 2, -2, 2, -2]


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


@pytest.fixture(scope="module")
def edge_weight():
    W = workloads.edge_weight()
    return W, bf16_bits_to_f32(W).reshape(-1)


@pytest.mark.parametrize("B", [64, 128, 256])
@pytest.mark.parametrize("kind", [ocb.NF4, ocb.FP4])
def test_edge_3000x4099_all_steps(edge_weight, B, kind):
    say(f"case: edge_3000x4099 B={B} kind={kind}")
    W, xf = edge_weight
    xd = dev_bf16(W)
    codes, absmax = _check_quant(xf, xd, B, kind, f"edge B={B} kind={kind}")
    nb = absmax.size
    assert nb == (xf.size + B - 1) // B
    assert int((absmax == 0).sum()) >= int(0.0099 * (nb - 1))   # the zeroed blocks are there
    lv = _levels(kind)
    # plain state
    st = qk.qk_state_init(kind, lv, 3000, 4099, B, dev_u8(codes), dev_f32(absmax))
    y = host(qk.qk_dequantize(st, torch.bfloat16))
    assert_bits_equal(y, odq.dequantize_bf16_bits(codes, xf.size, B, lv, absmax), "dequant plain bf16")
    # nested state
    q8, scale, mean = qk.qk_double_quant(dev_f32(absmax))
    oq, osig, omu = odd.double_quant(absmax)
    assert_bits_equal(host(mean), np.float32([omu]), "mean")
    assert_bits_equal(host(scale), osig, "scale")
    assert_bits_equal(host(q8), oq, "q8")
    st2 = qk.qk_state_init(kind, lv, 3000, 4099, B, dev_u8(codes), None, q8, scale, mean)
    y2 = host(qk.qk_dequantize(st2, torch.float32))
    assert_bits_equal(y2, odq.dequantize_f32(codes, xf.size, B, lv, odd.reconstruct_absmax(oq, osig, omu)),
                      "dequant nested f32")


def _near_midpoint_values(kind):
    lv = _levels(kind)
    u = sorted(set(float(v) for v in lv))
    vals = []
    for a, b in zip(u[:-1], u[1:]):
        m = np.float32((a + b) / 2)
        cur = m
        for _ in range(6):
            cur = np.nextafter(cur, np.float32(-2), dtype=np.float32)
        for _ in range(13):
            vals.append(cur)
            cur = np.nextafter(cur, np.float32(2), dtype=np.float32)
    vals += [np.float32(v) for v in lv]
    vals += [np.float32(0.0), np.float32(-0.0), np.float32(1e-45), np.float32(-1e-45), np.float32(1e-39)]
    return np.array(vals, dtype=np.float32)


@pytest.mark.parametrize("kind", [ocb.NF4, ocb.FP4])
def test_fp32_input_ties_and_midpoints(kind):
    """fp32 input, absmax 1 in every block: t = x exactly, so every fp32 value
    within 6 ulp of every decision midpoint is probed, ties included."""
    say(f"case: fp32 midpoints kind={kind}")
    vals = _near_midpoint_values(kind)
    B = 64
    per = B - 1
    nblk = (vals.size + per - 1) // per
    x = np.zeros(nblk * B, dtype=np.float32)
    for j in range(nblk):
        chunk = vals[j * per:(j + 1) * per]
        x[j * B] = 1.0
        x[j * B + 1: j * B + 1 + chunk.size] = chunk
    _check_quant(x, dev_f32(x), B, kind, "fp32 midpoints")
    # the same values scaled by an absmax of 3 (t is then a rounded quotient)
    x3 = (x * np.float32(3)).astype(np.float32)
    _check_quant(x3, dev_f32(x3), B, kind, "fp32 midpoints x3")


@pytest.mark.parametrize("kind", [ocb.NF4, ocb.FP4])
def test_bf16_input_hard_cases(kind):
    """bf16 inputs that exercise every division path: ordinary blocks, blocks
    with a subnormal element (IEEE fallback), absmax outside [2^-36, 2^64]
    (IEEE fallback), subnormal absmax, zero blocks, signed zeros, and values
    whose quotient lands next to a decision midpoint."""
    say(f"case: bf16 hard cases kind={kind}")
    g = np.random.default_rng(77 + kind)
    B = 64
    blocks = []
    for scale in [1.0, 1e-3, 2.0 ** -30, 2.0 ** -37, 2.0 ** -100, 2.0 ** -126, 2.0 ** 63, 2.0 ** 65, 2.0 ** 100]:
        for _ in range(8):
            blocks.append(g.standard_normal(B).astype(np.float32) * np.float32(scale))
    blk = g.standard_normal(B).astype(np.float32)
    blk[5] = 1e-40      # subnormal element in an ordinary block
    blk[6] = -3e-39
    blocks.append(blk)
    blocks.append(np.zeros(B, dtype=np.float32))
    z = np.zeros(B, dtype=np.float32)
    z[::2] = -0.0
    blocks.append(z)
    blocks.append(np.full(B, 1e-41, dtype=np.float32))   # subnormal absmax
    # bf16 values nearest to each midpoint times a few absmax values
    mids = _near_midpoint_values(kind)
    for a in [1.0, 0.75, 0.02, 3.0]:
        v = (mids * np.float32(a)).astype(np.float32)
        for j in range(0, v.size, B - 1):
            b = np.zeros(B, dtype=np.float32)
            b[0] = a
            c = v[j:j + B - 1]
            b[1:1 + c.size] = c
            blocks.append(b)
    x = np.concatenate(blocks)
    bits = ofl.f32_to_bf16_bits(x)
    xf = bf16_bits_to_f32(bits)
    _check_quant(xf, dev_bf16(bits), B, kind, "bf16 hard cases")
    # the same values as fp16 where they fit (fp16 path)
    h = xf[np.abs(xf) < 60000].astype(np.float16)
    hf = h.astype(np.float32)
    n = (hf.size // B) * B
    _check_quant(hf[:n], dev_f16(hf[:n]), B, kind, "fp16 hard cases")


# A level table whose two smallest levels are -2^-40 and 2^-40: their decision threshold
# is the least positive float (a tie at t = 0 goes to the smaller code), so the code of an
# element far below its block's absmax depends on its sign and on whether its quotient
# rounds to zero.  For such a table the kernel divides exactly (IEEE) for those elements;
# for FP4, whose thresholds are all far from 0, it does not need to.  (NF4 has the
# same kind of threshold at 0, between its two middle levels +-0.0396.)
_ZERO_THRESHOLD_LEVELS = np.array([-1, -0.75, -0.5, -0.375, -0.25, -0.125, -0.0625, -2.0 ** -40,
                                   2.0 ** -40, 0.0625, 0.125, 0.25, 0.375, 0.5, 0.75, 1], dtype=np.float32)


@pytest.mark.parametrize("order", ["sorted", "shuffled"])
def test_bf16_tiny_elements_with_a_threshold_at_zero(order):
    say(f"case: bf16 tiny elements, level table with a threshold at zero ({order})")
    lv = _ZERO_THRESHOLD_LEVELS.copy()
    if order == "shuffled":
        lv = lv[np.random.default_rng(3).permutation(16)]
    g = np.random.default_rng(41)
    B = 64
    tiny = np.array([2.0 ** -133, -(2.0 ** -133), 3 * 2.0 ** -133, 2.0 ** -130, -(2.0 ** -127), 2.0 ** -100,
                     -(2.0 ** -90), 0.0, -0.0, 1e-30, -1e-25, 2.0 ** -126, -(2.0 ** -126)], dtype=np.float32)
    blocks = []
    for a in [1.0, 3.0, 0.75, 2.0 ** -20, 5.0, 2.0 ** 40]:
        for rep in range(4):
            b = (g.standard_normal(B) * 0.3).astype(np.float32) * np.float32(a)
            b[0] = np.float32(a) * np.float32(1.5)
            idx = g.choice(np.arange(1, B), size=tiny.size, replace=False)
            b[idx] = tiny * np.float32(1 + rep)
            blocks.append(b)
    x = np.concatenate(blocks)
    bits = ofl.f32_to_bf16_bits(x)
    xf = bf16_bits_to_f32(bits)
    codes, absmax = qk.qk_quantize_blockwise(dev_bf16(bits), B, torch.from_numpy(lv))
    torch.cuda.synchronize()
    want_codes, want_absmax = obw.quantize_blockwise(xf, B, lv)
    assert_bits_equal(host(absmax), want_absmax, "absmax")
    assert_bits_equal(host(codes), want_codes, "codes")
    # the tiny elements do not all get one code: the table really separates them
    nib = np.stack([host(codes) >> 4, host(codes) & 15], axis=1).reshape(-1)[:xf.size]
    tiny_pos = np.abs(xf) < np.float32(2.0 ** -80)
    assert len(set(nib[tiny_pos].tolist())) == 2


# 2048 = one 32-element-per-lane unit of the dequantization; 18_532 and 61_447 leave
# 9 and 30 whole units (not a multiple of 8) and a tail that starts inside a
# double-quantization block (at block 288 or 960 of 64 elements)
@pytest.mark.parametrize("n", [1, 2, 7, 63, 64, 65, 511, 512, 513, 1023, 2047, 2048, 2049, 18_532, 61_447,
                               100_001, 1_000_003])
def test_ragged_sizes_and_guard_bands(n):
    say(f"case: ragged n={n}")
    g = np.random.default_rng(n)
    bits = ofl.f32_to_bf16_bits(g.standard_normal(n).astype(np.float32) * np.float32(0.05))
    xf = bf16_bits_to_f32(bits)
    lv = _levels(ocb.NF4)
    for B in (64, 256):
        nbytes = (n + 1) // 2
        nb = (n + B - 1) // B
        guard = 64
        codes_buf = torch.full((nbytes + guard,), 0xAB, dtype=torch.uint8, device="cuda")
        absmax_buf = torch.full((nb + guard,), -7.0, dtype=torch.float32, device="cuda")
        qk.qk_quantize_blockwise(dev_bf16(bits), B, torch.from_numpy(lv), codes_buf[:nbytes], absmax_buf[:nb])
        torch.cuda.synchronize()
        cb, ab = host(codes_buf), host(absmax_buf)
        want_c, want_a = obw.quantize_blockwise(xf, B, lv)
        assert_bits_equal(cb[:nbytes], want_c, f"codes n={n} B={B}")
        assert_bits_equal(ab[:nb], want_a, f"absmax n={n} B={B}")
        assert np.all(cb[nbytes:] == 0xAB), "codes guard band overwritten"
        assert np.all(ab[nb:] == -7.0), "absmax guard band overwritten"
        # double quant and dequant with guard bands
        q8_buf = torch.full((nb + guard,), 55, dtype=torch.int8, device="cuda")
        nd = (nb + 255) // 256
        sc_buf = torch.full((nd + guard,), -3.0, dtype=torch.float32, device="cuda")
        mean = torch.empty(1, dtype=torch.float32, device="cuda")
        qk.qk_double_quant(absmax_buf[:nb], 256, q8_buf[:nb], sc_buf[:nd], mean)
        oq, osig, omu = odd.double_quant(want_a)
        assert_bits_equal(host(q8_buf)[:nb], oq, "q8")
        assert_bits_equal(host(sc_buf)[:nd], osig, "scale")
        assert np.all(host(q8_buf)[nb:] == 55) and np.all(host(sc_buf)[nd:] == -3.0)
        assert host(mean)[0] == omu
        st = qk.qk_state_init(qk.NF4, lv, 1, n, B, codes_buf[:nbytes], None, q8_buf[:nb], sc_buf[:nd], mean)
        out = torch.full((n + 64,), 12345.0, dtype=torch.float32, device="cuda")
        qk.qk_dequantize(st, torch.float32, out[:n])
        want_y = odq.dequantize_f32(want_c, n, B, lv, odd.reconstruct_absmax(oq, osig, omu))
        yo = host(out)
        assert_bits_equal(yo[:n], want_y, "dequant")
        assert np.all(yo[n:] == 12345.0), "dequant guard band overwritten"


@pytest.mark.parametrize("offset", [0, 4, 8, 12])
def test_dequant_codes_alignment(offset):
    """Codes only need 4-byte alignment in a state: at every alignment the
    dequantization (bf16 and fp32, a partial last unit) must match the oracle."""
    n = 3 * 2048 + 517
    say(f"case: dequant codes offset {offset}, n={n}")
    g = np.random.default_rng(77 + offset)
    bits = ofl.f32_to_bf16_bits(g.standard_normal(n).astype(np.float32) * np.float32(0.02))
    xf = bf16_bits_to_f32(bits)
    lv = _levels(ocb.NF4)
    B = 64
    nbytes, nb = (n + 1) // 2, (n + B - 1) // B
    codes_buf = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    codes = codes_buf[offset:offset + nbytes]
    absmax = torch.empty(nb, dtype=torch.float32, device="cuda")
    qk.qk_quantize_blockwise(dev_bf16(bits), B, torch.from_numpy(lv), codes, absmax)
    want_c, want_a = obw.quantize_blockwise(xf, B, lv)
    assert_bits_equal(host(codes), want_c, "codes")
    st = qk.qk_state_init(qk.NF4, lv, 1, n, B, codes, absmax)
    want_y = odq.dequantize_f32(want_c, n, B, lv, want_a)
    out32 = torch.full((n + 64,), 999.0, dtype=torch.float32, device="cuda")
    qk.qk_dequantize(st, torch.float32, out32[:n])
    y = host(out32)
    assert_bits_equal(y[:n], want_y, "fp32 dequant")
    assert np.all(y[n:] == 999.0), "fp32 guard band overwritten"
    out16 = torch.full((n + 64,), 7.0, dtype=torch.bfloat16, device="cuda")
    qk.qk_dequantize(st, torch.bfloat16, out16[:n])
    y16 = host(out16.view(torch.int16)).view(np.uint16)
    assert_bits_equal(y16[:n], ofl.f32_to_bf16_bits(want_y), "bf16 dequant")
    assert np.all(y16[n:] == 0x40E0), "bf16 guard band overwritten"


def test_deterministic_repeat():
    W, _ = workloads.single_1024()
    xd = dev_bf16(W)
    a = [host(t) for t in qk.qk_quantize_blockwise(xd, 64)]
    b = [host(t) for t in qk.qk_quantize_blockwise(xd, 64)]
    assert_bits_equal(a[0], b[0], "codes repeat")
    assert_bits_equal(a[1], b[1], "absmax repeat")


def test_llama70b_largest_matrix_sampled():
    """The largest matrix of the 70B-shaped stack, [28672, 8192] ~ N(0, 0.015),
    drawn on the device; sampled DQ-aligned regions are checked against the
    oracle, the mean against the oracle's tree over the whole absmax array."""
    say("case: llama70b [28672, 8192] sampled")
    N, K = 28672, 8192
    w = workloads.device_normal_bf16((N, K), 0.015, workloads.llama70b_seed(0, 4))
    qw = qk.quantize(w, 64, qk.NF4, double_quant=False)
    q8, scale, mean = qk.qk_double_quant(qw.absmax)
    torch.cuda.synchronize()
    absmax = host(qw.absmax)
    oq, osig, omu = odd.double_quant(absmax)
    assert_bits_equal(host(mean), np.float32([omu]), "mean")
    assert_bits_equal(host(scale), osig, "scale")
    assert_bits_equal(host(q8), oq, "q8")
    g = np.random.default_rng(5)
    flat = w.view(-1)
    codes = qw.codes
    lv = _levels(ocb.NF4)
    region = 256 * 64        # one DQ block of absmax = 16384 elements
    for r in g.choice(N * K // region, size=24, replace=False):
        e0 = int(r) * region
        xs = bf16_bits_to_f32(host(flat[e0:e0 + region]))
        want_c, want_a = obw.quantize_blockwise(xs, 64, lv)
        assert_bits_equal(host(codes[e0 // 2:(e0 + region) // 2]), want_c, f"codes region {r}")
        assert_bits_equal(absmax[e0 // 64:(e0 + region) // 64], want_a, f"absmax region {r}")
