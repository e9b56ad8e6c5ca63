"""GPU parity of the 8-bit blockwise quantization with the dynamic map
(qk_quantize_blockwise_8bit / qk_dequantize_blockwise_8bit) against the oracle.
Codes, absmax and dequantized values are compared bit for bit."""

import numpy as np
import pytest
import torch

import bit_blockwise_weight_amd as qk
import workloads
from oracle import blockwise8 as o8
from tests.gpu_common import assert_bits_equal, dev_f16, dev_f32, host, require_gpu, say
from oracle.floats import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _check(x_f32, B, signed, dtype="f32", levels=None):
    """Quantize x (given as fp32 values exactly representable in `dtype`) on the GPU
    and in the oracle, then dequantize both ways."""
    lv = o8.dynamic_map(signed) if levels is None else levels
    n = x_f32.size
    if dtype == "f32":
        xd = dev_f32(x_f32)
    elif dtype == "bf16":
        xd = torch.from_numpy(f32_to_bf16_bits(x_f32).view(np.int16)).view(torch.bfloat16).cuda()
    else:
        xd = dev_f16(x_f32)
    codes, am = qk.qk_quantize_blockwise_8bit(xd, B, torch.from_numpy(lv))
    wc, wa = o8.quantize_blockwise8(x_f32, B, lv)
    assert_bits_equal(host(codes), wc, "codes")
    assert_bits_equal(host(am), wa, "absmax")
    y = qk.qk_dequantize_blockwise_8bit(codes, am, B, torch.from_numpy(lv), torch.float32)
    wy = o8.dequantize_blockwise8(wc, wa, n, B, lv)
    assert_bits_equal(host(y), wy, "dequantized fp32")
    yb = qk.qk_dequantize_blockwise_8bit(codes, am, B, torch.from_numpy(lv), torch.bfloat16)
    assert_bits_equal(host(yb), f32_to_bf16_bits(wy), "dequantized bf16")


@pytest.mark.parametrize("B", [256, 512, 1024, 2048, 4096])
@pytest.mark.parametrize("signed", [True, False])
def test_adam_states_ragged(B, signed):
    n = 2048 * 9 + 1237
    m, v = workloads.adam_states(n, tag=B)
    say(f"case: quant8 adam states n={n} B={B} signed={signed}")
    _check(m if signed else v, B, signed)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_16bit_inputs(dtype):
    m, _ = workloads.adam_states(50000, tag=3)
    x = (m * np.float32(1000.0)).astype(np.float32)            # keep fp16 normal
    x = x.astype(np.float16).astype(np.float32) if dtype == "f16" else \
        (f32_to_bf16_bits(x).astype(np.uint32) << 16).view(np.float32)
    _check(x, 2048, True, dtype)


def _ulp_steps(f: np.float32, k: int) -> np.float32:
    toward = np.float32(np.inf) if k > 0 else np.float32(-np.inf)
    for _ in range(abs(k)):
        f = np.nextafter(f, toward)
    return f


@pytest.mark.parametrize("signed", [True, False])
def test_every_threshold_and_its_neighbours(signed):
    """t = x / 1 lands on and around every decision threshold (the binary32
    value nearest each exact midpoint and 4 binary32 steps on each side), in one
    block with absmax 1."""
    lv = o8.dynamic_map(signed).astype(np.float64)
    mids = (lv[:-1] + lv[1:]) / 2
    vals = [np.float32(1.0)]
    for m in mids:
        f = np.float32(m)
        vals += [_ulp_steps(f, k) for k in range(-4, 5)]
    x = np.array(vals, dtype=np.float32)
    x = x[np.abs(x) <= 1.0]
    say(f"case: quant8 thresholds signed={signed} n={x.size}")
    _check(x, 4096, signed)


def test_zero_blocks_tiny_and_single_element():
    x = np.zeros(5000, dtype=np.float32)
    x[2100:2110] = np.float32(3e-4)
    _check(x, 2048, True)                     # blocks 0 and 2 all zero: codes 127 (tie at 0), absmax 0
    _check(np.array([np.float32(-2.5e-3)]), 2048, True)
    _check(np.array([np.float32(7e-6)] * 3), 256, False)


def test_unsorted_custom_table():
    """A level table in an order that is not value order (the signed map reversed,
    then two entries swapped): ties and codes follow the smaller code."""
    lv = o8.dynamic_map(True)[::-1].copy()
    lv[[10, 200]] = lv[[200, 10]]
    m, _ = workloads.adam_states(20000, tag=5)
    _check(m, 2048, True, levels=lv)


def test_on_grid_round_trip():
    lv = o8.dynamic_map(True)
    x = np.tile((lv * np.float32(0.02)).astype(np.float32), 16)
    codes, am = qk.qk_quantize_blockwise_8bit(dev_f32(x), 256)
    assert np.array_equal(host(codes), np.tile(np.arange(256, dtype=np.uint8), 16))
    y = qk.qk_dequantize_blockwise_8bit(codes, am, 256)
    assert_bits_equal(host(y), x, "round trip")


def test_full_size_states_sampled_blocks():
    """m and v of the Llama-7B layer set's 202,375,168 parameters (fp32, drawn on
    the device), block 2048: 64 sampled blocks of each against the oracle, and
    every block's absmax against torch's own max."""
    n = workloads.LLAMA7B_LAYER_PARAMS
    B = 2048
    m, v = workloads.device_adam_states(n, seed=1)
    for x, signed in ((m, True), (v, False)):
        lv = o8.dynamic_map(signed)
        say(f"case: quant8 full size n={n} signed={signed}")
        codes, am = qk.qk_quantize_blockwise_8bit(x, B, torch.from_numpy(lv))
        nb = (n + B - 1) // B
        pad = torch.zeros(nb * B - n, device="cuda")
        ref_am = torch.cat([x.abs(), pad]).view(nb, B).amax(dim=1)
        assert torch.equal(am, ref_am)
        blocks = np.random.default_rng(11).choice(nb, size=64, replace=False)
        for j in blocks:
            lo, hi = int(j) * B, min((int(j) + 1) * B, n)
            xs = host(x[lo:hi])
            wc, wa = o8.quantize_blockwise8(xs, B, lv)
            assert_bits_equal(host(codes[lo:hi]), wc, f"codes block {j}")
            assert host(am[j:j + 1])[0] == wa[0]
        y = qk.qk_dequantize_blockwise_8bit(codes, am, B, torch.from_numpy(lv))
        for j in blocks[:16]:
            lo, hi = int(j) * B, min((int(j) + 1) * B, n)
            wy = o8.dequantize_blockwise8(host(codes[lo:hi]), host(am[j:j + 1]), hi - lo, B, lv)
            assert_bits_equal(host(y[lo:hi]), wy, f"dequantized block {j}")
        del codes, am, y
    del m, v
    torch.cuda.empty_cache()
