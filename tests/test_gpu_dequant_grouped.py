"""GPU parity of qk_dequantize_grouped: the dequantization of several states in
as few launches as their level tables allow.  Every output must equal, bit for
bit, what qk_dequantize of that state alone writes and what the oracle gives."""

import numpy as np
import pytest
import torch

import bit_blockwise_weight_amd as qk
from oracle import blockwise as obw, codebook as ocb, dequant as odq, double_quant as odd, floats as ofl
from tests.gpu_common import assert_bits_equal, bf16_bits_to_f32, dev_bf16, host, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _weights(g, shapes):
    out = []
    for (N, K, B, kind, nested) in shapes:
        bits = ofl.f32_to_bf16_bits(g.standard_normal(N * K).astype(np.float32) * np.float32(0.02))
        qw = qk.quantize(dev_bf16(bits).reshape(N, K), B, kind, double_quant=nested)
        out.append((bits, qw, N, K, B, kind, nested))
    return out


def _oracle_f32(bits, N, K, B, kind, nested):
    xf = bf16_bits_to_f32(bits)
    lv = ocb.levels(kind)
    codes, amax = obw.quantize_blockwise(xf, B, lv)
    if nested:
        q, sig, mu = odd.double_quant(amax)
        amax = odd.reconstruct_absmax(q, sig, mu)
    return odq.dequantize_f32(codes, N * K, B, lv, amax)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_grouped_mixed_tables_blocks_nesting_and_ragged(dtype):
    """NF4 and FP4 (two launches), blocks 64 / 128 / 256, nested or not, sizes that
    end inside a turn, inside a unit and inside a code word, 20 arrays of one table
    (more than the 16 a launch takes)."""
    say(f"case: grouped dequant mixed {dtype}")
    g = np.random.default_rng(31)
    shapes = [(33, 64, 64, ocb.NF4, True), (100, 128, 128, ocb.NF4, False), (64, 256, 256, ocb.FP4, True),
              (257, 1024, 64, ocb.NF4, True), (31, 192, 64, ocb.FP4, False), (500, 2752, 64, ocb.NF4, True),
              (7, 333, 64, ocb.NF4, True), (1, 64, 64, ocb.NF4, False)]
    shapes += [(16 * (i + 1) + i % 3, 64 * (1 + i % 5), 64, ocb.NF4, True) for i in range(14)]
    ws = _weights(g, shapes)
    outs = qk.qk_dequantize_grouped([w[1].state for w in ws], dtype)
    singles = [qk.qk_dequantize(w[1].state, dtype) for w in ws]
    torch.cuda.synchronize()
    for i, ((bits, qw, N, K, B, kind, nested), o, o1) in enumerate(zip(ws, outs, singles)):
        ho, h1 = host(o), host(o1)
        if dtype == torch.bfloat16:
            ho, h1 = ho.view(np.uint16), h1.view(np.uint16)
        assert_bits_equal(ho, h1, f"task {i} grouped vs alone")
        want = _oracle_f32(bits, N, K, B, kind, nested)
        if dtype == torch.bfloat16:
            want = ofl.f32_to_bf16_bits(want)
        assert_bits_equal(ho, want, f"task {i} [{N}x{K}] B={B} vs oracle")


def test_grouped_outputs_written_exactly():
    """Guard bands around each output stay untouched."""
    say("case: grouped dequant guard bands")
    g = np.random.default_rng(32)
    ws = _weights(g, [(37, 128, 64, ocb.NF4, True), (300, 512, 64, ocb.NF4, True)])
    bufs = [torch.full((w[2] * w[3] + 64,), 1.5, dtype=torch.bfloat16, device="cuda") for w in ws]
    outs = [b[32:32 + w[2] * w[3]] for b, w in zip(bufs, ws)]
    qk.qk_dequantize_grouped([w[1].state for w in ws], torch.bfloat16, outs)
    torch.cuda.synchronize()
    for b, w in zip(bufs, ws):
        hb = host(b).view(np.uint16)
        n = w[2] * w[3]
        assert np.all(hb[:32] == 0x3FC0) and np.all(hb[32 + n:] == 0x3FC0), "guard band overwritten"
