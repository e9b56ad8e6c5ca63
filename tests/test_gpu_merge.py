"""GPU parity of qk_lora_merge (and of requantizing the merged weight) against
the oracle.  The merge is bit-exact by definition, so every comparison is
bitwise."""

import numpy as np
import pytest
import torch

import bit_blockwise_weight_amd as qk
import workloads
from oracle import blockwise as obw, codebook as ocb, dequant as odq, double_quant as odd, merge as omg
from tests.gpu_common import assert_bits_equal, dev_bf16, host, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _levels(kind):
    return ocb.nf4_levels() if kind == ocb.NF4 else ocb.fp4_levels()


def _oracle_merge(Wb, Ab, Bb, N, K, B, kind, nested, s):
    lv = _levels(kind)
    xf = workloads.bf16_bits_as_f32(Wb).reshape(-1)
    codes, absmax = obw.quantize_blockwise(xf, B, lv)
    if nested:
        q, sig, mu = odd.double_quant(absmax)
        aeff = odd.reconstruct_absmax(q, sig, mu)
    else:
        aeff = absmax
    D = odq.dequantize_bf16_bits(codes, N * K, B, lv, aeff).reshape(N, K)
    return omg.lora_merge_bf16_bits(D, Ab, Bb, s), D


def _gpu_state(Wb, N, K, B, kind, nested):
    w = dev_bf16(Wb).reshape(N, K)
    lv = torch.from_numpy(_levels(kind))
    return qk.quantize(w, B, kind, nested, lv)


@pytest.mark.parametrize("N,K,r,B,kind,nested", [
    (300, 512, 16, 64, ocb.NF4, True),       # vectorized path, one rank chunk
    (129, 1024, 40, 128, ocb.NF4, False),    # three rank chunks, the last partial
    (64, 256, 1, 256, ocb.FP4, True),        # rank 1
    (37, 4099, 5, 64, ocb.FP4, False),       # K % 8 != 0: per-element path, blocks straddle rows
    (3, 7, 3, 64, ocb.NF4, True),            # smaller than one tile
    (264, 512, 16, 64, ocb.NF4, True),       # 16-byte adapter staging (r % 8 == 0, N % 8 == 0), ragged rows
    (136, 1024, 40, 128, ocb.NF4, False),    # 16-byte adapter staging, rank chunks of 16, 16 and 8
    (40, 4099, 8, 64, ocb.FP4, False),       # 16-byte adapter staging with the per-element weight path
])
def test_merge_bit_exact(N, K, r, B, kind, nested):
    say(f"case: merge N={N} K={K} r={r} B={B} kind={kind} nested={nested}")
    Wb, Ab, Bb = workloads.lora_merge_case(N, K, r, tag=N * 7 + r)
    s = 2.0
    want, _ = _oracle_merge(Wb, Ab, Bb, N, K, B, kind, nested, s)
    qw = _gpu_state(Wb, N, K, B, kind, nested)
    guard = 64
    out_buf = torch.full((N * K + guard,), 3.0, dtype=torch.bfloat16, device="cuda")
    out = out_buf[:N * K].view(N, K)
    qk.qk_lora_merge(qw.state, dev_bf16(Ab).reshape(K, r), dev_bf16(Bb).reshape(r, N), s, out)
    got = host(out_buf.view(torch.int16)).view(np.uint16)
    assert_bits_equal(got[:N * K], want.reshape(-1), "merged weight")
    assert np.all(got[N * K:] == 0x4040), "guard band overwritten"


def test_merge_with_zero_adapter_equals_dequantize():
    N, K, r = 128, 512, 16
    Wb, Ab, _ = workloads.lora_merge_case(N, K, r, tag=1)
    qw = _gpu_state(Wb, N, K, 64, ocb.NF4, True)
    zeros = torch.zeros((r, N), dtype=torch.bfloat16, device="cuda")
    merged = qk.qk_lora_merge(qw.state, dev_bf16(Ab).reshape(K, r), zeros, 2.0)
    deq = qw.dequantize(torch.bfloat16).reshape(N, K)
    assert torch.equal(merged.view(torch.int16), deq.view(torch.int16))


def test_merge_then_requantize_matches_oracle():
    """The merge flow of the pages: dequantize, add the adapter, requantize (with
    double quantization), and read the result back."""
    N, K, r, B = 256, 1024, 16, 64
    say("case: merge + requantize 256x1024 r=16")
    Wb, Ab, Bb = workloads.lora_merge_case(N, K, r, tag=99)
    want_w, _ = _oracle_merge(Wb, Ab, Bb, N, K, B, ocb.NF4, True, 2.0)
    lv = _levels(ocb.NF4)
    want_c, want_a = obw.quantize_blockwise(workloads.bf16_bits_as_f32(want_w).reshape(-1), B, lv)
    q, sig, mu = odd.double_quant(want_a)
    want_back = odq.dequantize_f32(want_c, N * K, B, lv, odd.reconstruct_absmax(q, sig, mu))
    qw = _gpu_state(Wb, N, K, B, ocb.NF4, True)
    w_new, qw2 = qw.merge_lora(dev_bf16(Ab).reshape(K, r), dev_bf16(Bb).reshape(r, N), 2.0)
    assert_bits_equal(host(w_new.view(torch.int16)).view(np.uint16).reshape(-1), want_w.reshape(-1), "W_new")
    assert_bits_equal(host(qw2.codes), want_c, "requantized codes")
    assert_bits_equal(host(qw2.q8), q, "requantized q8")
    back = host(qw2.dequantize(torch.float32))
    assert_bits_equal(back, want_back, "requantized dequant")
    drift = omg.merge_drift(want_w, back)
    say(f"merge drift after requantization: rel_frobenius={drift['rel_frobenius']:.3e}")
    assert drift["rel_frobenius"] < 0.2


def test_merge_llama_shape_sampled_rows():
    """Full 4096 x 4096 merge at rank 16; the oracle checks 24 sampled rows (each
    row of W_new depends only on that row's codes, block scales and B column)."""
    N = K = 4096
    r, B = 16, 64
    say("case: merge 4096x4096 r=16, sampled rows")
    Wb, Ab, Bb = workloads.lora_merge_case(N, K, r, tag=4096)
    lv = _levels(ocb.NF4)
    qw = _gpu_state(Wb, N, K, B, ocb.NF4, True)
    out = qk.qk_lora_merge(qw.state, dev_bf16(Ab).reshape(K, r), dev_bf16(Bb).reshape(r, N), 2.0)
    got = host(out.view(torch.int16)).view(np.uint16)
    xf = workloads.bf16_bits_as_f32(Wb).reshape(-1)
    codes, absmax = obw.quantize_blockwise(xf, B, lv)
    q, sig, mu = odd.double_quant(absmax)
    aeff = odd.reconstruct_absmax(q, sig, mu)
    rows = np.random.default_rng(3).choice(N, 24, replace=False)
    for n in rows:
        cb = codes[n * K // 2:(n + 1) * K // 2]
        D = odq.dequantize_bf16_bits(cb, K, B, lv, aeff[n * K // B:(n + 1) * K // B]).reshape(1, K)
        want = omg.lora_merge_bf16_bits(D, Ab.reshape(K, r), Bb.reshape(r, N)[:, n:n + 1], 2.0)
        assert_bits_equal(got[n], want.reshape(-1), f"row {n}")
