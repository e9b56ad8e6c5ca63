"""GPU parity of qk_qlora_backward (input and adapter gradients of the QLoRA
layer) against the fp64 oracle, computed on the oracle's own bf16-dequantized
weight.

Tolerance (floating point, accumulation order free), per output: relative
Frobenius error <= 5e-3 and max abs error <= 2e-2 * max |ref|."""

import numpy as np
import pytest
import torch

import bit_blockwise_weight_amd as qk
import workloads
from oracle import backward as obw_, codebook as ocb, floats as ofl
from tests.gpu_common import bf16_bits_to_f32, dev_bf16, host, require_gpu, say
from tests.test_gpu_matmul import check_close, oracle_wd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _bits(g, shape, std):
    return ofl.f32_to_bf16_bits(g.standard_normal(shape).astype(np.float32) * np.float32(std))


def _run(dYb, Xb, Wb, Ab, Bb, M, N, K, r, B, kind, nested, s):
    qw = qk.quantize(dev_bf16(Wb).reshape(N, K), B, kind, double_quant=nested)
    dY = dev_bf16(dYb).reshape(M, N)
    if Ab is None:
        dX, dA, dB = qk.qk_qlora_backward(dY, qw.state)
        return host(dX), None, None, qw
    dX, dA, dB = qk.qk_qlora_backward(dY, qw.state, dev_bf16(Xb).reshape(M, K), dev_bf16(Ab).reshape(K, r),
                                      dev_bf16(Bb).reshape(r, N), s)
    return host(dX), dA.cpu().numpy(), dB.cpu().numpy(), qw


def _f(bits, *shape):
    return bf16_bits_to_f32(bits).reshape(*shape)


@pytest.mark.parametrize("M,N,K,B,r,kind,nested", [
    (128, 128, 64, 64, 16, ocb.NF4, True),       # K below one column tile
    (77, 128, 192, 128, 1, ocb.NF4, False),      # ragged M, rank 1, half a second column tile
    (300, 256, 320, 256, 64, ocb.NF4, True),     # maximum rank
    (1, 64, 512, 64, 16, ocb.FP4, True),         # one token row, one reduction step
    (129, 192, 1024, 64, 17, ocb.FP4, False),    # rank just past a 16 boundary
    (5, 64, 64, 256, 40, ocb.NF4, True),         # one column tile, three rank chunks of 16
])
def test_backward_small_and_ragged(M, N, K, B, r, kind, nested):
    say(f"case: backward M={M} N={N} K={K} B={B} r={r} kind={kind} nested={nested}")
    g = np.random.default_rng(M * 1000 + N + K + r)
    W, X, dY = _bits(g, (N, K), 0.02), _bits(g, (M, K), 1.0), _bits(g, (M, N), 1.0)
    A, Bm = _bits(g, (K, r), 0.01), _bits(g, (r, N), 0.01)
    s = 2.0
    dX, dA, dB, _ = _run(dY, X, W, A, Bm, M, N, K, r, B, kind, nested, s)
    wd = oracle_wd(W, N, K, B, kind, nested)
    rX, rA, rB = obw_.qlora_backward_f64(_f(dY, M, N), _f(X, M, K), wd, _f(A, K, r), _f(Bm, r, N), s)
    check_close(_f(dX, M, K), rX, "dX")
    check_close(dA, rA, "dA")
    check_close(dB, rB, "dB")


@pytest.mark.parametrize("nested", [True, False])
def test_backward_without_adapter(nested):
    M, N, K = 200, 320, 448
    g = np.random.default_rng(11)
    W, dY = _bits(g, (N, K), 0.02), _bits(g, (M, N), 1.0)
    dX, dA, dB, _ = _run(dY, None, W, None, None, M, N, K, 0, 64, ocb.NF4, nested, 0.0)
    assert dA is None and dB is None
    rX, _, _ = obw_.qlora_backward_f64(_f(dY, M, N), None, oracle_wd(W, N, K, 64, ocb.NF4, nested))
    check_close(_f(dX, M, K), rX, "dX base only")


def test_backward_lora_term_alone_with_zero_weight():
    """All-zero weight without double quantization dequantizes to exact zeros, so
    dX is s (dY B^T) A^T alone and its parity is not masked by the base term."""
    M, N, K, r = 256, 192, 320, 24
    g = np.random.default_rng(12)
    W = np.zeros((N, K), dtype=np.uint16)
    X, dY = _bits(g, (M, K), 1.0), _bits(g, (M, N), 1.0)
    A, Bm = _bits(g, (K, r), 0.01), _bits(g, (r, N), 0.01)
    dX, dA, dB, _ = _run(dY, X, W, A, Bm, M, N, K, r, 64, ocb.NF4, False, 2.0)
    rX, rA, rB = obw_.qlora_backward_f64(_f(dY, M, N), _f(X, M, K), np.zeros((N, K)), _f(A, K, r), _f(Bm, r, N), 2.0)
    check_close(_f(dX, M, K), rX, "dX lora only")
    check_close(dA, rA, "dA")
    check_close(dB, rB, "dB")


def test_backward_deterministic_and_in_bounds():
    """Two calls give the same bits; nothing is written past dX, dA or dB."""
    M, N, K, r = 130, 128, 256, 16
    g = np.random.default_rng(13)
    W, X, dY = _bits(g, (N, K), 0.02), _bits(g, (M, K), 1.0), _bits(g, (M, N), 1.0)
    A, Bm = _bits(g, (K, r), 0.01), _bits(g, (r, N), 0.01)
    qw = qk.quantize(dev_bf16(W).reshape(N, K), 64, ocb.NF4, double_quant=True)
    guard = 256
    outs = []
    for _ in range(2):
        dXb = torch.full((M * K + guard,), 3.0, dtype=torch.bfloat16, device="cuda")
        dAb = torch.full((K * r + guard,), 7.0, dtype=torch.float32, device="cuda")
        dBb = torch.full((r * N + guard,), 7.0, dtype=torch.float32, device="cuda")
        qk.qk_qlora_backward(dev_bf16(dY).reshape(M, N), qw.state, dev_bf16(X).reshape(M, K),
                             dev_bf16(A).reshape(K, r), dev_bf16(Bm).reshape(r, N), 2.0,
                             dX=dXb[:M * K].view(M, K), dA=dAb[:K * r].view(K, r), dB=dBb[:r * N].view(r, N))
        torch.cuda.synchronize()
        assert torch.all(dXb[M * K:] == 3.0) and torch.all(dAb[K * r:] == 7.0) and torch.all(dBb[r * N:] == 7.0)
        outs.append((dXb.view(torch.int16).cpu(), dAb.view(torch.int32).cpu(), dBb.view(torch.int32).cpu()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("N,K", [(4096, 4096), (11008, 4096), (4096, 11008)])
def test_backward_qlora_prefill_full_size(N, K):
    """X [4096, K], W [N, K] NF4 + DQ, LoRA r = 16, alpha / r = 2, dY [4096, N]
    (the layer set's three shapes): every element of dX, dA and dB."""
    say(f"case: backward qlora prefill N={N} K={K}")
    X, W, A, Bm = workloads.qlora_prefill(N, K=K)
    dY = workloads.qlora_upstream_grad(N)
    M, r = 4096, 16
    s = workloads.QLORA_ALPHA_OVER_R
    dX, dA, dB, _ = _run(dY, X, W, A, Bm, M, N, K, r, 64, ocb.NF4, True, s)
    wd = oracle_wd(W, N, K, 64, ocb.NF4, True)
    rX, rA, rB = obw_.qlora_backward_f64(_f(dY, M, N), _f(X, M, K), wd, _f(A, K, r), _f(Bm, r, N), s)
    check_close(_f(dX, M, K), rX, f"dX N={N} K={K}")
    check_close(dA, rA, f"dA N={N} K={K}")
    check_close(dB, rB, f"dB N={N} K={K}")
