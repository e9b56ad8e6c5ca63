"""GPU parity of LLM.int8() (qk_int8_quantize_rows, qk_int8_outlier_columns,
qk_int8_matmul) against the oracle: int8 codes, absmax, column maxima and the
outlier list bit for bit; the fp16 output within rel. Frobenius 5e-3 and max
error 2e-2 * max |ref| of the fp64 reference."""

import numpy as np
import pytest
import torch

import bit_blockwise_weight_amd as qk
import workloads
from oracle import int8 as oi
from oracle import matmul as omm
from oracle.floats import f32_to_bf16_bits
from tests.gpu_common import assert_bits_equal, bf16_bits_to_f32, dev_bf16, dev_f16, dev_f32, host, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def check_close(got, ref, what):
    rf = omm.rel_frobenius(got, ref)
    mx = omm.max_rel_to_peak(got, ref)
    say(f"  {what}: rel_frob {rf:.2e} max/peak {mx:.2e}")
    assert rf <= omm.REL_FROB_TOL, f"{what}: rel Frobenius {rf}"
    assert mx <= omm.MAX_REL_TOL, f"{what}: max error / peak {mx}"


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_row_quantization_bit_exact(dtype):
    g = np.random.default_rng(1)
    x = (g.standard_normal((37, 200)) * 3).astype(np.float32)
    x[5] = 0.0
    if dtype == "f16":
        x = x.astype(np.float16).astype(np.float32)
        xd = dev_f16(x)
    elif dtype == "bf16":
        bits = f32_to_bf16_bits(x)
        x = bf16_bits_to_f32(bits).reshape(x.shape)
        xd = dev_bf16(bits).reshape(x.shape)
    else:
        xd = dev_f32(x)
    skip = np.zeros(200, dtype=np.uint8)
    skip[[3, 77, 199]] = 1
    for sk in (None, skip):
        q, a = qk.qk_int8_quantize_rows(xd, None if sk is None else torch.from_numpy(sk).cuda())
        wq, wa = oi.quantize_rows(x, None if sk is None else sk == 0)
        assert_bits_equal(host(q).view(np.uint8), wq.view(np.uint8), "q")
        assert_bits_equal(host(a), wa, "absmax")


def test_outlier_columns_page_example():
    """X[:, 17] reaches 7.2, every other column stays below 6.0: column 17 alone."""
    g = np.random.default_rng(2)
    x = np.clip(g.standard_normal((16, 64)), -5.9, 5.9).astype(np.float16).astype(np.float32)
    x[3, 17] = np.float32(np.float16(7.2))
    colmax, flags, idx, count = qk.qk_int8_outlier_columns(dev_f16(x), 6.0)
    assert int(host(count)[0]) == 1 and int(host(idx)[0]) == 17
    assert np.flatnonzero(host(flags)).tolist() == [17]
    assert_bits_equal(host(colmax), np.abs(x).max(axis=0), "colmax")
    _, flags0, _, count0 = qk.qk_int8_outlier_columns(dev_f16(x), 0.0)
    assert int(host(count0)[0]) == 0 and not host(flags0).any()


def test_outlier_list_many_columns_in_order():
    x, cols = workloads.int8_activations(300, 8192, frac=0.01, tag=1)
    colmax, flags, idx, count = qk.qk_int8_outlier_columns(dev_f16(x), 6.0)
    want = np.flatnonzero(oi.outlier_columns(x, 6.0))
    n = int(host(count)[0])
    assert n == want.size and np.array_equal(host(idx)[:n], want)
    assert set(cols.tolist()) <= set(want.tolist())
    assert_bits_equal(host(colmax), np.abs(x).max(axis=0), "colmax")


def _run(x, w_bits, N, K, threshold):
    W = dev_bf16(w_bits).reshape(N, K)
    CB, SCB = qk.qk_int8_quantize_rows(W)
    xd = dev_f16(x)
    if threshold > 0:
        _, flags, idx, count = qk.qk_int8_outlier_columns(xd, threshold)
        Xq, SX = qk.qk_int8_quantize_rows(xd, flags)
        Y = qk.qk_int8_matmul(Xq, SX, CB, SCB, xd, idx, count)
    else:
        Xq, SX = qk.qk_int8_quantize_rows(xd)
        Y = qk.qk_int8_matmul(Xq, SX, CB, SCB)
    return host(Y).astype(np.float32), host(Xq), host(SX), host(CB), host(SCB)


@pytest.mark.parametrize("M,N,K,frac", [(1, 64, 16, 0.0), (77, 100, 144, 0.02), (300, 257, 512, 0.01),
                                        (128, 128, 4096, 0.001), (513, 130, 1040, 0.03)])
def test_matmul_small_and_ragged(M, N, K, frac):
    say(f"case: int8 matmul M={M} N={N} K={K} frac={frac}")
    x, _ = workloads.int8_activations(M, K, frac=frac, tag=M + K) if frac > 0 else (
        np.random.default_rng(M).standard_normal((M, K)).astype(np.float16).astype(np.float32), None)
    w_bits = workloads.lora_merge_case(N, K, 1, tag=N)[0]
    wf = bf16_bits_to_f32(w_bits).reshape(N, K)
    Y, Xq, SX, CB, SCB = _run(x, w_bits, N, K, 6.0)
    wCB, wSCB = oi.quantize_rows(wf)
    assert_bits_equal(CB.view(np.uint8), wCB.view(np.uint8), "CB")
    assert_bits_equal(SCB, wSCB, "SCB")
    ref, out, wXq, wSX = oi.int8_matmul_f64(x, wCB, wSCB, 6.0)
    assert_bits_equal(Xq.view(np.uint8), wXq.view(np.uint8), "Xq")
    assert_bits_equal(SX, wSX, "SX")
    check_close(Y, ref, "Y")


def test_matmul_many_outliers_and_no_decomposition():
    M, N, K = 200, 192, 1024
    x, _ = workloads.int8_activations(M, K, frac=0.04, tag=9)        # 41 outlier columns: 3 chunks of 16
    w_bits = workloads.lora_merge_case(N, K, 1, tag=9)[0]
    wCB, wSCB = oi.quantize_rows(bf16_bits_to_f32(w_bits).reshape(N, K))
    Y, *_ = _run(x, w_bits, N, K, 6.0)
    ref, out, _, _ = oi.int8_matmul_f64(x, wCB, wSCB, 6.0)
    assert out.sum() >= 33
    check_close(Y, ref, "Y mixed")
    Y0, *_ = _run(x, w_bits, N, K, 0.0)
    ref0, out0, _, _ = oi.int8_matmul_f64(x, wCB, wSCB, 0.0)
    assert not out0.any()
    check_close(Y0, ref0, "Y int8 only")


@pytest.mark.parametrize("N", [4096, 11008])
def test_matmul_full_size_sampled_rows(N):
    """X [4096, 4096] fp16 with 0.1% outlier columns (x20), threshold 6; the QLoRA
    prefill weight W [N, 4096]: 256 sampled rows of Y, Xq and SX against the oracle."""
    M, K = 4096, 4096
    say(f"case: int8 matmul full size N={N}")
    x, cols = workloads.int8_activations(M, K, tag=N)
    _, w_bits, _, _ = workloads.qlora_prefill(N)
    Y, Xq, SX, CB, SCB = _run(x, w_bits, N, K, 6.0)
    out = oi.outlier_columns(x, 6.0)
    assert set(np.flatnonzero(out).tolist()) >= set(cols.tolist())
    wCB, wSCB = oi.quantize_rows(bf16_bits_to_f32(w_bits).reshape(N, K))
    assert_bits_equal(CB.view(np.uint8), wCB.view(np.uint8), "CB")
    rows = np.sort(np.random.default_rng(N).choice(M, size=256, replace=False))
    ref, wXq, wSX = oi.decomposed_product_f64(x[rows], out, wCB, wSCB)
    assert_bits_equal(Xq[rows].view(np.uint8), wXq.view(np.uint8), "Xq rows")
    assert_bits_equal(SX[rows], wSX, "SX rows")
    check_close(Y[rows], ref, f"Y rows N={N}")
