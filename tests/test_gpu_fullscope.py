"""Full-scope bit-exact parity of the quantized state on the large workloads: for
every weight of the Llama-7B layer set, both QLoRA prefill weights and all seven
matrices of one layer of the 70B-shaped stack, the codes, the absmax array, the
double-quantization state (q8, scales, mean) and the bf16 dequantized weight are
compared whole, element by element, with the CPU oracle.  (The GEMV and GEMM
tests check the products; these check every stored bit.)  The 70B-stack checks
spread the oracle over host cores; the weights of that stack are drawn on the
device (torch Philox) and copied back as the oracle's input."""

import numpy as np
import pytest
import torch

import bit_blockwise_weight_amd as qk
import workloads
from oracle import codebook as ocb, dequant as odq, double_quant as odd
from tests import parallel_oracle as par
from tests.gpu_common import assert_bits_equal, dev_bf16, host, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _check_whole(w_dev: torch.Tensor, w_bits: np.ndarray, what: str, parallel: bool):
    N, K = w_dev.shape
    n = N * K
    lv = ocb.nf4_levels()
    qw = qk.quantize(w_dev, 64, qk.NF4, double_quant=True)
    _, absmax_dev = qk.qk_quantize_blockwise(w_dev, 64, torch.from_numpy(lv))
    deq = qw.dequantize(torch.bfloat16)
    torch.cuda.synchronize()
    got_codes, got_absmax = host(qw.codes), host(absmax_dev)
    got_q8, got_scale, got_mean, got_deq = host(qw.q8), host(qw.scale), host(qw.mean), host(deq)
    del deq
    if parallel:
        codes, absmax = par.quantize_bf16(w_bits, 64, lv)
    else:
        from oracle import blockwise as obw
        codes, absmax = obw.quantize_blockwise((w_bits.astype(np.uint32) << 16).view(np.float32).reshape(-1), 64, lv)
    assert_bits_equal(got_codes, codes, f"{what} codes")
    assert_bits_equal(got_absmax, absmax, f"{what} absmax")
    q8, scale, mean = odd.double_quant(absmax)
    assert_bits_equal(got_q8, q8, f"{what} q8")
    assert_bits_equal(got_scale, scale, f"{what} dq scale")
    assert_bits_equal(got_mean, np.float32([mean]), f"{what} mean")
    a_eff = odd.reconstruct_absmax(q8, scale, mean)
    if parallel:
        want = par.dequantize_bf16(codes, n, 64, lv, a_eff)
    else:
        want = odq.dequantize_bf16_bits(codes, n, 64, lv, a_eff)
    assert_bits_equal(got_deq, want, f"{what} bf16 dequant")
    say(f"  {what}: {n} elements bit-exact (codes, absmax, q8, scale, mean, bf16 dequant)")


@pytest.mark.parametrize("index", range(7))
def test_llama7b_layer_state_bitexact(index):
    name, N, K = workloads.LLAMA7B_SHAPES[index]
    say(f"case: full-scope llama7b {name} [{N},{K}]")
    W = workloads.llama7b_weight(index)
    _check_whole(dev_bf16(W).reshape(N, K), W, f"llama7b {name}", parallel=False)


@pytest.mark.parametrize("N", [4096, 11008])
def test_qlora_prefill_weight_state_bitexact(N):
    say(f"case: full-scope qlora prefill W [{N},4096]")
    _, W, _, _ = workloads.qlora_prefill(N)
    _check_whole(dev_bf16(W).reshape(N, 4096), W, f"qlora W[{N}]", parallel=False)


@pytest.mark.parametrize("index", range(7))
def test_llama70b_layer_state_bitexact(index):
    name, N, K = workloads.LLAMA70B_LAYER_SHAPES[index]
    say(f"case: full-scope llama70b layer 0 {name} [{N},{K}]")
    w = workloads.device_normal_bf16((N, K), 0.015, workloads.llama70b_seed(0, index))
    _check_whole(w, host(w), f"llama70b {name}", parallel=True)
