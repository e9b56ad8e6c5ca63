"""qk_gemm_nf4_noalloc (the GEMM whose LoRA partials live in the library's
static device scratch) against qk_gemm_nf4 with a caller workspace: the same
kernels, so the outputs must be equal bit for bit.  Two calls in a row with the
second smaller (the scratch keeps the first call's contents), the largest
adapter the scratch takes, and a base-only call."""

import numpy as np
import pytest
import torch

import bit_blockwise_weight_amd as qk
from oracle import matmul as omm
from tests.gpu_common import assert_bits_equal, bf16_bits_to_f32, host, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _case(seed, M, N, K, r):
    g = torch.Generator(device="cuda").manual_seed(seed)
    W = (torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    X = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
    A = (torch.randn((K, r), generator=g, device="cuda") * 0.01).to(torch.bfloat16) if r else None
    B = (torch.randn((r, N), generator=g, device="cuda") * 0.01).to(torch.bfloat16) if r else None
    return qk.quantize(W, 64, qk.NF4, double_quant=True), X, A, B


def _both(qw, X, A, B):
    Yn = qk.qk_gemm_nf4_noalloc(X, qw.state, A, B, 2.0)
    Yw = qk.qk_gemm_nf4(X, qw.state, A, B, 2.0)
    torch.cuda.synchronize()
    return host(Yn), host(Yw)


def test_noalloc_matches_workspace_call_twice_second_smaller():
    for seed, (M, N, K, r) in ((1, (1024, 512, 1024, 32)), (2, (300, 256, 512, 16))):
        say(f"case: gemm noalloc M={M} N={N} K={K} r={r}")
        qw, X, A, B = _case(seed, M, N, K, r)
        yn, yw = _both(qw, X, A, B)
        assert_bits_equal(yn, yw, f"noalloc vs workspace M={M} r={r}")
        # and within the matmul tolerance of the fp64 oracle on the dequantized weight
        wd = bf16_bits_to_f32(host(qw.dequantize(torch.bfloat16))).reshape(N, K)
        ref = omm.qlora_forward_f64(bf16_bits_to_f32(host(X)).reshape(M, K), wd,
                                    bf16_bits_to_f32(host(A)).reshape(K, r), bf16_bits_to_f32(host(B)).reshape(r, N), 2.0)
        got = bf16_bits_to_f32(yn).reshape(M, N)
        assert omm.rel_frobenius(got, ref) <= omm.REL_FROB_TOL
        assert omm.max_rel_to_peak(got, ref) <= omm.MAX_REL_TOL


def test_noalloc_largest_adapter_and_base_only():
    say("case: gemm noalloc at the scratch limit M=16384 r=16, then base only")
    qw, X, A, B = _case(3, 16384, 256, 256, 16)
    yn, yw = _both(qw, X, A, B)
    assert_bits_equal(yn, yw, "noalloc at the limit")
    qw, X, _, _ = _case(4, 77, 320, 640, 0)
    yn, yw = _both(qw, X, None, None)
    assert_bits_equal(yn, yw, "noalloc base only")
    # one row past the limit is refused, and launches nothing
    qw, X, A, B = _case(5, 16385, 256, 256, 16)
    with pytest.raises(qk.QKError) as ei:
        qk.qk_gemm_nf4_noalloc(X, qw.state, A, B, 2.0)
    assert ei.value.status == qk.QK_ERR_WORKSPACE
