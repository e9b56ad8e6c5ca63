"""GPU parity of qk_gemv_nf4_grouped: several weights, each with its own x and y,
in as few launches as their tables allow.  Every y must equal, bit for bit, what
qk_gemv_nf4 of that weight alone writes, and lie within the matmul tolerance of
the fp64 oracle on the oracle's bf16-dequantized weight."""

import numpy as np
import pytest
import torch

import bit_blockwise_weight_amd as qk
import workloads
from oracle import codebook as ocb, floats as ofl, matmul as omm
from tests.gpu_common import assert_bits_equal, bf16_bits_to_f32, dev_bf16, host, require_gpu, say
from tests.test_gpu_matmul import check_close, oracle_wd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _rand_weight(g, N, K):
    return ofl.f32_to_bf16_bits(g.standard_normal((N, K)).astype(np.float32) * np.float32(0.02))


def _check_group(weights, M, g, oracle_every=1):
    """weights: list of (bits [N, K], B, kind, nested)."""
    qws, xs, xbits = [], [], []
    for (W, B, kind, nested) in weights:
        N, K = W.shape
        qws.append(qk.quantize(dev_bf16(W).reshape(N, K), B, kind, double_quant=nested))
        xb = ofl.f32_to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
        xbits.append(xb)
        xs.append(dev_bf16(xb).reshape(M, K))
    ys = qk.qk_gemv_nf4_grouped([(x, qw.state) for x, qw in zip(xs, qws)])
    singles = [qk.qk_gemv_nf4(x, qw.state) for x, qw in zip(xs, qws)]
    torch.cuda.synchronize()
    for i, ((W, B, kind, nested), y, y1) in enumerate(zip(weights, ys, singles)):
        N, K = W.shape
        assert_bits_equal(host(y), host(y1), f"task {i} [{N},{K}] grouped vs alone")
        if i % oracle_every == 0:
            ref = omm.qlora_forward_f64(bf16_bits_to_f32(xbits[i]).reshape(M, K), oracle_wd(W, N, K, B, kind, nested))
            check_close(bf16_bits_to_f32(host(y)).reshape(M, N), ref, f"task {i} [{N},{K}] M={M}")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_grouped_llama7b_layer(M):
    say(f"case: grouped gemv llama7b layer M={M}")
    g = np.random.default_rng(100 + M)
    weights = [(workloads.llama7b_weight(i).reshape(N, K), 64, ocb.NF4, True)
               for i, (_, N, K) in enumerate(workloads.LLAMA7B_SHAPES)]
    _check_group(weights, M, g, oracle_every=3)


@pytest.mark.parametrize("B", [64, 128])
@pytest.mark.parametrize("M", [1, 4])
def test_double_quant_block_boundaries_inside_jobs(M, B):
    """Rows of K = 4160 or 4224 (not a multiple of 512) whose magnitude jumps by 40x every 8
    rows (about two double-quantization blocks of 256 absmax values), so
    neighbouring dq blocks get different scales, each absmax is the mean plus a
    large correction, and the dq-block boundaries fall inside the kernel's 512-k
    jobs at many offsets: a block that took its neighbour's dq scale would be off
    by far more than the tolerance."""
    say(f"case: gemv dq-block boundaries inside jobs M={M} B={B}")
    g = np.random.default_rng(7 + M + B)
    N, K = 96, (4160 if B == 64 else 4224)      # K % 512 != 0, K % B == 0
    mag = np.where((np.arange(N) // 8) % 2 == 0, 0.02, 0.8).astype(np.float32)[:, None]
    W = ofl.f32_to_bf16_bits((g.standard_normal((N, K)).astype(np.float32) * mag).astype(np.float32))
    _check_group([(W, B, ocb.NF4, True)], M, g)


def test_grouped_mixed_tables_blocks_nesting_and_ragged():
    """NF4 / FP4, blocks 64 / 128 / 256, nested or not, ragged rows, K not a multiple
    of 512, and one weight on the generic path (K % 64 != 0): several launches."""
    say("case: grouped gemv mixed")
    g = np.random.default_rng(7)
    shapes = [(33, 64, 64, ocb.NF4, True), (100, 128, 128, ocb.NF4, False), (64, 256, 256, ocb.FP4, True),
              (257, 1024, 64, ocb.NF4, True), (31, 192, 64, ocb.FP4, False), (500, 11008 // 4, 64, ocb.NF4, True),
              (77, 4160, 128, ocb.NF4, True), (129, 100, 64, ocb.NF4, True), (16, 64, 64, ocb.NF4, True)]
    for M in (1, 7):
        _check_group([(_rand_weight(g, N, K), B, kind, nested) for (N, K, B, kind, nested) in shapes], M, g)


def test_grouped_more_than_one_launch_of_tasks():
    """20 weights sharing one table: more than the 16 a launch takes."""
    say("case: grouped gemv 20 weights")
    g = np.random.default_rng(20)
    weights = [(_rand_weight(g, 16 * (i + 1) + (i % 3), 64 * (1 + i % 5)), 64, ocb.NF4, True) for i in range(20)]
    _check_group(weights, 3, g, oracle_every=4)


def test_grouped_tall_weight_cut_into_slices():
    """A weight with more 16-row tiles than the workgroups' LDS holds in one launch
    (64 per workgroup) is cut into row slices; the second slice starts inside the
    scale arrays, away from their first dq block."""
    N, K, M = 64 * 256 * 16 + 48, 64, 4
    say(f"case: grouped gemv tall [{N},{K}] M={M}")
    g = np.random.default_rng(262)
    _check_group([(_rand_weight(g, N, K), 64, ocb.NF4, True)], M, g)


def test_grouped_outputs_written_exactly():
    """Guard bands around each y stay untouched."""
    say("case: grouped gemv guard bands")
    g = np.random.default_rng(5)
    shapes = [(37, 128), (300, 512)]
    qws, xs = [], []
    for N, K in shapes:
        qws.append(qk.quantize(dev_bf16(_rand_weight(g, N, K)).reshape(N, K), 64, qk.NF4, True))
        xs.append(dev_bf16(ofl.f32_to_bf16_bits(g.standard_normal((2, K)).astype(np.float32))).reshape(2, K))
    bufs = [torch.full((2 * N + 64,), 1.5, dtype=torch.bfloat16, device="cuda") for N, _ in shapes]
    ys = [b[32:32 + 2 * N].view(2, N) for b, (N, _) in zip(bufs, shapes)]
    qk.qk_gemv_nf4_grouped([(x, qw.state) for x, qw in zip(xs, qws)], ys)
    torch.cuda.synchronize()
    for b, (N, _) in zip(bufs, shapes):
        hb = host(b)
        assert np.all(hb[:32] == 0x3FC0) and np.all(hb[32 + 2 * N:] == 0x3FC0), "guard band overwritten"
