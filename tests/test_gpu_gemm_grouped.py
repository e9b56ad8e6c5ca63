"""GPU parity of qk_gemm_nf4_grouped: several prefill GEMMs (each with its own X,
adapter and Y) in as few launches as their shapes allow.  Every Y must equal, bit
for bit, what qk_gemm_nf4 of that task alone writes (the same kernels compute
every tile the same way), and a few lie within the matmul tolerance of the fp64
oracle on the oracle's bf16-dequantized weight."""

import numpy as np
import pytest
import torch

import bit_blockwise_weight_amd as qk
import workloads
from oracle import codebook as ocb, floats as ofl, matmul as omm
from tests.gpu_common import assert_bits_equal, bf16_bits_to_f32, dev_bf16, host, require_gpu, say
from tests.test_gpu_matmul import _lora, check_close, oracle_wd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _task(g, M, N, K, B=64, kind=ocb.NF4, nested=True, r=16):
    W = ofl.f32_to_bf16_bits(g.standard_normal((N, K)).astype(np.float32) * np.float32(0.02))
    X = ofl.f32_to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    qw = qk.quantize(dev_bf16(W).reshape(N, K), B, kind, double_quant=nested)
    if r:
        A, Bm = _lora(K, N, r, M + N + K + r)
        Ad, Bd = dev_bf16(A).reshape(K, r), dev_bf16(Bm).reshape(r, N)
    else:
        A = Bm = Ad = Bd = None
    return dict(W=W, X=X, A=A, Bm=Bm, qw=qw, Xd=dev_bf16(X).reshape(M, K), Ad=Ad, Bd=Bd, M=M, N=N, K=K, B=B,
                kind=kind, nested=nested, r=r)


def _check(tasks, oracle_idx=()):
    ys = qk.qk_gemm_nf4_grouped([(t["Xd"], t["qw"].state, t["Ad"], t["Bd"], t.get("s", 2.0)) for t in tasks])
    singles = [t["qw"].gemm(t["Xd"], t["Ad"], t["Bd"], t.get("s", 2.0)) for t in tasks]
    torch.cuda.synchronize()
    for i, (t, y, y1) in enumerate(zip(tasks, ys, singles)):
        assert_bits_equal(host(y), host(y1), f"task {i} [{t['M']}x{t['N']}x{t['K']}] r={t['r']} grouped vs alone")
    for i in oracle_idx:
        t = tasks[i]
        M, N, K, r = t["M"], t["N"], t["K"], t["r"]
        wd = oracle_wd(t["W"], N, K, t["B"], t["kind"], t["nested"])
        Xf = bf16_bits_to_f32(t["X"]).reshape(M, K)
        if r:
            ref = omm.qlora_forward_f64(Xf, wd, bf16_bits_to_f32(t["A"]).reshape(K, r),
                                        bf16_bits_to_f32(t["Bm"]).reshape(r, N), t.get("s", 2.0))
        else:
            ref = omm.qlora_forward_f64(Xf, wd)
        check_close(bf16_bits_to_f32(host(ys[i])).reshape(M, N), ref, f"task {i} vs oracle")


def test_grouped_llama7b_layer_shapes():
    """The Llama-7B layer's seven weights at M = 512 with LoRA r = 16: one launch."""
    say("case: grouped gemm llama7b layer M=512 r=16")
    g = np.random.default_rng(9)
    tasks = [_task(g, 512, N, K) for _, N, K in workloads.LLAMA7B_SHAPES]
    _check(tasks)


def test_grouped_mixed_ranks_shapes_and_paths():
    """Ragged M and N, ranks 0 / 16 / 17 / 40 / 64 (four rank classes), nested and
    plain states, block 128, and one weight the 256 x 256 kernel cannot take
    (K = 4099): several launches, one of them alone on the generic kernel."""
    say("case: grouped gemm mixed")
    g = np.random.default_rng(10)
    tasks = [_task(g, 300, 257, 512, r=16), _task(g, 77, 100, 256, r=0), _task(g, 512, 384, 1024, r=17),
             _task(g, 129, 129, 192, r=40, nested=False), _task(g, 256, 300, 320, r=64, B=64, kind=ocb.FP4),
             _task(g, 200, 96, 4099, r=16), _task(g, 64, 512, 768, B=128, r=16), _task(g, 1, 33, 512, r=16),
             _task(g, 96, 64, 11008, r=16)]
    _check(tasks, oracle_idx=(0, 3, 5, 7))


def test_grouped_shared_input_and_scales():
    """Seven GEMMs reading one X, with adapters of 16, 16, 32, 16, 48, 16 and 24 ranks
    and scales of their own, and one more on another X: every Y must equal its
    single call bit for bit."""
    say("case: grouped gemm shared X, own scales")
    g = np.random.default_rng(13)
    M, K = 512, 1024
    X = ofl.f32_to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    Xd = dev_bf16(X).reshape(M, K)
    tasks = []
    for j, (N, r, sc) in enumerate([(256, 16, 2.0), (384, 16, 0.5), (300, 32, 1.0), (256, 16, 3.0), (512, 48, 0.25),
                                    (128, 16, 2.0), (256, 24, 1.5)]):
        t = _task(g, M, N, K, r=r)
        t.update(X=X, Xd=Xd, s=sc)
        tasks.append(t)
    tasks.append(_task(g, M, 256, 2048, r=16))
    _check(tasks, oracle_idx=(2, 4, 6))


def test_grouped_more_than_one_launch_of_tasks():
    """Ten weights of one rank class and nesting: more than the 8 a launch takes."""
    say("case: grouped gemm 10 tasks")
    g = np.random.default_rng(11)
    tasks = [_task(g, 64 * (1 + i % 3), 128 + 64 * (i % 4), 256 * (1 + i % 2)) for i in range(10)]
    _check(tasks, oracle_idx=(9,))


def test_grouped_outputs_written_exactly():
    """Guard bands around each Y stay untouched."""
    say("case: grouped gemm guard bands")
    g = np.random.default_rng(12)
    tasks = [_task(g, 100, 70, 256), _task(g, 33, 300, 512)]
    bufs = [torch.full((t["M"] * t["N"] + 128,), 1.5, dtype=torch.bfloat16, device="cuda") for t in tasks]
    ys = [b[64:64 + t["M"] * t["N"]].view(t["M"], t["N"]) for b, t in zip(bufs, tasks)]
    qk.qk_gemm_nf4_grouped([(t["Xd"], t["qw"].state, t["Ad"], t["Bd"], 2.0) for t in tasks], ys)
    torch.cuda.synchronize()
    for b, t in zip(bufs, tasks):
        hb = host(b)
        n = t["M"] * t["N"]
        assert np.all(hb[:64] == 0x3FC0) and np.all(hb[64 + n:] == 0x3FC0), "guard band overwritten"
