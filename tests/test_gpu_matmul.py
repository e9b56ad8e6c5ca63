"""GPU parity of the dequantize-fused GEMV and GEMM (+ LoRA) against the fp64
oracle computed on the oracle's own bf16-dequantized weight.

Tolerance (floating point, accumulation order free): relative Frobenius error
<= 5e-3 and max abs error <= 2e-2 * max |ref|."""

import numpy as np
import pytest
import torch

import bit_blockwise_weight_amd as qk
import workloads
from oracle import blockwise as obw, codebook as ocb, dequant as odq, double_quant as odd, floats as ofl
from oracle import matmul as omm
from tests.gpu_common import bf16_bits_to_f32, dev_bf16, host, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def oracle_wd(w_bits: np.ndarray, N: int, K: int, B: int, kind: int, nested: bool) -> np.ndarray:
    """The oracle's bf16-dequantized weight [N, K] as fp32 values."""
    xf = bf16_bits_to_f32(w_bits).reshape(-1)
    lv = ocb.levels(kind)
    packed, amax = obw.quantize_blockwise(xf, B, lv)
    if nested:
        q, sig, mu = odd.double_quant(amax)
        a_eff = odd.reconstruct_absmax(q, sig, mu)
    else:
        a_eff = amax
    yb = odq.dequantize_bf16_bits(packed, xf.size, B, lv, a_eff)
    return bf16_bits_to_f32(yb).reshape(N, K)


def check_close(got, ref, what):
    rf = omm.rel_frobenius(got, ref)
    mx = omm.max_rel_to_peak(got, ref)
    say(f"  {what}: rel_frob {rf:.2e} max/peak {mx:.2e}")
    assert rf <= omm.REL_FROB_TOL, f"{what}: rel Frobenius {rf}"
    assert mx <= omm.MAX_REL_TOL, f"{what}: max error / peak {mx}"


def _quantized(w_bits, N, K, B=64, kind=ocb.NF4, nested=True):
    return qk.quantize(dev_bf16(w_bits).reshape(N, K), B, kind, double_quant=nested)


def test_gemv_single_1024():
    say("case: gemv single_1024 M=1")
    W, x = workloads.single_1024()
    qw = _quantized(W, 1024, 1024)
    y = host(qw.gemv(dev_bf16(x).reshape(1, 1024)))
    ref = omm.qlora_forward_f64(bf16_bits_to_f32(x).reshape(1, 1024), oracle_wd(W, 1024, 1024, 64, ocb.NF4, True))
    check_close(bf16_bits_to_f32(y), ref, "gemv 1024")


@pytest.mark.parametrize("index", range(7))
def test_gemv_llama7b_layer(index):
    name, N, K = workloads.LLAMA7B_SHAPES[index]
    say(f"case: gemv llama7b {name} [{N},{K}]")
    W = workloads.llama7b_weight(index)
    qw = _quantized(W, N, K)
    wd = oracle_wd(W, N, K, 64, ocb.NF4, True)
    for M in (1, 4, 8, 16):
        x = workloads.activations("llama7b_layer", M, K, tag=index)
        y = host(qw.gemv(dev_bf16(x).reshape(M, K)))
        ref = omm.qlora_forward_f64(bf16_bits_to_f32(x).reshape(M, K), wd)
        check_close(bf16_bits_to_f32(y), ref, f"gemv {name} M={M}")


@pytest.mark.parametrize("B", [64, 128, 256])
@pytest.mark.parametrize("kind", [ocb.NF4, ocb.FP4])
def test_gemv_edge_generic_path(B, kind):
    say(f"case: gemv edge 3000x4099 B={B} kind={kind}")
    W = workloads.edge_weight()
    qw = _quantized(W, 3000, 4099, B, kind, True)
    wd = oracle_wd(W, 3000, 4099, B, kind, True)
    for M in (1, 16):
        x = workloads.activations("edge_3000x4099", M, 4099, tag=M)
        y = host(qw.gemv(dev_bf16(x).reshape(M, 4099)))
        ref = omm.qlora_forward_f64(bf16_bits_to_f32(x).reshape(M, 4099), wd)
        check_close(bf16_bits_to_f32(y), ref, f"gemv edge M={M}")


@pytest.mark.parametrize("N,K,B,M", [(33, 64, 64, 3), (100, 128, 128, 16), (64, 256, 256, 7), (1, 64, 64, 1),
                                     (257, 1024, 64, 9), (31, 192, 64, 16),
                                     # at least two 16-row tiles per CU: the 4-wave kernel (one chunk, partial)
                                     (8200, 320, 64, 5), (8193, 1536, 128, 16)])
def test_gemv_small_and_ragged(N, K, B, M):
    say(f"case: gemv ragged N={N} K={K} B={B} M={M}")
    g = np.random.default_rng(N * 7 + K)
    W = ofl.f32_to_bf16_bits(g.standard_normal((N, K)).astype(np.float32) * np.float32(0.02))
    x = ofl.f32_to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    for nested in (False, True):
        qw = _quantized(W, N, K, B, ocb.NF4, nested)
        y = host(qw.gemv(dev_bf16(x).reshape(M, K)))
        ref = omm.qlora_forward_f64(bf16_bits_to_f32(x).reshape(M, K), oracle_wd(W, N, K, B, ocb.NF4, nested))
        check_close(bf16_bits_to_f32(y), ref, f"gemv nested={nested}")


def test_gemv_llama70b_shapes_sampled_rows():
    """One matrix of each 70B-stack shape (device-drawn), M in {1, 4, 8}; the
    oracle dequantizes 96 sampled rows (its absmax and mean come from the whole
    matrix, copied back as input)."""
    g = np.random.default_rng(70)
    for idx, (name, N, K) in enumerate(workloads.LLAMA70B_LAYER_SHAPES[3:]):
        say(f"case: gemv llama70b {name} [{N},{K}] sampled")
        w = workloads.device_normal_bf16((N, K), 0.015, workloads.llama70b_seed(1, idx))
        qw = qk.quantize(w, 64, qk.NF4, True)
        wb = host(w).reshape(N, K)
        wf = bf16_bits_to_f32(wb).reshape(-1)
        amax = obw.absmax(wf, 64)
        q, sig, mu = odd.double_quant(amax)
        a_eff = odd.reconstruct_absmax(q, sig, mu)
        rows = np.sort(g.choice(N, size=96, replace=False))
        lv = ocb.nf4_levels()
        wd = np.empty((rows.size, K), dtype=np.float32)
        for t, r in enumerate(rows):
            seg = wf[r * K:(r + 1) * K]
            packed, _ = obw.quantize_blockwise(seg, 64, lv)
            yb = odq.dequantize_bf16_bits(packed, K, 64, lv, a_eff[r * K // 64:(r + 1) * K // 64])
            wd[t] = bf16_bits_to_f32(yb)
        for M in (1, 4, 8):
            x = workloads.activations("llama70b_stack", M, K, tag=idx)
            y = host(qw.gemv(dev_bf16(x).reshape(M, K)))
            got = bf16_bits_to_f32(y).reshape(M, N)[:, rows]
            ref = omm.qlora_forward_f64(bf16_bits_to_f32(x).reshape(M, K), wd)
            check_close(got, ref, f"gemv 70b {name} M={M}")
        del w, qw
        torch.cuda.empty_cache()


# ------------------------------------------------------------------------ GEMM

def _lora(K, N, r, seed):
    g = np.random.default_rng(seed)
    A = ofl.f32_to_bf16_bits(g.standard_normal((K, r)).astype(np.float32) * np.float32(0.01))
    B = ofl.f32_to_bf16_bits(g.standard_normal((r, N)).astype(np.float32) * np.float32(0.01))
    return A, B


@pytest.mark.parametrize("M,N,K,B,r", [(128, 128, 64, 64, 16), (77, 100, 128, 128, 1), (300, 257, 256, 256, 64),
                                       (1, 33, 512, 64, 16), (256, 384, 1024, 64, 8), (129, 129, 192, 64, 17),
                                       (200, 300, 320, 64, 40), (65, 96, 448, 64, 45),
                                       # K = 11008: each K split of the X*A pre-pass takes several A chunks
                                       (96, 64, 11008, 64, 16), (70, 48, 11008, 64, 64)])
def test_gemm_small_and_ragged(M, N, K, B, r):
    say(f"case: gemm ragged M={M} N={N} K={K} B={B} r={r}")
    g = np.random.default_rng(M + N + K)
    W = ofl.f32_to_bf16_bits(g.standard_normal((N, K)).astype(np.float32) * np.float32(0.02))
    X = ofl.f32_to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    A, Bm = _lora(K, N, r, M)
    qw = _quantized(W, N, K, B, ocb.NF4, True)
    wd = oracle_wd(W, N, K, B, ocb.NF4, True)
    Xf = bf16_bits_to_f32(X).reshape(M, K)
    Af, Bf = bf16_bits_to_f32(A).reshape(K, r), bf16_bits_to_f32(Bm).reshape(r, N)
    Y = host(qw.gemm(dev_bf16(X).reshape(M, K), dev_bf16(A).reshape(K, r), dev_bf16(Bm).reshape(r, N), 2.0))
    check_close(bf16_bits_to_f32(Y).reshape(M, N), omm.qlora_forward_f64(Xf, wd, Af, Bf, 2.0), "gemm+lora")
    Y0 = host(qw.gemm(dev_bf16(X).reshape(M, K)))
    check_close(bf16_bits_to_f32(Y0).reshape(M, N), omm.qlora_forward_f64(Xf, wd), "gemm base only")


def test_gemm_lora_only_with_zero_weight():
    """All-zero weight without double quantization: the base term is exactly 0,
    so Y is the LoRA term alone."""
    M, N, K, r = 256, 256, 512, 16
    W = np.zeros((N, K), dtype=np.uint16)
    g = np.random.default_rng(3)
    X = ofl.f32_to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    A, Bm = _lora(K, N, r, 4)
    qw = _quantized(W, N, K, 64, ocb.NF4, False)
    Y = host(qw.gemm(dev_bf16(X).reshape(M, K), dev_bf16(A).reshape(K, r), dev_bf16(Bm).reshape(r, N), 2.0))
    ref = omm.qlora_forward_f64(bf16_bits_to_f32(X).reshape(M, K), np.zeros((N, K)),
                                bf16_bits_to_f32(A).reshape(K, r), bf16_bits_to_f32(Bm).reshape(r, N), 2.0)
    check_close(bf16_bits_to_f32(Y).reshape(M, N), ref, "lora only")


@pytest.mark.parametrize("N,K", [(4096, 4096), (11008, 4096), (4096, 11008)])
def test_gemm_qlora_prefill_full_size_sampled_rows(N, K):
    """X [4096, K], W [N, K] NF4 + DQ, LoRA r=16, alpha/r=2 (the layer set's three
    GEMM shapes): 256 sampled output rows against the fp64 oracle."""
    say(f"case: gemm qlora prefill N={N} K={K}")
    X, W, A, Bm = workloads.qlora_prefill(N, K=K)
    M, r = 4096, 16
    qw = _quantized(W, N, K)
    Y = host(qw.gemm(dev_bf16(X).reshape(M, K), dev_bf16(A).reshape(K, r), dev_bf16(Bm).reshape(r, N),
                     workloads.QLORA_ALPHA_OVER_R)).reshape(M, N)
    wd = oracle_wd(W, N, K, 64, ocb.NF4, True)
    rows = np.sort(np.random.default_rng(N).choice(M, size=256, replace=False))
    Xf = bf16_bits_to_f32(X).reshape(M, K)[rows]
    ref = omm.qlora_forward_f64(Xf, wd, bf16_bits_to_f32(A).reshape(K, r), bf16_bits_to_f32(Bm).reshape(r, N),
                                workloads.QLORA_ALPHA_OVER_R)
    check_close(bf16_bits_to_f32(Y[rows]), ref, f"gemm prefill N={N}")


@pytest.mark.parametrize("B", [64, 128, 256])
@pytest.mark.parametrize("kind", [ocb.NF4, ocb.FP4])
def test_gemm_edge_generic_path(B, kind):
    say(f"case: gemm edge 512x3000x4099 B={B} kind={kind}")
    W = workloads.edge_weight()
    X = workloads.edge_activations()
    M, N, K, r = 512, 3000, 4099, 16
    A, Bm = _lora(K, N, r, 5)
    qw = _quantized(W, N, K, B, kind, True)
    Y = host(qw.gemm(dev_bf16(X).reshape(M, K), dev_bf16(A).reshape(K, r), dev_bf16(Bm).reshape(r, N), 2.0))
    wd = oracle_wd(W, N, K, B, kind, True)
    ref = omm.qlora_forward_f64(bf16_bits_to_f32(X).reshape(M, K), wd, bf16_bits_to_f32(A).reshape(K, r),
                                bf16_bits_to_f32(Bm).reshape(r, N), 2.0)
    check_close(bf16_bits_to_f32(Y).reshape(M, N), ref, "gemm edge")


def _at_offset(bits: np.ndarray, off: int, shape) -> torch.Tensor:
    """A device bf16 tensor of `shape` whose data starts `off` elements into a
    larger allocation, so its address is 2-byte but not 4- or 16-byte aligned."""
    flat = dev_bf16(np.concatenate([np.zeros(off, dtype=np.uint16), bits.reshape(-1)]))
    return flat[off:].reshape(shape)


@pytest.mark.parametrize("r", [8, 24, 64, 16, 17, 1])
@pytest.mark.parametrize("xoff,aoff", [(0, 0), (1, 1), (3, 2)])
def test_gemm_generic_lora_ranks_and_offsets(r, xoff, aoff):
    """K = 333 (blocks straddle rows, odd row starts) with X and A at element
    offsets: the generic kernel's realigned X, code and LoRA A loads, including
    ranks that leave padding rows of the A tile (8, 24) and ranks not a multiple
    of 8, which take the element loads."""
    M, N, K, B = 130, 200, 333, 64
    say(f"case: gemm generic M={M} N={N} K={K} r={r} xoff={xoff} aoff={aoff}")
    g = np.random.default_rng(1000 + r)
    W = ofl.f32_to_bf16_bits(g.standard_normal((N, K)).astype(np.float32) * np.float32(0.02))
    X = ofl.f32_to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    A, Bm = _lora(K, N, r, 7 + r)
    qw = _quantized(W, N, K, B, ocb.NF4, True)
    Y = host(qw.gemm(_at_offset(X, xoff, (M, K)), _at_offset(A, aoff, (K, r)), dev_bf16(Bm).reshape(r, N), 2.0))
    wd = oracle_wd(W, N, K, B, ocb.NF4, True)
    ref = omm.qlora_forward_f64(bf16_bits_to_f32(X).reshape(M, K), wd, bf16_bits_to_f32(A).reshape(K, r),
                                bf16_bits_to_f32(Bm).reshape(r, N), 2.0)
    check_close(bf16_bits_to_f32(Y).reshape(M, N), ref, "gemm generic lora")
