"""Grouped quantization (qk_quantize_blockwise_grouped) on the GPU: for groups of
tensors of every size class around the kernel's unit (512 elements) and batch
(1024) boundaries, more than 16 tensors (two launches), bf16 / fp16 / fp32
input, NF4 and FP4, blocks of 64, 128 and 256, each tensor's codes and absmax
are bit-for-bit those of qk_quantize_blockwise on that tensor alone and those
of the CPU oracle (blockwise quantization: the xyzblog page, §2.2 【例子】 and
figure 2-2), and nothing is written past any output."""

import numpy as np
import pytest
import torch

import bit_blockwise_weight_amd as qk
import workloads
from oracle import blockwise as obw, codebook as ocb, floats as ofl
from tests.gpu_common import assert_bits_equal, bf16_bits_to_f32, dev_bf16, host, require_gpu, say

pytestmark = pytest.mark.gpu

SIZES = [1, 7, 8, 63, 64, 65, 511, 512, 513, 1023, 1024, 1025, 1536, 2047, 2048, 2049, 4097, 65539, 300001,
         1 << 20]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _inputs(dtype, sizes, seed):
    """Host fp32 values (exact in dtype) and the device tensors; some blocks zero."""
    g = np.random.default_rng(seed)
    vals, devs = [], []
    for n in sizes:
        v = (g.standard_t(3, n) * 0.02).astype(np.float32)
        if n >= 256:
            v[128:192] = 0.0                       # a zero block (absmax 0) at every block size
        if dtype == torch.bfloat16:
            bits = ofl.f32_to_bf16_bits(v)
            vals.append(bf16_bits_to_f32(bits))
            devs.append(dev_bf16(bits))
        elif dtype == torch.float16:
            h = v.astype(np.float16)
            vals.append(h.astype(np.float32))
            devs.append(torch.from_numpy(h).cuda())
        else:
            vals.append(v)
            devs.append(torch.from_numpy(v).cuda())
    return vals, devs


@pytest.mark.parametrize("dtype,kind,B", [(torch.bfloat16, ocb.NF4, 64), (torch.float16, ocb.FP4, 128),
                                          (torch.float32, ocb.NF4, 256)])
def test_grouped_matches_single_calls_and_oracle(dtype, kind, B):
    lv = ocb.nf4_levels() if kind == ocb.NF4 else ocb.fp4_levels()
    vals, devs = _inputs(dtype, SIZES, seed=B)
    say(f"case: grouped quantize of {len(devs)} tensors, {dtype}, kind {kind}, block {B}")
    # outputs with guard bands past their ends
    guard = 64
    codes = [torch.full(((n + 1) // 2 + guard,), 0xA5, dtype=torch.uint8, device="cuda") for n in SIZES]
    absm = [torch.full(((n + B - 1) // B + guard,), -7.0, dtype=torch.float32, device="cuda") for n in SIZES]
    qk.qk_quantize_blockwise_grouped(devs, B, torch.from_numpy(lv),
                                     codes=[c[: (n + 1) // 2] for c, n in zip(codes, SIZES)],
                                     absmaxes=[a[: (n + B - 1) // B] for a, n in zip(absm, SIZES)])
    single = [qk.qk_quantize_blockwise(d, B, torch.from_numpy(lv)) for d in devs]
    torch.cuda.synchronize()
    for n, v, c, a, (sc, sa) in zip(SIZES, vals, codes, absm, single):
        hc, ha = host(c), host(a)
        nc, na = (n + 1) // 2, (n + B - 1) // B
        assert (hc[nc:] == 0xA5).all(), f"n={n}: codes written past the end"
        assert (ha[na:] == np.float32(-7.0)).all(), f"n={n}: absmax written past the end"
        assert_bits_equal(hc[:nc], host(sc), f"n={n} codes vs single call")
        assert_bits_equal(ha[:na], host(sa), f"n={n} absmax vs single call")
        if n <= 300001:
            oc, oa = obw.quantize_blockwise(v, B, lv)
            assert_bits_equal(hc[:nc], oc, f"n={n} codes vs oracle")
            assert_bits_equal(ha[:na], oa, f"n={n} absmax vs oracle")
    say(f"  {len(SIZES)} tensors bit-exact against single calls (and the oracle up to 300001 elements)")


def test_grouped_llama7b_layer():
    """The seven weights of the Llama-7B layer set in one call."""
    lv = ocb.nf4_levels()
    ws = []
    for i, (name, N, K) in enumerate(workloads.LLAMA7B_SHAPES):
        ws.append(dev_bf16(workloads.llama7b_weight(i)).reshape(N, K))
    say("case: grouped quantize of the 7 Llama-7B weights")
    got = qk.qk_quantize_blockwise_grouped(ws, 64, torch.from_numpy(lv))
    single = [qk.qk_quantize_blockwise(w, 64, torch.from_numpy(lv)) for w in ws]
    torch.cuda.synchronize()
    for (name, _, _), (c, a), (sc, sa) in zip(workloads.LLAMA7B_SHAPES, got, single):
        assert_bits_equal(host(c), host(sc), f"{name} codes")
        assert_bits_equal(host(a), host(sa), f"{name} absmax")


def test_grouped_with_a_tensor_launched_alone():
    """A tensor of 2^26 elements or more goes in a launch of its own between the
    launches of the smaller ones; every result still equals its single call."""
    lv = ocb.nf4_levels()
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    big = (torch.randn((1 << 26) + 4099, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    _, smalls = _inputs(torch.bfloat16, [513, 4097, 1 << 20], seed=3)
    xs = [smalls[0], big, smalls[1], smalls[2]]
    say(f"case: grouped quantize with one tensor of {big.numel()} elements among three small ones")
    got = qk.qk_quantize_blockwise_grouped(xs, 64, torch.from_numpy(lv))
    single = [qk.qk_quantize_blockwise(x, 64, torch.from_numpy(lv)) for x in xs]
    torch.cuda.synchronize()
    for i, ((c, a), (sc, sa)) in enumerate(zip(got, single)):
        assert_bits_equal(host(c), host(sc), f"tensor {i} codes")
        assert_bits_equal(host(a), host(sa), f"tensor {i} absmax")


def test_grouped_of_tensors_smaller_than_a_batch():
    """Every tensor under one batch (1024 elements): the launch has no full batch and
    every unit goes through the per-element tail path."""
    lv = ocb.nf4_levels()
    sizes = [1, 2, 33, 511, 512, 513, 1023]
    vals, devs = _inputs(torch.bfloat16, sizes, seed=17)
    say(f"case: grouped quantize of {len(sizes)} tensors under 1024 elements")
    got = qk.qk_quantize_blockwise_grouped(devs, 64, torch.from_numpy(lv))
    torch.cuda.synchronize()
    for n, v, (c, a) in zip(sizes, vals, got):
        oc, oa = obw.quantize_blockwise(v, 64, lv)
        assert_bits_equal(host(c), oc, f"n={n} codes vs oracle")
        assert_bits_equal(host(a), oa, f"n={n} absmax vs oracle")
