"""Grouped double quantization (qk_double_quant_grouped) on the GPU: for groups
of absmax arrays of every size class, including more than one run of 16 arrays
and an array too large for the grouped launch, each array's q8, scale and mean
are bit-for-bit those of qk_double_quant on that array alone, and those of the
CPU oracle (double quantization: the xyzblog page, §2.2 【原理】②)."""

import numpy as np
import pytest
import torch

import bit_blockwise_weight_amd as qk
import workloads
from oracle import codebook as ocb, double_quant as odd
from tests.gpu_common import assert_bits_equal, dev_bf16, host, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _arrays():
    g = np.random.default_rng(31)
    ties = np.float32(200.0) + np.float32([127.0, -127.0, 0.5, -0.5, 2.5, -2.5, 1.5, -1.5])
    out = [
        ("ties", ties),
        ("wide-sum mean", np.float32([1.0, 2.0 ** -24, 0.0, 0.0, 0.0])),
        ("one value", np.float32([3.5])),
        ("all zero", np.zeros(300, np.float32)),
        ("ties x 700", np.tile(ties, 700)),
        ("ties x 1200", np.tile(ties, 1200)),
    ]
    for nb in (1, 255, 256, 257, 4095, 4096, 4097, 65539, 1_000_003):
        out.append((f"random nb={nb}", (np.abs(g.standard_normal(nb)) * 0.05).astype(np.float32)))
    for k in range(6):
        out.append((f"random chunk-sized {k}", (np.abs(g.standard_normal(4096 * (k + 1) + 17 * k)) * 0.03)
                    .astype(np.float32)))
    return out


def test_grouped_matches_single_calls_and_oracle():
    arrays = _arrays()
    assert len(arrays) > 16                      # two runs of the grouped launch
    devs = [_dev_f32(a) for _, a in arrays]
    say(f"case: grouped double quant of {len(arrays)} arrays, nb from 1 to 1000003")
    got = qk.qk_double_quant_grouped(devs)
    single = [qk.qk_double_quant(d) for d in devs]
    torch.cuda.synchronize()
    for (name, a), (q8, sc, mu), (sq8, ssc, smu) in zip(arrays, got, single):
        assert_bits_equal(host(q8), host(sq8), f"{name} q8 vs single call")
        assert_bits_equal(host(sc), host(ssc), f"{name} scale vs single call")
        assert_bits_equal(host(mu), host(smu), f"{name} mean vs single call")
        oq, osig, omu = odd.double_quant(a)
        assert_bits_equal(host(q8), oq, f"{name} q8")
        assert_bits_equal(host(sc), osig, f"{name} scale")
        assert_bits_equal(host(mu), np.float32([omu]), f"{name} mean")
    say(f"  {len(arrays)} arrays bit-exact against single calls and the oracle")


def test_grouped_repeat_is_deterministic_and_outputs_are_exact():
    """Two calls on fresh outputs filled with different garbage write the same bits,
    and nothing past each array's q8 / scale is written."""
    arrays = _arrays()[:10]
    devs = [_dev_f32(a) for _, a in arrays]
    res = []
    for fill in (0x55, -0x56):
        q8s = [torch.full((a.size + 64,), fill, dtype=torch.int8, device="cuda") for _, a in arrays]
        scs = [torch.full(((a.size + 255) // 256 + 16,), float(fill), dtype=torch.float32, device="cuda")
               for _, a in arrays]
        mus = [torch.full((2,), float(fill), dtype=torch.float32, device="cuda") for _ in arrays]
        qk.qk_double_quant_grouped(devs, q8s=[q[: a.size] for q, (_, a) in zip(q8s, arrays)],
                                   scales=[s[: (a.size + 255) // 256] for s, (_, a) in zip(scs, arrays)],
                                   means=[m[:1] for m in mus])
        torch.cuda.synchronize()
        for (name, a), q, s, m in zip(arrays, q8s, scs, mus):
            nd = (a.size + 255) // 256
            assert (host(q)[a.size:] == fill).all(), f"{name}: q8 written past the end"
            assert (host(s)[nd:] == np.float32(fill)).all(), f"{name}: scale written past the end"
            assert host(m)[1] == np.float32(fill), f"{name}: mean written past the end"
        res.append([(host(q)[: a.size], host(s)[: (a.size + 255) // 256], host(m)[:1])
                    for q, s, m, (_, a) in zip(q8s, scs, mus, arrays)])
    for (name, _), r0, r1 in zip(arrays, res[0], res[1]):
        for x0, x1 in zip(r0, r1):
            assert_bits_equal(x0, x1, f"{name}: repeat")


def test_grouped_with_an_array_past_the_grouped_limit():
    """An array of more than 4096 * 4096 absmax values takes the per-array path
    inside the grouped call; the others still share the grouped launches."""
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    big = (torch.randn(4096 * 4096 + 1001, device="cuda", generator=g).abs() * 0.02).contiguous()
    small = [_dev_f32(a) for _, a in _arrays()[:4]]
    say(f"case: grouped double quant with one array of {big.numel()} absmax")
    got = qk.qk_double_quant_grouped([small[0], big] + small[1:])
    single = [qk.qk_double_quant(d) for d in [small[0], big] + small[1:]]
    torch.cuda.synchronize()
    for i, ((q8, sc, mu), (sq8, ssc, smu)) in enumerate(zip(got, single)):
        assert_bits_equal(host(q8), host(sq8), f"array {i} q8")
        assert_bits_equal(host(sc), host(ssc), f"array {i} scale")
        assert_bits_equal(host(mu), host(smu), f"array {i} mean")
    # the big array against the oracle's mean (the tree over 16.8 M values)
    assert_bits_equal(host(got[1][2]), np.float32([odd.mean_f32(host(big))]), "big array mean")


def test_grouped_llama7b_layer_absmax():
    """The seven absmax arrays the quantize kernel writes for the Llama-7B layer set."""
    lv = ocb.nf4_levels()
    absmaxes = []
    for i, (name, N, K) in enumerate(workloads.LLAMA7B_SHAPES):
        W = workloads.llama7b_weight(i)
        _, am = qk.qk_quantize_blockwise(dev_bf16(W).reshape(N, K), 64, torch.from_numpy(lv))
        absmaxes.append(am)
    say("case: grouped double quant of the 7 Llama-7B absmax arrays")
    got = qk.qk_double_quant_grouped(absmaxes)
    single = [qk.qk_double_quant(a) for a in absmaxes]
    torch.cuda.synchronize()
    for (name, _, _), (q8, sc, mu), (sq8, ssc, smu), am in zip(workloads.LLAMA7B_SHAPES, got, single, absmaxes):
        assert_bits_equal(host(q8), host(sq8), f"{name} q8")
        assert_bits_equal(host(sc), host(ssc), f"{name} scale")
        assert_bits_equal(host(mu), host(smu), f"{name} mean")
        oq, osig, omu = odd.double_quant(host(am))
        assert_bits_equal(host(q8), oq, f"{name} q8 vs oracle")
        assert_bits_equal(host(mu), np.float32([omu]), f"{name} mean vs oracle")
