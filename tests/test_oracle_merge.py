"""Pins for the oracle's LoRA merge and requantization (CPU only).

The merge follows "LLM 相關知識" (technicalnotes, tag qlora), section 8: the
4-bit weight is dequantized to BF16, the LoRA product is added, the result is a
BF16 W_new, which can be requantized."""

import numpy as np

from oracle import blockwise as bw, codebook, dequant, floats, merge


def _bf16(x):
    return floats.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_zero_adapter_leaves_the_dequantized_weight():
    g = np.random.default_rng(5)
    D = _bf16(g.standard_normal((7, 33)).astype(np.float32) * 0.02)
    A = _bf16(g.standard_normal((33, 4)).astype(np.float32) * 0.01)
    B = np.zeros((4, 7), dtype=np.uint16)                 # LoRA B starts at zero
    assert np.array_equal(merge.lora_merge_bf16_bits(D, A, B, 2.0), D)
    assert np.array_equal(merge.lora_merge_bf16_bits(D, A, _bf16(np.ones((4, 7))), 0.0), D)


def test_exact_integer_case_equals_w_plus_s_ab_transposed():
    # small integers keep every intermediate exact, so W_new = D + s (A B)^T exactly
    g = np.random.default_rng(9)
    N, K, r = 6, 10, 3
    Di = g.integers(-40, 40, size=(N, K))
    Ai = g.integers(-6, 7, size=(K, r))
    Bi = g.integers(-6, 7, size=(r, N))
    s = 0.5
    want = Di + s * (Ai @ Bi).T                            # exact in python floats (halves of small ints)
    assert np.all(np.abs(want) < 128)                      # 8 significant bits: exact in bf16
    got = merge.lora_merge_bf16_bits(_bf16(Di), _bf16(Ai), _bf16(Bi), s)
    assert np.array_equal(floats.bf16_bits_to_f32(got), want.astype(np.float32))


def test_products_are_summed_in_rank_order_in_fp32():
    # ranks 0, 1, 2 contribute 1, 2^-24, 2^-24 to P: in order, 1 + 2^-24 rounds back to 1
    # (a tie, to even) twice; summed the other way round P would be 1 + 2^-23
    t = 2.0 ** -12
    A = _bf16([[1.0, t, t]])                               # K = 1, r = 3
    B = _bf16([[1.0], [t], [t]])                           # N = 1
    P = merge.lora_product_f32(A, B)
    assert P.shape == (1, 1) and P[0, 0] == np.float32(1.0)


def test_final_value_is_rounded_once_to_bf16_nearest_even():
    # D + s P is formed in fp32 and rounded once to bf16: 1 + 2^-8 is the midpoint of
    # bf16 1 and 1 + 2^-7 (ties to even: 1); 1 + 3 2^-9 rounds up to 1 + 2^-7
    D = _bf16([[1.0], [1.0]])                              # N = 2, K = 1
    A = _bf16([[1.0]])                                     # K = 1, r = 1
    for p, want in ((2.0 ** -8, 1.0), (3 * 2.0 ** -9, 1.0 + 2.0 ** -7)):
        B = _bf16([[p, p]])                                # r = 1, N = 2
        got = floats.bf16_bits_to_f32(merge.lora_merge_bf16_bits(D, A, B, 1.0))
        assert np.all(got == np.float32(want)), (p, got)


def test_merged_forward_matches_the_unmerged_one_within_bf16_rounding():
    # the pages warn a merge is not always equivalent; the only difference here is the
    # fp32 sum of the adapter and the final bf16 rounding of W_new
    g = np.random.default_rng(12)
    N, K, r, M = 24, 40, 8, 5
    D = _bf16(g.standard_normal((N, K)).astype(np.float32) * 0.05)
    A = _bf16(g.standard_normal((K, r)).astype(np.float32) * 0.05)
    B = _bf16(g.standard_normal((r, N)).astype(np.float32) * 0.05)
    X = g.standard_normal((M, K))
    s = 2.0
    Wn = floats.bf16_bits_to_f32(merge.lora_merge_bf16_bits(D, A, B, s)).astype(np.float64)
    Df = floats.bf16_bits_to_f32(D).astype(np.float64)
    Af = floats.bf16_bits_to_f32(A).astype(np.float64)
    Bf = floats.bf16_bits_to_f32(B).astype(np.float64)
    unmerged = X @ Df.T + s * (X @ Af) @ Bf
    merged = X @ Wn.T
    exact_w = Df + s * (Af @ Bf).T
    per_elem = np.abs(exact_w) * 2.0 ** -8 + np.abs(s * (Af @ Bf).T) * 2.0 ** -20 + 1e-30
    bound = np.abs(X) @ per_elem.T
    assert np.all(np.abs(merged - unmerged) <= bound)


def test_requantized_merge_error_is_within_half_a_level_gap():
    g = np.random.default_rng(21)
    N, K, r, B = 16, 128, 4, 64
    lv = codebook.nf4_levels()
    D = _bf16(g.standard_normal((N, K)).astype(np.float32) * 0.02)
    A = _bf16(g.standard_normal((K, r)).astype(np.float32) * 0.01)
    Bm = _bf16(g.standard_normal((r, N)).astype(np.float32) * 0.01)
    Wn = merge.lora_merge_bf16_bits(D, A, Bm, 2.0)
    x = floats.bf16_bits_to_f32(Wn).reshape(-1)
    codes, absmax = bw.quantize_blockwise(x, B, lv)
    back = dequant.dequantize_f32(codes, x.size, B, lv, absmax)
    gap = np.max(np.diff(np.sort(np.asarray(lv, dtype=np.float64))))
    a = np.repeat(absmax.astype(np.float64), B)[:x.size]
    # nearest level: |t - l| <= gap / 2, plus the two fp32 roundings (t and l * a)
    assert np.all(np.abs(back.astype(np.float64) - x) <= a * (gap / 2 + 2.0 ** -22))
    d = merge.merge_drift(Wn, back)
    assert 0 < d["rel_frobenius"] < 0.2
