"""Double quantization of the absmax array (step a5) — oracle, test infrastructure only.

"篇2-bitsandbytes-具体观-算法与实现剖析", §2.2 QLoRA / NF4, 【原理】 ② and
figure 2-2: the per-block absmax values are themselves quantized to 8 bits
(the nested "state2"), cutting the per-parameter overhead from 4 + 0.5 bit to
4 + 0.13 bit.  §2.2 【代码】 lists the quant_state fields absmax / code /
state2 / offset / nested_absmax; the "offset" field is read as a mean that is
subtracted before the second quantization.  "Tim Dettmers 如何用 bitsandbytes
與 QLoRA 降低 LLM 訓練門檻？", section "Double quantization 連 scale 本身也壓縮",
states the same idea.

Readings taken where the pages are silent (each is listed in the design notes):

* mean:   mu = RN_fp32( T(a) / nb ), T = the fp64 sum of a in a perfect binary
          tree (a zero-padded to the next power of two, neighbours added level
          by level), the division in fp64, then one rounding to fp32.
* centre: c_j = RN_fp32(a_j - mu).
* 8-bit map: linear symmetric absmax int8 over blocks of 256 absmax values
          (the last block may be partial):
          s_d = max_j |c_j|,  sigma_d = RN_fp32(s_d / 127) (stored),
          q_j = 0 if s_d == 0 else rint_half_even( RN_fp32( RN_fp32(c_j / s_d) * 127 ) ).
"""

import numpy as np

DQ_BLOCK = 256
DQ_LEVELS = np.float32(127.0)


def tree_sum_f64(v: np.ndarray) -> np.float64:
    """Sum in fp64 along a perfect binary tree over v zero-padded to 2^ceil(log2 len)."""
    v = np.asarray(v, dtype=np.float64).reshape(-1)
    if v.size == 0:
        return np.float64(0.0)
    p = 1
    while p < v.size:
        p *= 2
    level = np.zeros(p, dtype=np.float64)
    level[: v.size] = v
    while level.size > 1:
        level = level[0::2] + level[1::2]
    return level[0]


def mean_f32(absmax: np.ndarray) -> np.float32:
    a = np.asarray(absmax, dtype=np.float32).reshape(-1)
    total = tree_sum_f64(a)
    return np.float32(total / np.float64(a.size))


def double_quant(absmax: np.ndarray, dq_block: int = DQ_BLOCK):
    """Returns (q int8[nb], sigma fp32[ceil(nb/dq_block)], mu fp32)."""
    a = np.asarray(absmax, dtype=np.float32).reshape(-1)
    nb = a.size
    mu = mean_f32(a)
    c = (a - mu).astype(np.float32)
    nd = (nb + dq_block - 1) // dq_block
    q = np.zeros(nb, dtype=np.int8)
    sigma = np.zeros(nd, dtype=np.float32)
    for d in range(nd):
        cd = c[d * dq_block:(d + 1) * dq_block]
        s = np.abs(cd).max()
        sigma[d] = np.float32(s / DQ_LEVELS)
        if s == np.float32(0.0):
            continue
        with np.errstate(under="ignore"):
            ratio = (cd / s).astype(np.float32)
            scaled = (ratio * DQ_LEVELS).astype(np.float32)
        q[d * dq_block:(d + 1) * dq_block] = np.rint(scaled).astype(np.int8)
    return q, sigma, mu


def reconstruct_absmax(q: np.ndarray, sigma: np.ndarray, mu, dq_block: int = DQ_BLOCK) -> np.ndarray:
    """a'_j = RN_fp32( RN_fp32(q_j * sigma_d) + mu ): two separate roundings, no fused multiply-add."""
    q = np.asarray(q, dtype=np.int8).reshape(-1)
    sig = np.repeat(np.asarray(sigma, dtype=np.float32), dq_block)[: q.size]
    prod = (q.astype(np.float32) * sig).astype(np.float32)
    return (prod + np.float32(mu)).astype(np.float32)
