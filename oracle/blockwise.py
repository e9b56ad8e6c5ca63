"""Blockwise quantization (steps a2-a4) — oracle, test infrastructure only.

Follows "篇2-bitsandbytes-具体观-算法与实现剖析", §2.2 QLoRA / NF4, 【例子】
and figure 2-2: cut the weight into blocks of `blocksize` (64 by default),
take each block's absmax, divide the block by it so it lies in [-1, 1], map
every normalised value to one of the 16 levels, and pack two 4-bit codes per
byte.  "Tim Dettmers 如何用 bitsandbytes 與 QLoRA 降低 LLM 訓練門檻？",
section "8-bit optimizer 先處理訓練狀態的隱形成本", motivates the per-block
scale (each block is scaled on its own so one extreme value cannot spoil the
range of the whole tensor).

Readings taken where the pages are silent:

* Blocking is over the row-major *flattened* tensor: block j covers elements
  [j*B, min((j+1)*B, n)); the last block may be partial, and blocks may
  straddle rows when the row length is not a multiple of B.
* absmax is kept in fp32 (the page's "+0.5 bit per parameter" at block 64 only
  fits a 32-bit scale).
* t = RN_fp32(x / a) with IEEE division; a block with a == 0 has t = +0.
* code = the index of the nearest level, exactly; on a tie between two levels
  the smaller index wins.  For a table in code order that is not sorted (FP4),
  "smaller index" is the smaller code, not the smaller value.
* Packing: element 2t goes to the high nibble of byte t, element 2t+1 to the
  low nibble; when n is odd the last low nibble is 0.
"""

from fractions import Fraction

import numpy as np


def num_blocks(n: int, blocksize: int) -> int:
    return (n + blocksize - 1) // blocksize


def absmax(x: np.ndarray, blocksize: int) -> np.ndarray:
    """fp32 max |x| per block of the flattened input (exact: max is exact)."""
    x = np.asarray(x, dtype=np.float32).reshape(-1)
    n = x.size
    nb = num_blocks(n, blocksize)
    out = np.zeros(nb, dtype=np.float32)
    full = n // blocksize
    if full:
        out[:full] = np.abs(x[: full * blocksize].reshape(full, blocksize)).max(axis=1)
    if nb > full:
        out[full] = np.abs(x[full * blocksize:]).max()
    return out


def normalize(x: np.ndarray, amax: np.ndarray, blocksize: int) -> np.ndarray:
    """t_k = RN_fp32(x_k / a_j) (numpy float32 division is IEEE, correctly rounded,
    subnormals kept); t = +0 in a block whose absmax is 0."""
    x = np.asarray(x, dtype=np.float32).reshape(-1)
    a = np.repeat(np.asarray(amax, dtype=np.float32), blocksize)[: x.size]
    zero = a == np.float32(0.0)
    safe = np.where(zero, np.float32(1.0), a).astype(np.float32)
    with np.errstate(under="ignore"):
        t = (x / safe).astype(np.float32)
    t[zero] = np.float32(0.0)
    return t


def _sorted_unique_levels(levels: np.ndarray):
    """Distinct level values in increasing order, and for each the smallest
    code that carries it (+0 and -0 are the same value)."""
    lv = [float(v) for v in np.asarray(levels, dtype=np.float32)]
    values = sorted(set(lv))
    min_code = [min(i for i, v in enumerate(lv) if v == u) for u in values]
    return np.array(values, dtype=np.float64), np.array(min_code, dtype=np.int64)


def nearest_code(t: np.ndarray, levels: np.ndarray) -> np.ndarray:
    """code = smallest i with |t - l_i| = min_j |t - l_j|, computed exactly.

    Between two neighbouring distinct values u_s < u_{s+1} the nearer one is
    decided by comparing t with their midpoint m_s = (u_s + u_{s+1}) / 2.  For
    binary32 levels the midpoint is exact in binary64 (checked below), and
    comparing a binary32 t with it is exact.  A t equal to a midpoint is a tie:
    the smaller code of the two wins."""
    t = np.asarray(t, dtype=np.float32).reshape(-1).astype(np.float64)
    u, min_code = _sorted_unique_levels(levels)
    mids = (u[:-1] + u[1:]) / 2.0
    for i, m in enumerate(mids):
        assert Fraction(float(m)) == (Fraction(float(u[i])) + Fraction(float(u[i + 1]))) / 2, \
            "level midpoint is not exact in binary64"
    s = np.searchsorted(mids, t, side="left")          # = #{i : t > m_i}
    code = min_code[s]
    tie_idx = np.minimum(s, len(mids) - 1)
    tie = (s < len(mids)) & (mids[tie_idx] == t)
    if np.any(tie):
        other = min_code[np.minimum(s + 1, len(u) - 1)]
        code = np.where(tie, np.minimum(code, other), code)
    return code.astype(np.uint8)


def nearest_code_bruteforce(t_values, levels) -> list:
    """The definition itself, in exact rational arithmetic (tiny inputs only)."""
    lv = [Fraction(float(v)) for v in np.asarray(levels, dtype=np.float32)]
    out = []
    for tv in np.asarray(t_values, dtype=np.float32).reshape(-1):
        tf = Fraction(float(tv))
        d = [abs(tf - l) for l in lv]
        best = min(d)
        out.append(d.index(best))  # first (smallest) index among the minima
    return out


def pack(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    if c.size % 2:
        c = np.concatenate([c, np.zeros(1, dtype=np.uint8)])
    return ((c[0::2] << 4) | c[1::2]).astype(np.uint8)


def unpack(packed: np.ndarray, n: int) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    c = np.empty(p.size * 2, dtype=np.uint8)
    c[0::2] = p >> 4
    c[1::2] = p & 0x0F
    return c[:n]


def quantize_blockwise(x: np.ndarray, blocksize: int, levels: np.ndarray):
    """Returns (packed codes uint8[ceil(n/2)], absmax fp32[ceil(n/B)])."""
    x = np.asarray(x, dtype=np.float32).reshape(-1)
    a = absmax(x, blocksize)
    t = normalize(x, a, blocksize)
    codes = nearest_code(t, levels)
    return pack(codes), a
