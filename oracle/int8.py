"""LLM.int8(): vector-wise int8 matmul with outlier decomposition — oracle, test
infrastructure only.

"篇2-bitsandbytes-具体观-算法与实现剖析", §2.1 LLM.int8(), 【原理】, 【代码】,
【例子】 and figure 2-1: the columns of the activation X (batch, hidden) whose
largest magnitude exceeds `threshold` are outlier features and go through a
16-bit matmul with the matching weight columns; every other column is quantized
vector-wise (one absmax per row, values scaled to [-127, 127], int8) and
multiplied with the int8 weight (one absmax per weight row: CB and SCB); the two
results are added.  A threshold of 0 disables the decomposition.

Readings taken where the page is silent:

* Quantizing a row with absmax a: q = rint_even(RN_fp32(RN_fp32(x / a) * 127)),
  q = 0 when a == 0 (the same steps as the absmax double quantization).
* The weight W [N, K] (out, in) is quantized by rows (CB int8 [N, K], SCB fp32
  [N]); only the int8 weight is kept, so the outlier columns of W are its int8
  values dequantized, Wd[n, k] = CB[n, k] * SCB[n] / 127.
* Outlier columns: O = {k : max_m |X[m, k]| > threshold} (strictly greater, as in
  the example: 7.2 > 6.0); O is empty when threshold <= 0.  The row absmax of X
  is taken over the columns not in O; the columns in O quantize to 0.
* Y = sum_{k not in O} Xq CB * SX[m] SCB[n] / 127^2 + sum_{k in O} X Wd, in fp64
  here; the library writes fp16.
"""

import numpy as np


def quantize_rows(x: np.ndarray, keep=None):
    """Row-wise absmax int8 quantization of a 2-D fp32 array.  `keep` is a bool
    mask over columns (None: all); columns not kept are excluded from the absmax
    and quantize to 0.  Returns (q int8, absmax fp32 per row)."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    keep = np.ones(cols, dtype=bool) if keep is None else np.asarray(keep, dtype=bool)
    xk = np.where(keep[None, :], x, np.float32(0.0))
    a = np.abs(xk).max(axis=1).astype(np.float32) if cols else np.zeros(rows, np.float32)
    safe = np.where(a == 0, np.float32(1.0), a).astype(np.float32)
    with np.errstate(under="ignore"):
        t = (xk / safe[:, None]).astype(np.float32)
        u = (t * np.float32(127.0)).astype(np.float32)
    q = np.rint(u).astype(np.int32)
    q[a == 0, :] = 0
    q[:, ~keep] = 0
    return q.astype(np.int8), a


def outlier_columns(x: np.ndarray, threshold: float) -> np.ndarray:
    """Bool mask of the columns whose max |x| exceeds threshold (none if threshold <= 0)."""
    x = np.asarray(x, dtype=np.float32)
    if threshold <= 0:
        return np.zeros(x.shape[1], dtype=bool)
    return np.abs(x).max(axis=0) > np.float32(threshold)


def decomposed_product_f64(x: np.ndarray, out: np.ndarray, CB: np.ndarray, SCB: np.ndarray):
    """Y for the rows of x given the outlier mask `out` (found over all rows of
    the activation).  Returns (Y, Xq, SX)."""
    x = np.asarray(x, dtype=np.float32)
    out = np.asarray(out, dtype=bool)
    Xq, SX = quantize_rows(x, ~out)
    acc = Xq.astype(np.float64) @ np.asarray(CB, dtype=np.float64).T          # exact: |sum| < 2^53
    Y = acc * SX.astype(np.float64)[:, None] * np.asarray(SCB, dtype=np.float64)[None, :] / (127.0 * 127.0)
    if out.any():
        Wd = np.asarray(CB, dtype=np.float64)[:, out] * np.asarray(SCB, dtype=np.float64)[:, None] / 127.0
        Y = Y + x[:, out].astype(np.float64) @ Wd.T
    return Y, Xq, SX


def int8_matmul_f64(x: np.ndarray, CB: np.ndarray, SCB: np.ndarray, threshold: float):
    """Y [M, N] in fp64 for X [M, K] (fp16 values given as fp32) and the int8
    weight (CB [N, K], SCB [N]).  Returns (Y, outlier mask, Xq, SX)."""
    x = np.asarray(x, dtype=np.float32)
    out = outlier_columns(x, threshold)
    Y, Xq, SX = decomposed_product_f64(x, out, CB, SCB)
    return Y, out, Xq, SX
