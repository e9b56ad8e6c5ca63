"""Dequantized matmul with the LoRA term (steps a7, a8) — oracle, test infrastructure only.

"LLM 相關知識" (technicalnotes, tag qlora), section 2-2 LoRA: the frozen base
weight W gets a trainable low-rank update ΔW = A × B, the layer acts as
W + ΔW; section 8 (Merge) says that without merging every layer computes the
base output and the LoRA output separately and adds them.  "篇2-bitsandbytes-
具体观-算法与实现剖析", §2.2 【代码】: the 4-bit linear layer's forward is a
dequantize followed by a matmul.

With W stored as [N, K] (out, in) and X as [M, K]:

    Y = X · W_d^T + s · (X · A) · B,    A: [K, r], B: [r, N], s = alpha / r

computed in fp64 from the exact values of the bf16 inputs and of the
dequantized weight W_d (the bf16 output of the dequantization step).  The
order of accumulation is free, so any result within the stated tolerance is
correct; this function gives the reference value.
"""

from fractions import Fraction

import numpy as np


def qlora_forward_f64(X, Wd, A=None, B=None, scale: float = 0.0) -> np.ndarray:
    X = np.asarray(X, dtype=np.float64)
    Wd = np.asarray(Wd, dtype=np.float64)
    Y = X @ Wd.T
    if A is not None and B is not None:
        Y = Y + np.float64(scale) * ((X @ np.asarray(A, dtype=np.float64)) @ np.asarray(B, dtype=np.float64))
    return Y


def qlora_forward_exact(X, Wd, A=None, B=None, scale=0) -> list:
    """Exact rational triple loop over the definition (tiny shapes only)."""
    X = np.asarray(X, dtype=np.float64)
    Wd = np.asarray(Wd, dtype=np.float64)
    M, K = X.shape
    N = Wd.shape[0]
    s = Fraction(scale)
    out = []
    for m in range(M):
        row = []
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += Fraction(float(X[m, k])) * Fraction(float(Wd[n, k]))
            if A is not None and B is not None:
                A_ = np.asarray(A, dtype=np.float64)
                B_ = np.asarray(B, dtype=np.float64)
                r = A_.shape[1]
                lora = Fraction(0)
                for j in range(r):
                    xa = Fraction(0)
                    for k in range(K):
                        xa += Fraction(float(X[m, k])) * Fraction(float(A_[k, j]))
                    lora += xa * Fraction(float(B_[j, n]))
                acc += s * lora
            row.append(acc)
        out.append(row)
    return out


def rel_frobenius(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got - ref))


def max_rel_to_peak(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    peak = np.abs(ref).max()
    err = np.abs(got - ref).max()
    return float(err / peak) if peak > 0 else float(err)


# Tolerances for floating-point matmul outputs against the fp64 reference.
REL_FROB_TOL = 5e-3
MAX_REL_TOL = 2e-2
