"""QLoRA backward of the frozen 4-bit base layer — oracle, test infrastructure only.

"Tim Dettmers 如何用 bitsandbytes 與 QLoRA 降低 LLM 訓練門檻？", section "QLoRA 把
frozen 4-bit base 與可訓練 adapter 分開": the base stays frozen in 4 bits and is
dequantized to the compute dtype in the forward and in the backward pass; only
the low-rank adapter is trained.  The gradients below are the plain chain rule
of the forward layer (matmul.py); the pages print no formula for them.

For the layer Y = X Wd^T + s (X A) B (Wd [N, K] the bf16 dequantized weight,
A [K, r], B [r, N]) and an upstream gradient dY [M, N], in fp64:

    G  = dY B^T
    dX = dY Wd + s G A^T
    dA = s X^T G
    dB = s (X A)^T dY
"""

import numpy as np


def qlora_backward_f64(dY, X, Wd, A=None, B=None, scale: float = 0.0):
    dY = np.asarray(dY, dtype=np.float64)
    Wd = np.asarray(Wd, dtype=np.float64)
    dX = dY @ Wd
    if A is None:
        return dX, None, None
    X = np.asarray(X, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    G = dY @ B.T
    dX = dX + scale * (G @ A.T)
    dA = scale * (X.T @ G)
    dB = scale * ((X @ A).T @ dY)
    return dX, dA, dB
