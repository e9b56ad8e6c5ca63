"""LoRA merge and requantization — oracle, test infrastructure only.

"LLM 相關知識" (technicalnotes, tag qlora), section 8 LoRA 的合併 (Merge): the
merged weight is W_new = W + A x B; because an INT4 weight cannot be added to a
BF16 one, the flow is dequantize to BF16, add the LoRA product to get W_new in
BF16, and requantize to 4 bits when needed for deployment; section 9 (the QLoRA
life cycle) repeats dequantize + merge -> BF16 -> requantize.  "Tim Dettmers 如何用
bitsandbytes 與 QLoRA 降低 LLM 訓練門檻？" warns that a merge is not always
equivalent to the unmerged adapter (read the merged weights back and compare).

With W stored [N, K] (out, in), A [K, r], B [r, N] and the LoRA scale s (the
layer computes X W^T + s X A B), the merged weight is W + s (A B)^T.  Reading
used here (the pages give no precision beyond "BF16 + (A x B) = W_new (BF16)"):

    D[n, k] = the BF16 dequantized weight (dequant.dequantize_bf16_bits)
    P[n, k] = sum_{j = 0 .. r-1} B[j, n] * A[k, j], accumulated in fp32 in the
              order j = 0, 1, ..., each product of two bf16 values being exact
    W_new   = RNE_bf16( RN_fp32( D + RN_fp32(s * P) ) )

Requantization is the blockwise quantizer of blockwise.py applied to W_new.
"""

import numpy as np

from .floats import bf16_bits_to_f32, f32_to_bf16_bits


def lora_product_f32(A_bits, B_bits) -> np.ndarray:
    """P[n, k] = sum_j B[j, n] * A[k, j] in fp32, j in increasing order."""
    A = bf16_bits_to_f32(np.asarray(A_bits, dtype=np.uint16))
    B = bf16_bits_to_f32(np.asarray(B_bits, dtype=np.uint16))
    K, r = A.shape
    r2, N = B.shape
    assert r == r2
    P = np.zeros((N, K), dtype=np.float32)
    with np.errstate(under="ignore"):
        for j in range(r):
            prod = np.multiply.outer(B[j], A[:, j]).astype(np.float32)   # exact: 8-bit x 8-bit significands
            P = (P + prod).astype(np.float32)
    return P


def lora_merge_bf16_bits(D_bits, A_bits, B_bits, scale: float) -> np.ndarray:
    """W_new as bf16 bits [N, K] from the bf16 dequantized weight D [N, K]."""
    D = bf16_bits_to_f32(np.asarray(D_bits, dtype=np.uint16))
    P = lora_product_f32(A_bits, B_bits)
    with np.errstate(under="ignore"):
        T = (np.float32(scale) * P).astype(np.float32)
        W = (D + T).astype(np.float32)
    return f32_to_bf16_bits(W)


def merge_drift(W_new_bits, W_requant_f32) -> dict:
    """How far the requantized merged weight is from the merged BF16 weight."""
    w = bf16_bits_to_f32(np.asarray(W_new_bits, dtype=np.uint16)).astype(np.float64).reshape(-1)
    q = np.asarray(W_requant_f32, dtype=np.float64).reshape(-1)
    d = q - w
    return {"max_abs": float(np.max(np.abs(d))) if d.size else 0.0,
            "rel_frobenius": float(np.linalg.norm(d) / max(np.linalg.norm(w), 1e-300))}
