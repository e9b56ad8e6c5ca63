"""Dequantization (step a6) — oracle, test infrastructure only.

"LLM 相關知識" (technicalnotes, tag qlora), section 5 動態反量化 (Dynamic
Dequantization): in the forward pass the 4-bit base weight of a layer is
restored to BF16 just before its matmul and discarded right after.  "Tim
Dettmers 如何用 bitsandbytes 與 QLoRA 降低 LLM 訓練門檻？", section "QLoRA 把
frozen 4-bit base 與可訓練 adapter 分開", says the same (dequantize to the
compute dtype in forward and backward).

    a'_j = a_j                                   (plain absmax), or
    a'_j = RN_fp32( RN_fp32(q_j * sigma_d) + mu ) (double-quantized absmax)
    y_k  = RN_fp32( l[code_k] * a'_{block(k)} )
    bf16 output = RNE_bf16(y_k)

Signed zeros are kept (a negative level times a zero absmax is -0).
"""

import numpy as np

from .blockwise import unpack
from .double_quant import reconstruct_absmax, DQ_BLOCK
from .floats import f32_to_bf16_bits


def dequantize_f32(packed, n: int, blocksize: int, levels, absmax_eff) -> np.ndarray:
    codes = unpack(packed, n)
    lv = np.asarray(levels, dtype=np.float32)
    a = np.repeat(np.asarray(absmax_eff, dtype=np.float32), blocksize)[:n]
    with np.errstate(under="ignore"):
        return (lv[codes] * a).astype(np.float32)


def dequantize_bf16_bits(packed, n: int, blocksize: int, levels, absmax_eff) -> np.ndarray:
    return f32_to_bf16_bits(dequantize_f32(packed, n, blocksize, levels, absmax_eff))


def effective_absmax(absmax=None, q=None, sigma=None, mu=None, dq_block: int = DQ_BLOCK) -> np.ndarray:
    if absmax is not None:
        return np.asarray(absmax, dtype=np.float32)
    return reconstruct_absmax(q, sigma, mu, dq_block)
