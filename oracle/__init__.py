"""CPU oracle for blockwise 4-bit weight quantization (NF4 / FP4, double quantization,
dequantization and the dequantized QLoRA matmul).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never imports, links or calls it, and
this package imports nothing from the product path.

Everything here is plain, slow and written to be checked by eye against the
pages it follows:

* "篇2-bitsandbytes-具体观-算法与实现剖析" (xyzblog), §2.2 QLoRA / NF4 and
  figure 2-2 (the quantization pipeline and the nested quant_state), §2.3 and
  figure 2-3 (8-bit blockwise states with the dynamic map), §2.1 and figure 2-1
  (LLM.int8() vector-wise quantization with outlier decomposition);
* "Tim Dettmers 如何用 bitsandbytes 與 QLoRA 降低 LLM 訓練門檻？" (yololab),
  the sections on NF4, double quantization and QLoRA;
* "bitsandbytes：让大语言模型在消费级硬件上运行的量化神器" (zingnex), the
  sections on 4-bit quantization and double quantization;
* "LLM 相關知識" (technicalnotes, tag qlora), the precision table, LoRA,
  dynamic dequantization and merge sections.

Floating point follows the precision each step is defined in (fp32 for the
per-element steps, fp64 for sums and matmuls); exact modes use
``fractions.Fraction`` and ``mpmath``.

Modules
-------
codebook      NF4 and FP4 level tables (step a1)
blockwise     block absmax, normalisation, nearest level, packing (a2-a4)
double_quant  mean-centred int8 quantization of the absmax array (a5)
dequant       absmax reconstruction and dequantization to fp32 / bf16 (a6)
matmul        Y = X·deq(W)^T + s·(X·A)·B in fp64 (a7, a8)
merge         LoRA merge into the dequantized weight, and requantization
backward      gradients of the QLoRA layer for the input and the adapter
blockwise8    8-bit blockwise quantization with the dynamic (quantile) map
int8          LLM.int8(): vector-wise int8 matmul with outlier decomposition
floats        exact rounding helpers (Fraction -> fp32, fp32 -> bf16 RNE)
memory        storage arithmetic (bytes of a quantized tensor, bits/param)

Parity pins: every function here is pinned by a test under ``tests/`` that
does not re-type its formula (closed forms, invariants, brute force, the
values the pages print).  No function is "parity unpinned".
"""

from . import floats, codebook, blockwise, double_quant, dequant, matmul, memory, merge, backward, blockwise8, int8  # noqa: F401
