"""Storage arithmetic of a quantized weight — oracle, test infrastructure only.

"bitsandbytes：让大语言模型在消费级硬件上运行的量化神器" (zingnex), sections
背景 (70B at fp16 is about 140 GB) and 4-bit 量化 (about 35 GB at 4 bit) and
分页优化器与双量化 (double quantization saves about 0.37 bit per parameter);
"篇2-bitsandbytes-具体观-算法与实现剖析", §2.2 【原理】 ② (4 + 0.5 bit becomes
4 + 0.13 bit) and §2.4 【例子】 (13B: 26 GB at fp16, 6.5 GB at 4 bit).

Bytes of one quantized tensor of n elements at block size B:
    codes      ceil(n/2)
    absmax     4 * nb                         (plain), or
    q8 + sigma + mu   nb + 4 * ceil(nb/256) + 4   (double-quantized)
"""

from fractions import Fraction


def nblocks(n: int, blocksize: int) -> int:
    return (n + blocksize - 1) // blocksize


def state_bytes(n: int, blocksize: int = 64, nested: bool = True, dq_block: int = 256) -> int:
    nb = nblocks(n, blocksize)
    codes = (n + 1) // 2
    if not nested:
        return codes + 4 * nb
    nd = (nb + dq_block - 1) // dq_block
    return codes + nb + 4 * nd + 4


def bits_per_param(blocksize: int = 64, nested: bool = True, dq_block: int = 256) -> Fraction:
    """Asymptotic bits per parameter (large n): 4 for the code plus the scale overhead."""
    if not nested:
        return Fraction(4) + Fraction(32, blocksize)
    return Fraction(4) + Fraction(8, blocksize) + Fraction(32, blocksize * dq_block)


def dense_bytes(n: int, bytes_per_elem: float) -> float:
    return n * bytes_per_elem
