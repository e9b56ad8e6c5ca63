"""8-bit blockwise quantization with a dynamic map — oracle, test infrastructure only.

"篇2-bitsandbytes-具体观-算法与实现剖析", §2.3 8-bit Optimizers, 【原理】 and
figure 2-3: the optimizer states (Adam's m and v) are cut into blocks of 2048
elements, each block is scaled by its own absmax and quantized to 8 bits through
a dynamic quantization map: 256 non-uniform levels shaped by the distribution,
dense near zero and sparse in the tails, chosen to maximise the information
entropy of the codes (the page calls it the int8 version of the NF4 idea).  The
same page's 【代码】 names a signed map ("dynamic") and an unsigned one
("udynamic").

Readings taken where the page is silent (it names the map and its properties but
gives no construction):

* Signed map: the NF4 construction with 256 slabs, l_i = RN_fp32(q_i / q_255),
  q_i = Phi^-1((2i+1)/512).  Equal probability mass per level is what maximises
  the code entropy for normally distributed data; the levels are densest at 0.
* Unsigned map (non-negative states such as v): the same on the half-normal,
  q_i = Phi^-1(1/2 + (2i+1)/1024), l_i = RN_fp32(q_i / q_255), all in (0, 1].
* Blocking, absmax, t = RN(x / a) and the nearest level (ties to the lower
  index) are those of the 4-bit path (blockwise.py); one code per byte.
* Dequantization: y = RN_fp32(l[code] * a).
"""

import mpmath
import numpy as np

from .blockwise import absmax, normalize, nearest_code, num_blocks
from .codebook import _mpf_to_fraction
from .floats import fraction_to_f32

SIGNED = 1
UNSIGNED = 0
DEFAULT_BLOCK = 2048


def dynamic_quantiles(signed: bool, dps: int = 50):
    """q_i as mpmath numbers, i = 0..255."""
    with mpmath.workdps(dps):
        if signed:
            p = [mpmath.mpf(2 * i + 1) / 512 for i in range(256)]
        else:
            p = [mpmath.mpf(1) / 2 + mpmath.mpf(2 * i + 1) / 1024 for i in range(256)]
        return [mpmath.sqrt(2) * mpmath.erfinv(2 * pi - 1) for pi in p]


def dynamic_map(signed: bool) -> np.ndarray:
    with mpmath.workdps(50):
        q = dynamic_quantiles(signed, 50)
        fr = [_mpf_to_fraction(q[i] / q[255]) for i in range(256)]
    return np.array([fraction_to_f32(f) for f in fr], dtype=np.float32)


def quantize_blockwise8(x: np.ndarray, blocksize: int, levels: np.ndarray):
    """Returns (codes uint8[n], absmax fp32[ceil(n/B)])."""
    x = np.asarray(x, dtype=np.float32).reshape(-1)
    a = absmax(x, blocksize)
    t = normalize(x, a, blocksize)
    return nearest_code(t, levels), a


def dequantize_blockwise8(codes, absmax_, n: int, blocksize: int, levels) -> np.ndarray:
    lv = np.asarray(levels, dtype=np.float32)
    a = np.repeat(np.asarray(absmax_, dtype=np.float32), blocksize)[:n]
    with np.errstate(under="ignore"):
        return (lv[np.asarray(codes).reshape(-1)[:n]] * a).astype(np.float32)


def state_bytes8(n: int, blocksize: int = DEFAULT_BLOCK) -> int:
    """Bytes of one 8-bit state: one code per element plus an fp32 absmax per block."""
    return n + 4 * num_blocks(n, blocksize)
