"""The oracle's quantize / dequantize steps over a large tensor, spread across host
cores (test helper).  Blocks are independent, so the flattened tensor is cut into
chunks at multiples of the block size (and of 2, so code bytes do not straddle
chunks); each worker runs the oracle's own functions on its chunk.  The double
quantization needs the whole absmax array and runs once, in this process.

Workers are started with "spawn" (no inherited GPU state) and import only
numpy and the oracle."""

import multiprocessing as mp
import os

import numpy as np

CHUNK = 1 << 24            # elements per task, a multiple of every block size


def _quantize_chunk(args):
    from oracle import blockwise as obw
    bits, B, levels = args
    xf = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return obw.quantize_blockwise(xf, B, levels)


def _dequant_chunk(args):
    from oracle import dequant as odq
    packed, n, B, levels, a_eff = args
    return odq.dequantize_bf16_bits(packed, n, B, levels, a_eff)


def _pool():
    workers = min(16, os.cpu_count() or 1)
    return mp.get_context("spawn").Pool(workers)


def quantize_bf16(bits: np.ndarray, B: int, levels: np.ndarray):
    """(codes, absmax) of the oracle for bf16 bits, chunk by chunk."""
    flat = np.ascontiguousarray(bits, dtype=np.uint16).reshape(-1)
    tasks = [(flat[i:i + CHUNK], B, levels) for i in range(0, flat.size, CHUNK)]
    with _pool() as p:
        parts = p.map(_quantize_chunk, tasks)
    return np.concatenate([c for c, _ in parts]), np.concatenate([a for _, a in parts])


def dequantize_bf16(codes: np.ndarray, n: int, B: int, levels: np.ndarray, a_eff: np.ndarray):
    """bf16 bits of the oracle's dequantization, chunk by chunk."""
    tasks = []
    for i in range(0, n, CHUNK):
        m = min(CHUNK, n - i)
        tasks.append((codes[i // 2:(i + m + 1) // 2], m, B, levels, a_eff[i // B:(i + m + B - 1) // B]))
    with _pool() as p:
        parts = p.map(_dequant_chunk, tasks)
    return np.concatenate(parts)
