"""Helpers shared by the GPU parity tests (host-side marshalling only)."""

import sys

import numpy as np
import pytest
import torch

import bit_blockwise_weight_amd as qk


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    # the product path must load; a missing library is a failure, not a skip
    qk.lib()


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_f16(a_f32: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a_f32, dtype=np.float16)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str):
    got = np.ascontiguousarray(got)
    want = np.ascontiguousarray(want)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    if got.dtype.itemsize == 4:
        g, w = got.view(np.uint32), want.view(np.uint32)
    elif got.dtype.itemsize == 2:
        g, w = got.view(np.uint16), want.view(np.uint16)
    else:
        g, w = got.view(np.uint8), want.view(np.uint8)
    bad = np.nonzero(g != w)[0]
    assert bad.size == 0, (f"{what}: {bad.size} of {g.size} differ; first at {bad[:5].tolist()}: "
                           f"got {g[bad[:5]].tolist()} want {w[bad[:5]].tolist()}")
