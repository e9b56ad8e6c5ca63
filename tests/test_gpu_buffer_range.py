"""The GEMV kernels put a tile's first row and a job's chunk into the scalar
offset of their buffer loads and rely on the hardware's range check to turn
rows past a weight's end into zeros.  This checks that on the device the check
covers the vector plus the scalar offset (a raw buffer load with the LDS bit,
512 bytes in range): with a scalar offset of 256 every lane whose vector offset
is 256 or more must read zero, though its address lies inside the allocation."""

import ctypes
import os

import numpy as np
import pytest
import torch

from tests.gpu_common import require_gpu, say

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "bit_blockwise_weight_amd",
                     "libqk_probe.so")


def test_scalar_offset_takes_part_in_the_range_check():
    require_gpu()
    if not os.path.exists(PROBE):
        pytest.fail("libqk_probe.so is not built; run python -m bit_blockwise_weight_amd.build")
    lib = ctypes.CDLL(PROBE)
    lib.qk_probe_buffer_range.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_uint32,
                                          ctypes.c_void_p]
    lib.qk_probe_buffer_range.restype = ctypes.c_int
    words = np.arange(0x1000, 0x1000 + 1024, dtype=np.uint32)          # 4096 bytes, all nonzero
    src = torch.from_numpy(words.view(np.int32)).cuda()
    out = torch.empty(256, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for soff in (0, 256):
        say(f"case: buffer range check, scalar offset {soff}")
        assert lib.qk_probe_buffer_range(src.data_ptr(), 4096, out.data_ptr(), soff, stream) == 0
        torch.cuda.synchronize()
        got = out.cpu().numpy().view(np.uint32).reshape(64, 4)
        for lane in range(64):
            start = 16 * lane + soff
            want = words[start // 4: start // 4 + 4] if 16 * lane + soff < 512 else np.zeros(4, np.uint32)
            assert (got[lane] == want).all(), (soff, lane, got[lane], want)
