"""C-ABI tests that need no GPU: the library loads, exports every call that
include/qk.h declares, builds the level tables on the host exactly as the
oracle defines them, and rejects bad arguments and corrupted descriptors with
the documented status before touching any device."""

import ctypes
import os
import re

import numpy as np
import pytest

import bit_blockwise_weight_amd as qk
from oracle import codebook

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x10000)        # never dereferenced: every case fails validation first


def _declared_symbols():
    src = open(os.path.join(ROOT, "include", "qk.h"), encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qk_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(qk.LIB_PATH):
        pytest.fail("libqk.so is not built; run python -m bit_blockwise_weight_amd.build")
    return qk.lib()


def test_exports_every_declared_symbol(L):
    names = _declared_symbols()
    assert len(names) >= 11
    for name in names:
        assert hasattr(L, name), name


def test_version_and_backend_strings(L):
    assert "gfx950" in qk.qk_version()
    assert "quantize" in qk.qk_backend_info()


def test_nf4_table_matches_oracle_bitwise(L):
    got = qk.qk_make_codebook(qk.NF4).numpy()
    np.testing.assert_array_equal(got.view(np.uint32), codebook.nf4_levels().view(np.uint32))


def test_fp4_table_matches_oracle_bitwise(L):
    got = qk.qk_make_codebook(qk.FP4).numpy()
    np.testing.assert_array_equal(got.view(np.uint32), codebook.fp4_levels().view(np.uint32))


def test_make_codebook_errors(L):
    buf = (ctypes.c_float * 16)()
    assert L.qk_make_codebook(7, buf) == qk.QK_ERR_INVALID_ARG
    assert "unknown kind" in qk.qk_last_error()
    assert L.qk_make_codebook(0, None) == qk.QK_ERR_INVALID_ARG


def _levels(kind=qk.NF4):
    lv = qk.qk_make_codebook(kind).tolist()
    return (ctypes.c_float * 16)(*lv)


def test_quantize_argument_errors(L):
    lv = _levels()
    s = None
    assert L.qk_quantize_blockwise(None, qk.QK_BF16, 64, 64, lv, FAKE, FAKE, s) == qk.QK_ERR_INVALID_ARG
    assert L.qk_quantize_blockwise(FAKE, qk.QK_BF16, 0, 64, lv, FAKE, FAKE, s) == qk.QK_ERR_INVALID_ARG
    assert L.qk_quantize_blockwise(FAKE, qk.QK_BF16, 64, 32, lv, FAKE, FAKE, s) == qk.QK_ERR_INVALID_ARG
    assert "block size" in qk.qk_last_error()
    assert L.qk_quantize_blockwise(FAKE, 9, 64, 64, lv, FAKE, FAKE, s) == qk.QK_ERR_INVALID_ARG
    assert L.qk_quantize_blockwise(ctypes.c_void_p(0x10002), qk.QK_BF16, 64, 64, lv, FAKE, FAKE, s) \
        == qk.QK_ERR_INVALID_ARG
    assert "aligned" in qk.qk_last_error()
    bad = (ctypes.c_float * 16)(*([2.0] + [0.0] * 15))
    assert L.qk_quantize_blockwise(FAKE, qk.QK_BF16, 64, 64, bad, FAKE, FAKE, s) == qk.QK_ERR_INVALID_ARG
    nan = (ctypes.c_float * 16)(*([float("nan")] + [0.0] * 15))
    assert L.qk_quantize_blockwise(FAKE, qk.QK_BF16, 64, 64, nan, FAKE, FAKE, s) == qk.QK_ERR_INVALID_ARG


def test_quantize_rejects_table_whose_lookup_is_not_exact(L):
    # three levels one ulp apart: two thresholds one ulp apart cannot sit in different bins
    lv = qk.qk_make_codebook(qk.NF4).numpy().copy()
    lv[13] = np.nextafter(lv[12], np.float32(1.0))
    lv[14] = np.nextafter(lv[13], np.float32(1.0))
    arr = (ctypes.c_float * 16)(*lv.tolist())
    assert L.qk_quantize_blockwise(FAKE, qk.QK_BF16, 64, 64, arr, FAKE, FAKE, None) == qk.QK_ERR_UNSUPPORTED


def test_quantize_accepts_table_with_a_threshold_at_zero(L):
    """Levels +-2^-40 (threshold: the least positive float) pass the table build:
    on a host without a GPU the call gets as far as the device check."""
    lv = [-1, -0.75, -0.5, -0.375, -0.25, -0.125, -0.0625, -2.0 ** -40, 2.0 ** -40, 0.0625, 0.125, 0.25,
          0.375, 0.5, 0.75, 1]
    arr = (ctypes.c_float * 16)(*lv)
    st = L.qk_quantize_blockwise(FAKE, qk.QK_BF16, 64, 64, arr, FAKE, FAKE, None)
    assert st not in (qk.QK_OK, qk.QK_ERR_INVALID_ARG, qk.QK_ERR_UNSUPPORTED), qk.qk_last_error()


def test_double_quant_errors_and_workspace(L):
    assert qk.qk_double_quant_workspace_size(1) >= 8
    assert qk.qk_double_quant_workspace_size(4096 * 4096 + 1) >= 8 * 4097
    out = ctypes.c_size_t()
    assert L.qk_double_quant_workspace_size(0, ctypes.byref(out)) == qk.QK_ERR_INVALID_ARG
    assert L.qk_double_quant(FAKE, 1000, 128, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == qk.QK_ERR_UNSUPPORTED
    assert L.qk_double_quant(FAKE, 1000, 256, FAKE, FAKE, FAKE, None, 0, None) == qk.QK_ERR_WORKSPACE
    assert L.qk_double_quant(FAKE, 1000, 256, FAKE, FAKE, FAKE, FAKE, 0, None) == qk.QK_ERR_WORKSPACE
    assert "workspace" in qk.qk_last_error()
    assert L.qk_double_quant(FAKE, 0, 256, FAKE, FAKE, FAKE, FAKE, 64, None) == qk.QK_ERR_INVALID_ARG


def _state(nested=True):
    st = qk.QuantState()
    lv = _levels()
    if nested:
        rc = L_().qk_state_init(ctypes.byref(st), qk.NF4, lv, 4, 64, 64, FAKE, None, FAKE, FAKE, FAKE)
    else:
        rc = L_().qk_state_init(ctypes.byref(st), qk.NF4, lv, 4, 64, 64, FAKE, FAKE, None, None, None)
    assert rc == qk.QK_OK
    return st


def L_():
    return qk.lib()


def test_state_init_fills_descriptor(L):
    st = _state()
    assert st.magic == qk.QK_STATE_MAGIC and st.version == qk.QK_STATE_VERSION
    assert st.struct_bytes == ctypes.sizeof(qk.QuantState) == 160
    assert st.n == 256 and st.nested == 1 and st.dq_blocksize == 256
    lv = _levels()
    bad = qk.QuantState()
    assert L.qk_state_init(ctypes.byref(bad), qk.NF4, lv, 4, 64, 64, FAKE, FAKE, FAKE, FAKE, FAKE) \
        == qk.QK_ERR_INVALID_ARG
    assert L.qk_state_init(ctypes.byref(bad), qk.NF4, lv, 0, 64, 64, FAKE, FAKE, None, None, None) \
        == qk.QK_ERR_INVALID_ARG
    assert L.qk_state_init(ctypes.byref(bad), qk.NF4, lv, 4, 64, 48, FAKE, FAKE, None, None, None) \
        == qk.QK_ERR_INVALID_ARG


@pytest.mark.parametrize("field,value", [
    ("magic", 0xDEADBEEF), ("version", 99), ("struct_bytes", 100), ("blocksize", 32), ("n", 255),
    ("nested", 2), ("dq_blocksize", 128), ("q8", None), ("codes", None), ("reserved", 1),
    ("codebook_kind", 17), ("codes", 0x10001),
])
def test_corrupted_descriptor_is_rejected_by_every_consumer(L, field, value):
    st = _state()
    setattr(st, field, value)
    y = FAKE
    assert L.qk_dequantize(ctypes.byref(st), y, qk.QK_BF16, None) == qk.QK_ERR_BAD_STATE
    assert L.qk_gemv_nf4(FAKE, 1, ctypes.byref(st), y, None) == qk.QK_ERR_BAD_STATE
    assert L.qk_gemm_nf4(FAKE, 4, ctypes.byref(st), None, None, 0, 0.0, y, None, 0, None) == qk.QK_ERR_BAD_STATE
    assert L.qk_lora_merge(ctypes.byref(st), FAKE, FAKE, 16, 2.0, y, None) == qk.QK_ERR_BAD_STATE
    assert "quant state" in qk.qk_last_error()


def test_nonfinite_level_in_descriptor(L):
    st = _state()
    st.levels[3] = float("inf")
    assert L.qk_dequantize(ctypes.byref(st), FAKE, qk.QK_BF16, None) == qk.QK_ERR_BAD_STATE


def test_consumer_argument_errors(L):
    st = _state()
    assert L.qk_dequantize(ctypes.byref(st), None, qk.QK_BF16, None) == qk.QK_ERR_INVALID_ARG
    assert L.qk_dequantize(ctypes.byref(st), FAKE, qk.QK_F16, None) == qk.QK_ERR_INVALID_ARG
    assert L.qk_dequantize(None, FAKE, qk.QK_BF16, None) == qk.QK_ERR_INVALID_ARG
    assert L.qk_gemv_nf4(FAKE, 0, ctypes.byref(st), FAKE, None) == qk.QK_ERR_INVALID_ARG
    assert L.qk_gemv_nf4(FAKE, 17, ctypes.byref(st), FAKE, None) == qk.QK_ERR_INVALID_ARG
    assert L.qk_gemm_nf4(FAKE, 0, ctypes.byref(st), None, None, 0, 0.0, FAKE, None, 0, None) == qk.QK_ERR_INVALID_ARG
    assert L.qk_gemm_nf4(FAKE, 8, ctypes.byref(st), FAKE, None, 16, 2.0, FAKE, FAKE, 1 << 20, None) \
        == qk.QK_ERR_INVALID_ARG
    assert L.qk_gemm_nf4(FAKE, 8, ctypes.byref(st), FAKE, FAKE, 65, 2.0, FAKE, FAKE, 1 << 20, None) \
        == qk.QK_ERR_INVALID_ARG
    assert L.qk_gemm_nf4(FAKE, 8, ctypes.byref(st), FAKE, FAKE, 16, float("inf"), FAKE, FAKE, 1 << 20, None) \
        == qk.QK_ERR_INVALID_ARG
    # LoRA needs a workspace of the queried size
    need = qk.qk_gemm_nf4_workspace_size(8, 16)
    assert need >= 8 * 16 * 4
    assert qk.qk_gemm_nf4_workspace_size(8, 0) == 0
    assert L.qk_gemm_nf4(FAKE, 8, ctypes.byref(st), FAKE, FAKE, 16, 2.0, FAKE, None, 0, None) == qk.QK_ERR_WORKSPACE
    assert L.qk_gemm_nf4(FAKE, 8, ctypes.byref(st), FAKE, FAKE, 16, 2.0, FAKE, FAKE, need - 1, None) \
        == qk.QK_ERR_WORKSPACE
    assert "workspace" in qk.qk_last_error()
    out = ctypes.c_size_t()
    assert L.qk_gemm_nf4_workspace_size(8, 65, ctypes.byref(out)) == qk.QK_ERR_INVALID_ARG


def test_lora_merge_argument_errors(L):
    st = _state()
    assert L.qk_lora_merge(ctypes.byref(st), None, FAKE, 16, 2.0, FAKE, None) == qk.QK_ERR_INVALID_ARG
    assert L.qk_lora_merge(ctypes.byref(st), FAKE, None, 16, 2.0, FAKE, None) == qk.QK_ERR_INVALID_ARG
    assert L.qk_lora_merge(ctypes.byref(st), FAKE, FAKE, 16, 2.0, None, None) == qk.QK_ERR_INVALID_ARG
    assert L.qk_lora_merge(ctypes.byref(st), FAKE, FAKE, 0, 2.0, FAKE, None) == qk.QK_ERR_INVALID_ARG
    assert L.qk_lora_merge(ctypes.byref(st), FAKE, FAKE, 1025, 2.0, FAKE, None) == qk.QK_ERR_INVALID_ARG
    assert "rank" in qk.qk_last_error()
    assert L.qk_lora_merge(ctypes.byref(st), FAKE, FAKE, 16, float("nan"), FAKE, None) == qk.QK_ERR_INVALID_ARG
    assert L.qk_lora_merge(ctypes.byref(st), FAKE, FAKE, 16, 2.0, ctypes.c_void_p(0x10001), None) \
        == qk.QK_ERR_INVALID_ARG
    assert L.qk_lora_merge(None, FAKE, FAKE, 16, 2.0, FAKE, None) == qk.QK_ERR_INVALID_ARG


def test_missing_library_error_is_deferred(tmp_path, monkeypatch):
    """A missing .so does not break import; the first call raises QKError."""
    monkeypatch.setattr(qk, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(qk, "_lib", None)
    monkeypatch.setattr(qk, "_load_error", None)
    with pytest.raises(qk.QKError) as ei:
        qk.qk_make_codebook(qk.NF4)
    assert "not built" in str(ei.value)


def test_qlora_backward_argument_errors(L):
    st = qk.QuantState()
    assert L.qk_state_init(ctypes.byref(st), qk.NF4, _levels(), 128, 64, 64, FAKE, None, FAKE, FAKE, FAKE) == qk.QK_OK
    ws = ctypes.c_size_t(0)
    assert L.qk_qlora_backward_workspace_size(8, ctypes.byref(st), 16, ctypes.byref(ws)) == qk.QK_OK
    need = ws.value
    assert need > 0
    assert L.qk_qlora_backward_workspace_size(8, ctypes.byref(st), 0, ctypes.byref(ws)) == qk.QK_OK and ws.value == 0
    assert L.qk_qlora_backward_workspace_size(8, ctypes.byref(st), 65, ctypes.byref(ws)) == qk.QK_ERR_INVALID_ARG
    assert L.qk_qlora_backward_workspace_size(0, ctypes.byref(st), 16, ctypes.byref(ws)) == qk.QK_ERR_INVALID_ARG

    def call(dY=FAKE, M=8, s=st, X=FAKE, A=FAKE, B=FAKE, r=16, scale=2.0, dX=FAKE, dA=FAKE, dB=FAKE, w=FAKE,
             wb=need):
        return L.qk_qlora_backward(dY, M, None if s is None else ctypes.byref(s), X, A, B, r, scale, dX, dA, dB,
                                   w, wb, None)

    assert call(dY=None) == qk.QK_ERR_INVALID_ARG
    assert call(dX=None) == qk.QK_ERR_INVALID_ARG
    assert call(M=0) == qk.QK_ERR_INVALID_ARG
    assert call(B=None) == qk.QK_ERR_INVALID_ARG
    assert call(r=65) == qk.QK_ERR_INVALID_ARG
    assert "rank" in qk.qk_last_error()
    assert call(X=None) == qk.QK_ERR_INVALID_ARG
    assert call(dA=None) == qk.QK_ERR_INVALID_ARG
    assert call(scale=float("inf")) == qk.QK_ERR_INVALID_ARG
    assert call(dY=ctypes.c_void_p(0x10008)) == qk.QK_ERR_INVALID_ARG          # not 16-byte aligned
    assert call(wb=need - 1) == qk.QK_ERR_WORKSPACE
    assert call(w=None) == qk.QK_ERR_WORKSPACE
    assert call(s=None) == qk.QK_ERR_INVALID_ARG
    small = _state()                                                            # W [4, 64]: N % 64 != 0
    assert call(s=small) == qk.QK_ERR_UNSUPPORTED
    assert "multiples of 64" in qk.qk_last_error()


def test_dynamic_map_matches_oracle_bitwise(L):
    """The library's host map (AS 241 quantiles in binary64) equals the oracle's
    (mpmath, 50 digits) after rounding to binary32."""
    from oracle import blockwise8 as o8
    for signed in (True, False):
        got = qk.qk_make_dynamic_map(signed).numpy()
        assert np.array_equal(got.view(np.uint32), o8.dynamic_map(signed).view(np.uint32))


def test_quantize8_argument_errors(L):
    lv = (ctypes.c_float * 256)(*qk.qk_make_dynamic_map(True).tolist())
    q = L.qk_quantize_blockwise_8bit
    assert q(None, qk.QK_F32, 10, 2048, lv, FAKE, FAKE, None) == qk.QK_ERR_INVALID_ARG
    assert q(FAKE, qk.QK_F32, 0, 2048, lv, FAKE, FAKE, None) == qk.QK_ERR_INVALID_ARG
    assert q(FAKE, 7, 10, 2048, lv, FAKE, FAKE, None) == qk.QK_ERR_INVALID_ARG
    assert q(FAKE, qk.QK_F32, 10, 64, lv, FAKE, FAKE, None) == qk.QK_ERR_INVALID_ARG
    assert "block size" in qk.qk_last_error()
    assert q(FAKE, qk.QK_F32, 10, 2048, lv, ctypes.c_void_p(0x10004), FAKE, None) == qk.QK_ERR_INVALID_ARG
    bad = (ctypes.c_float * 256)(*([0.5] * 255 + [1.5]))
    assert q(FAKE, qk.QK_F32, 10, 2048, bad, FAKE, FAKE, None) == qk.QK_ERR_INVALID_ARG
    close = (ctypes.c_float * 256)(*[i * 1e-5 for i in range(256)])     # thresholds 1e-5 apart
    assert q(FAKE, qk.QK_F32, 10, 2048, close, FAKE, FAKE, None) == qk.QK_ERR_UNSUPPORTED
    d = L.qk_dequantize_blockwise_8bit
    assert d(None, FAKE, 10, 2048, lv, FAKE, qk.QK_F32, None) == qk.QK_ERR_INVALID_ARG
    assert d(FAKE, FAKE, 10, 2048, lv, FAKE, qk.QK_F16, None) == qk.QK_ERR_INVALID_ARG
    assert d(FAKE, FAKE, 10, 100, lv, FAKE, qk.QK_F32, None) == qk.QK_ERR_INVALID_ARG
    assert d(ctypes.c_void_p(0x10004), FAKE, 10, 2048, lv, FAKE, qk.QK_F32, None) == qk.QK_ERR_INVALID_ARG
    nan = (ctypes.c_float * 256)(*([float("nan")] + [0.0] * 255))
    assert d(FAKE, FAKE, 10, 2048, nan, FAKE, qk.QK_F32, None) == qk.QK_ERR_INVALID_ARG


def test_int8_argument_errors(L):
    q = L.qk_int8_quantize_rows
    assert q(None, qk.QK_F16, 4, 64, None, FAKE, FAKE, None) == qk.QK_ERR_INVALID_ARG
    assert q(FAKE, 9, 4, 64, None, FAKE, FAKE, None) == qk.QK_ERR_INVALID_ARG
    assert q(FAKE, qk.QK_F16, 0, 64, None, FAKE, FAKE, None) == qk.QK_ERR_INVALID_ARG
    assert q(FAKE, qk.QK_F16, 4, 60, None, FAKE, FAKE, None) == qk.QK_ERR_INVALID_ARG     # cols % 8
    assert q(FAKE, qk.QK_F16, 4, 64, ctypes.c_void_p(0x10004), FAKE, FAKE, None) == qk.QK_ERR_INVALID_ARG
    o = L.qk_int8_outlier_columns
    assert o(FAKE, qk.QK_F16, 4, 64, 6.0, None, FAKE, FAKE, FAKE, None) == qk.QK_ERR_INVALID_ARG
    assert o(FAKE, qk.QK_F16, 4, 64, -1.0, FAKE, FAKE, FAKE, FAKE, None) == qk.QK_ERR_INVALID_ARG
    assert o(FAKE, qk.QK_F16, 4, 64, float("nan"), FAKE, FAKE, FAKE, FAKE, None) == qk.QK_ERR_INVALID_ARG
    assert o(FAKE, qk.QK_F16, 4, 12, 6.0, FAKE, FAKE, FAKE, FAKE, None) == qk.QK_ERR_INVALID_ARG  # K % 8
    m = L.qk_int8_matmul
    assert m(FAKE, FAKE, FAKE, FAKE, 4, 4, 64, None, None, None, None, None) == qk.QK_ERR_INVALID_ARG
    assert m(FAKE, FAKE, FAKE, FAKE, 4, 4, 64, FAKE, None, FAKE, FAKE, None) == qk.QK_ERR_INVALID_ARG
    assert "together" in qk.qk_last_error()
    assert m(FAKE, FAKE, FAKE, FAKE, 4, 4, 8, None, None, None, FAKE, None) == qk.QK_ERR_INVALID_ARG   # K >= 16
    assert m(FAKE, FAKE, FAKE, FAKE, 4, 4, 72, None, None, None, FAKE, None) == qk.QK_ERR_INVALID_ARG  # K % 16
    assert m(ctypes.c_void_p(0x10008), FAKE, FAKE, FAKE, 4, 4, 64, None, None, None, FAKE, None) \
        == qk.QK_ERR_INVALID_ARG
    assert m(FAKE, FAKE, FAKE, FAKE, 0, 4, 64, None, None, None, FAKE, None) == qk.QK_ERR_INVALID_ARG


def test_binding_checks_gemv_gemm_operands(L):
    """The binding refuses operands whose dtype or shape does not match the
    descriptor before anything reaches the device (W here is [4, 64])."""
    import torch
    st = _state()
    bf = torch.bfloat16
    x = torch.zeros(2, 64, dtype=bf)
    with pytest.raises(ValueError, match="bf16"):
        qk.qk_gemv_nf4(x.float(), st)
    with pytest.raises(ValueError, match="columns"):
        qk.qk_gemv_nf4(torch.zeros(2, 48, dtype=bf), st)
    with pytest.raises(ValueError, match="does not hold"):
        qk.qk_gemv_nf4(x, st, torch.zeros(2, 3, dtype=bf))
    with pytest.raises(ValueError, match="must be"):
        qk.qk_gemv_nf4(x, st, torch.zeros(2, 4, dtype=torch.float32))
    A, B = torch.zeros(64, 16, dtype=bf), torch.zeros(16, 4, dtype=bf)
    with pytest.raises(ValueError, match="X must be bf16"):
        qk.qk_gemm_nf4(x.half(), st, A, B, 2.0)
    with pytest.raises(ValueError, match="A must be bf16"):
        qk.qk_gemm_nf4(x, st, A.float(), B, 2.0)
    with pytest.raises(ValueError, match="B must be bf16"):
        qk.qk_gemm_nf4(x, st, A, B.half(), 2.0)
    with pytest.raises(ValueError, match="do not match"):
        qk.qk_gemm_nf4(x, st, torch.zeros(32, 16, dtype=bf), B, 2.0)
    with pytest.raises(ValueError, match="do not match"):
        qk.qk_gemm_nf4(x, st, A, torch.zeros(16, 3, dtype=bf), 2.0)
    with pytest.raises(ValueError, match="do not match"):
        qk.qk_gemm_nf4(x, st, A, torch.zeros(8, 4, dtype=bf), 2.0)
    with pytest.raises(ValueError, match="neither"):
        qk.qk_gemm_nf4(x, st, A, None, 2.0)
    with pytest.raises(ValueError, match="does not hold"):
        qk.qk_gemm_nf4(x, st, A, B, 2.0, Y=torch.zeros(3, 4, dtype=bf))
    with pytest.raises(ValueError, match="must be"):
        qk.qk_gemm_nf4(x, st, Y=torch.zeros(2, 4, dtype=torch.float16))
    # well-formed host tensors get as far as the device check
    with pytest.raises(ValueError, match="HIP device"):
        qk.qk_gemm_nf4(x, st, A, B, 2.0)


def test_gemm_noalloc_argument_errors(L):
    """qk_gemm_nf4_noalloc validates like qk_gemm_nf4 and refuses LoRA partials
    beyond its static scratch (M * 16 * ceil(r / 16) <= 262144) before any device
    work."""
    st = _state()
    call = L.qk_gemm_nf4_noalloc
    assert call(None, 8, ctypes.byref(st), None, None, 0, 0.0, FAKE, None) == qk.QK_ERR_INVALID_ARG
    assert call(FAKE, 0, ctypes.byref(st), None, None, 0, 0.0, FAKE, None) == qk.QK_ERR_INVALID_ARG
    assert call(FAKE, 8, ctypes.byref(st), FAKE, None, 16, 2.0, FAKE, None) == qk.QK_ERR_INVALID_ARG
    assert call(FAKE, 8, ctypes.byref(st), FAKE, FAKE, 65, 2.0, FAKE, None) == qk.QK_ERR_INVALID_ARG
    assert call(FAKE, 8, ctypes.byref(st), FAKE, FAKE, 16, float("nan"), FAKE, None) == qk.QK_ERR_INVALID_ARG
    bad = _state()
    bad.magic = 0
    assert call(FAKE, 8, ctypes.byref(bad), None, None, 0, 0.0, FAKE, None) == qk.QK_ERR_BAD_STATE
    assert call(FAKE, 16385, ctypes.byref(st), FAKE, FAKE, 16, 2.0, FAKE, None) == qk.QK_ERR_WORKSPACE
    assert "static scratch" in qk.qk_last_error()
    assert call(FAKE, 4097, ctypes.byref(st), FAKE, FAKE, 64, 2.0, FAKE, None) == qk.QK_ERR_WORKSPACE
    assert call(FAKE, 8193, ctypes.byref(st), FAKE, FAKE, 17, 2.0, FAKE, None) == qk.QK_ERR_WORKSPACE


def test_gemm_grouped_argument_errors_and_workspace(L):
    st = _state()                        # W [4, 64]: X [M, 64], Y [M, 4]
    T = qk.GemmTask

    def arr(*entries):
        a = (T * len(entries))()
        for i, (x, m, s, A, B, r, y) in enumerate(entries):
            a[i].X, a[i].M, a[i].A, a[i].B, a[i].r, a[i].lora_scale, a[i].Y = x, m, A, B, r, 2.0, y
            a[i].st = None if s is None else ctypes.pointer(s)
        return a

    X0, Y0, Y1, A0, B0 = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000
    size = ctypes.c_size_t()
    ws = L.qk_gemm_nf4_grouped_workspace_size
    # workspace: the tasks' LoRA partials, each rounded up to 256 bytes; none without adapters
    assert ws(arr((X0, 10, st, None, None, 0, Y0)), 1, ctypes.byref(size)) == qk.QK_OK and size.value == 0
    assert ws(arr((X0, 10, st, A0, B0, 16, Y0), (X0, 300, st, A0, B0, 40, Y1)), 2, ctypes.byref(size)) == qk.QK_OK
    one = lambda M, r: (qk.qk_gemm_nf4_workspace_size(M, r) + 255) // 256 * 256
    assert size.value == one(10, 16) + one(300, 40)
    assert ws(arr((X0, 10, st, A0, B0, 16, Y0)), 1, None) == qk.QK_ERR_INVALID_ARG
    call = L.qk_gemm_nf4_grouped
    ok = arr((X0, 10, st, None, None, 0, Y0))
    assert call(None, 1, None, 0, None) == qk.QK_ERR_INVALID_ARG
    assert call(ok, 0, None, 0, None) == qk.QK_ERR_INVALID_ARG
    assert call(ok, 257, None, 0, None) == qk.QK_ERR_INVALID_ARG
    assert call(arr((X0, 10, None, None, None, 0, Y0)), 1, None, 0, None) == qk.QK_ERR_INVALID_ARG
    bad = _state()
    bad.version = 7
    assert call(arr((X0, 10, st, None, None, 0, Y0), (X0, 10, bad, None, None, 0, Y1)), 2, None, 0, None) \
        == qk.QK_ERR_BAD_STATE
    assert call(arr((X0, 0, st, None, None, 0, Y0)), 1, None, 0, None) == qk.QK_ERR_INVALID_ARG      # M < 1
    assert call(arr((X0, 10, st, A0, None, 16, Y0)), 1, None, 0, None) == qk.QK_ERR_INVALID_ARG      # A without B
    assert call(arr((X0, 10, st, A0, B0, 65, Y0)), 1, None, 0, None) == qk.QK_ERR_INVALID_ARG        # rank > 64
    assert "task 0" in qk.qk_last_error()
    # workspace missing, too small, misaligned
    lora = arr((X0, 10, st, A0, B0, 16, Y0))
    need = one(10, 16)
    assert call(lora, 1, None, 0, None) == qk.QK_ERR_WORKSPACE
    assert call(lora, 1, ctypes.c_void_p(0x600000), need - 1, None) == qk.QK_ERR_WORKSPACE
    assert call(lora, 1, ctypes.c_void_p(0x600008), need, None) == qk.QK_ERR_INVALID_ARG
    # Y [10, 4] bf16 = 80 bytes: overlapping outputs, an output over an input or the workspace
    assert call(arr((X0, 10, st, None, None, 0, Y0), (X0, 10, st, None, None, 0, Y0 + 78)), 2, None, 0, None) \
        == qk.QK_ERR_INVALID_ARG
    assert "overlaps Y" in qk.qk_last_error()
    assert call(arr((X0, 10, st, None, None, 0, Y0), (X0, 10, st, None, None, 0, X0 + 64)), 2, None, 0, None) \
        == qk.QK_ERR_INVALID_ARG
    assert "overlaps X" in qk.qk_last_error()
    assert call(lora, 1, ctypes.c_void_p(Y0 - 64), need, None) == qk.QK_ERR_INVALID_ARG
    assert "workspace" in qk.qk_last_error()
    # valid arguments get as far as the device check (no GPU here)
    st_ok = call(arr((X0, 10, st, None, None, 0, Y0), (X0, 10, st, None, None, 0, Y1)), 2, None, 0, None)
    assert st_ok not in (qk.QK_OK, qk.QK_ERR_INVALID_ARG, qk.QK_ERR_BAD_STATE, qk.QK_ERR_WORKSPACE)


def test_dequantize_grouped_argument_errors(L):
    st = _state()                        # W [4, 64]: 256 elements
    T = qk.DequantTask

    def arr(*entries):
        a = (T * len(entries))()
        for i, (s, o) in enumerate(entries):
            a[i].st = None if s is None else ctypes.pointer(s)
            a[i].out = o
        return a

    O0, O1 = 0x100000, 0x200000
    call = L.qk_dequantize_grouped
    ok = arr((st, O0), (st, O1))
    assert call(None, 1, qk.QK_BF16, None) == qk.QK_ERR_INVALID_ARG
    assert call(ok, 0, qk.QK_BF16, None) == qk.QK_ERR_INVALID_ARG
    assert call(ok, 257, qk.QK_BF16, None) == qk.QK_ERR_INVALID_ARG
    assert call(ok, 2, 9, None) == qk.QK_ERR_INVALID_ARG                           # out dtype
    assert call(arr((None, O0)), 1, qk.QK_BF16, None) == qk.QK_ERR_INVALID_ARG
    bad = _state()
    bad.version = 7
    assert call(arr((st, O0), (bad, O1)), 2, qk.QK_BF16, None) == qk.QK_ERR_BAD_STATE
    assert call(arr((st, None)), 1, qk.QK_BF16, None) == qk.QK_ERR_INVALID_ARG
    assert call(arr((st, O0 + 8)), 1, qk.QK_BF16, None) == qk.QK_ERR_INVALID_ARG    # out not 16-byte aligned
    # 256 bf16 = 512 bytes, 256 fp32 = 1024 bytes
    assert call(arr((st, O0), (st, O0 + 496)), 2, qk.QK_BF16, None) == qk.QK_ERR_INVALID_ARG
    assert "overlaps" in qk.qk_last_error()
    assert call(arr((st, O0), (st, O0 + 512)), 2, qk.QK_F32, None) == qk.QK_ERR_INVALID_ARG
    st_ok = call(arr((st, O0), (st, O0 + 512)), 2, qk.QK_BF16, None)
    assert st_ok not in (qk.QK_OK, qk.QK_ERR_INVALID_ARG, qk.QK_ERR_BAD_STATE)


def test_gemv_grouped_argument_errors(L):
    st = _state()                        # W [4, 64]
    T = qk.GemvTask

    def arr(*entries):
        a = (T * len(entries))()
        for i, (x, s, y) in enumerate(entries):
            a[i].x = x
            a[i].st = None if s is None else ctypes.pointer(s)
            a[i].y = y
        return a

    X0, Y0, Y1 = 0x100000, 0x200000, 0x300000
    ok = arr((X0, st, Y0))
    call = L.qk_gemv_nf4_grouped
    assert call(None, 1, 1, None) == qk.QK_ERR_INVALID_ARG
    assert call(ok, 0, 1, None) == qk.QK_ERR_INVALID_ARG
    assert call(ok, 257, 1, None) == qk.QK_ERR_INVALID_ARG
    assert call(ok, 1, 0, None) == qk.QK_ERR_INVALID_ARG
    assert call(ok, 1, 17, None) == qk.QK_ERR_INVALID_ARG
    assert call(arr((X0, None, Y0)), 1, 1, None) == qk.QK_ERR_INVALID_ARG
    bad = _state()
    bad.version = 7
    assert call(arr((X0, st, Y0), (X0, bad, Y1)), 2, 1, None) == qk.QK_ERR_BAD_STATE
    assert call(arr((None, st, Y0)), 1, 1, None) == qk.QK_ERR_INVALID_ARG
    assert call(arr((X0 + 8, st, Y0)), 1, 1, None) == qk.QK_ERR_INVALID_ARG      # x not 16-byte aligned
    assert call(arr((X0, st, Y0 + 1)), 1, 1, None) == qk.QK_ERR_INVALID_ARG      # y not 2-byte aligned
    # y [M, 4] bf16 = 8 bytes per row: overlapping outputs, an output over an input
    assert call(arr((X0, st, Y0), (X0, st, Y0 + 6)), 2, 1, None) == qk.QK_ERR_INVALID_ARG
    assert "overlaps y" in qk.qk_last_error()
    assert call(arr((X0, st, Y0), (X0, st, X0 + 64)), 2, 1, None) == qk.QK_ERR_INVALID_ARG
    assert "overlaps x" in qk.qk_last_error()


def test_double_quant_grouped_argument_errors(L):
    T = qk.DqTask

    def arr(*entries):
        a = (T * len(entries))()
        for i, (am, nb, q8, sc, mu) in enumerate(entries):
            a[i].absmax, a[i].nblocks, a[i].q8, a[i].scale, a[i].mean = am, nb, q8, sc, mu
        return a

    A0, A1, Q0, Q1, S0, S1, M0, M1 = (0x100000 * k for k in range(1, 9))
    one = arr((A0, 1000, Q0, S0, M0))
    two = arr((A0, 1000, Q0, S0, M0), (A1, 5000, Q1, S1, M1))
    size = ctypes.c_size_t()
    ws = L.qk_double_quant_grouped_workspace_size
    assert ws(two, 2, ctypes.byref(size)) == qk.QK_OK
    assert size.value == qk.qk_double_quant_workspace_size(1000) + qk.qk_double_quant_workspace_size(5000)
    assert qk.qk_double_quant_grouped_workspace_size([1000, 5000]) == size.value
    assert ws(None, 1, ctypes.byref(size)) == qk.QK_ERR_INVALID_ARG
    assert ws(one, 0, ctypes.byref(size)) == qk.QK_ERR_INVALID_ARG
    assert ws(one, 1, None) == qk.QK_ERR_INVALID_ARG
    assert ws(arr((A0, 0, Q0, S0, M0)), 1, ctypes.byref(size)) == qk.QK_ERR_INVALID_ARG
    call = L.qk_double_quant_grouped
    big = 1 << 20
    assert call(None, 1, 256, FAKE, big, None) == qk.QK_ERR_INVALID_ARG
    assert call(one, 0, 256, FAKE, big, None) == qk.QK_ERR_INVALID_ARG
    assert call(one, 257, 256, FAKE, big, None) == qk.QK_ERR_INVALID_ARG
    assert call(one, 1, 128, FAKE, big, None) == qk.QK_ERR_UNSUPPORTED
    assert call(one, 1, 256, None, 0, None) == qk.QK_ERR_WORKSPACE
    assert call(two, 2, 256, FAKE, qk.qk_double_quant_workspace_size(1000), None) == qk.QK_ERR_WORKSPACE
    assert call(arr((A0, 1000, None, S0, M0)), 1, 256, FAKE, big, None) == qk.QK_ERR_INVALID_ARG
    assert call(arr((A0, 0, Q0, S0, M0)), 1, 256, FAKE, big, None) == qk.QK_ERR_INVALID_ARG
    assert call(arr((A0 + 2, 1000, Q0, S0, M0)), 1, 256, FAKE, big, None) == qk.QK_ERR_INVALID_ARG
    assert call(one, 1, 256, ctypes.c_void_p(0x10004), big, None) == qk.QK_ERR_INVALID_ARG   # workspace alignment
    # an output over another task's output, over an absmax, or two outputs of one task
    assert call(arr((A0, 1000, Q0, S0, M0), (A1, 1000, Q0 + 512, S1, M1)), 2, 256, FAKE, big, None) == qk.QK_ERR_INVALID_ARG
    assert "overlaps" in qk.qk_last_error()
    assert call(arr((A0, 1000, Q0, S0, M0), (A1, 1000, Q1, S1, A0 + 4)), 2, 256, FAKE, big, None) == qk.QK_ERR_INVALID_ARG
    assert call(arr((A0, 1000, Q0, S0, S0 + 8)), 1, 256, FAKE, big, None) == qk.QK_ERR_INVALID_ARG
    # two tasks may read the same absmax
    assert ws(arr((A0, 1000, Q0, S0, M0), (A0, 1000, Q1, S1, M1)), 2, ctypes.byref(size)) == qk.QK_OK


def test_quantize_grouped_argument_errors(L):
    T = qk.QuantTask
    lv = _levels()

    def arr(*entries):
        a = (T * len(entries))()
        for i, (x, n, c, am) in enumerate(entries):
            a[i].x, a[i].n, a[i].codes, a[i].absmax = x, n, c, am
        return a

    X0, X1, C0, C1, A0, A1 = (0x1000000 * k for k in range(1, 7))
    one = arr((X0, 4096, C0, A0))
    call = L.qk_quantize_blockwise_grouped
    assert call(None, 1, qk.QK_BF16, 64, lv, None) == qk.QK_ERR_INVALID_ARG
    assert call(one, 1, qk.QK_BF16, 64, None, None) == qk.QK_ERR_INVALID_ARG
    assert call(one, 0, qk.QK_BF16, 64, lv, None) == qk.QK_ERR_INVALID_ARG
    assert call(one, 257, qk.QK_BF16, 64, lv, None) == qk.QK_ERR_INVALID_ARG
    assert call(one, 1, 9, 64, lv, None) == qk.QK_ERR_INVALID_ARG
    assert call(one, 1, qk.QK_BF16, 32, lv, None) == qk.QK_ERR_INVALID_ARG
    assert call(arr((X0, 0, C0, A0)), 1, qk.QK_BF16, 64, lv, None) == qk.QK_ERR_INVALID_ARG
    assert call(arr((X0, (1 << 40) + 1, C0, A0)), 1, qk.QK_BF16, 64, lv, None) == qk.QK_ERR_INVALID_ARG
    assert call(arr((None, 4096, C0, A0)), 1, qk.QK_BF16, 64, lv, None) == qk.QK_ERR_INVALID_ARG
    assert call(arr((X0 + 8, 4096, C0, A0)), 1, qk.QK_BF16, 64, lv, None) == qk.QK_ERR_INVALID_ARG   # x alignment
    assert call(arr((X0, 4096, C0 + 2, A0)), 1, qk.QK_BF16, 64, lv, None) == qk.QK_ERR_INVALID_ARG   # codes alignment
    # an output over another task's output or over an input (bf16: 2 bytes per element)
    assert call(arr((X0, 4096, C0, A0), (X1, 4096, C0 + 1024, A1)), 2, qk.QK_BF16, 64, lv, None) == qk.QK_ERR_INVALID_ARG
    assert "overlaps" in qk.qk_last_error()
    assert call(arr((X0, 4096, C0, A0), (X1, 4096, C1, X0 + 8188)), 2, qk.QK_BF16, 64, lv, None) == qk.QK_ERR_INVALID_ARG
    assert call(arr((X0, 4096, C0, C0 + 2044)), 1, qk.QK_BF16, 64, lv, None) == qk.QK_ERR_INVALID_ARG
    bad = (ctypes.c_float * 16)(*([2.0] * 16))
    assert call(one, 1, qk.QK_BF16, 64, bad, None) == qk.QK_ERR_INVALID_ARG
    assert L.qk_quantize_blockwise(FAKE, qk.QK_BF16, (1 << 40) + 1, 64, lv, FAKE, FAKE, None) == qk.QK_ERR_INVALID_ARG


def test_probe_library_exports_and_argument_checks():
    """libqk_probe.so (the HBM ceiling probes bench.py times) exports its three calls
    and refuses bad arguments before launching anything."""
    import os
    path = os.path.join(os.path.dirname(qk.LIB_PATH), "libqk_probe.so")
    if not os.path.exists(path):
        pytest.fail("libqk_probe.so is not built; run python -m bit_blockwise_weight_amd.build")
    P = ctypes.CDLL(path)
    for name in ("qk_probe_read_stream", "qk_probe_mix_stream", "qk_probe_buffer_range", "qk_probe_rowblock_stream"):
        assert hasattr(P, name), name
    P.qk_probe_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p]
    P.qk_probe_mix_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p]
    F = 0x100000
    assert P.qk_probe_read_stream(None, 1024, F, 64, 0, None) == 1
    assert P.qk_probe_read_stream(F, 1000, F, 64, 0, None) == 1            # not a multiple of 16
    assert P.qk_probe_read_stream(F + 8, 1024, F, 64, 0, None) == 1        # misaligned
    assert P.qk_probe_read_stream(F, 1024, F, 0, 0, None) == 1             # no grid
    assert P.qk_probe_mix_stream(None, F, 64, 64, 1, None) == 1
    assert P.qk_probe_mix_stream(F, F + 8, 64, 64, 1, None) == 1           # misaligned dst
    assert P.qk_probe_mix_stream(F, F, 0, 64, 1, None) == 1
    assert P.qk_probe_mix_stream(F, F, 6, 64, 2, None) == 1                # 16-byte stores need n16 % 4 == 0
    P.qk_probe_rowblock_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_void_p, ctypes.c_void_p]
    assert P.qk_probe_rowblock_stream(F, 64, 100, 1, 0, F, None) == 1     # K not a multiple of 64
    assert P.qk_probe_rowblock_stream(F, 64, 128, 3, 0, F, None) == 1     # more splits than steps
    assert P.qk_probe_rowblock_stream(F + 8, 64, 128, 1, 0, F, None) == 1  # misaligned x
    assert P.qk_probe_rowblock_stream(F, 64, 128, 1, 3, F, None) == 1     # no such pattern
