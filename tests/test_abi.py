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
