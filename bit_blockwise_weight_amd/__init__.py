"""Python binding of libqk — blockwise 4-bit (NF4 / FP4) weight quantization on
AMD MI355X (gfx950).

Argument marshalling only: every step runs in the HIP kernels of libqk.so
(built in-tree by ``bit_blockwise_weight_amd.build``); PyTorch provides device
memory and the current stream.  Each function has the name of the C call it
wraps (see include/qk.h) and raises ``QKError`` on a non-zero status.  If the
library is missing or fails to load, the error is raised at the first call,
not at import.
"""

import contextlib
import ctypes
import os

import torch

__all__ = [
    "QKError", "QuantState", "QuantizedWeight", "NF4", "FP4", "CUSTOM", "lib",
    "qk_make_codebook", "qk_quantize_blockwise", "qk_quantize_blockwise_grouped", "qk_double_quant_workspace_size",
    "qk_double_quant",
    "qk_double_quant_grouped_workspace_size", "qk_double_quant_grouped",
    "qk_state_init", "qk_dequantize", "qk_gemv_nf4", "qk_gemv_nf4_grouped", "qk_gemm_nf4_workspace_size", "qk_gemm_nf4", "qk_gemm_nf4_noalloc",
    "qk_gemm_nf4_grouped_workspace_size", "qk_gemm_nf4_grouped", "GemmTask", "qk_dequantize_grouped", "DequantTask", "qk_last_error", "qk_version",
    "qk_backend_info", "quantize",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqk.so")

QK_OK, QK_ERR_INVALID_ARG, QK_ERR_UNSUPPORTED, QK_ERR_BAD_STATE, QK_ERR_HIP, QK_ERR_NO_DEVICE, QK_ERR_WORKSPACE = \
    0, -1, -2, -3, -4, -5, -6
STATUS_NAMES = {0: "QK_OK", -1: "QK_ERR_INVALID_ARG", -2: "QK_ERR_UNSUPPORTED", -3: "QK_ERR_BAD_STATE",
                -4: "QK_ERR_HIP", -5: "QK_ERR_NO_DEVICE", -6: "QK_ERR_WORKSPACE"}
QK_F32, QK_BF16, QK_F16 = 0, 1, 2
NF4, FP4, CUSTOM = 0, 1, 2
QK_STATE_MAGIC = 0x314B5451
QK_STATE_VERSION = 1
QK_DQ_BLOCK = 256

_DTYPE_CODE = {torch.float32: QK_F32, torch.bfloat16: QK_BF16, torch.float16: QK_F16}


class QKError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class QuantState(ctypes.Structure):
    """Mirror of qk_quant_state (include/qk.h)."""
    _fields_ = [
        ("magic", ctypes.c_uint32),
        ("version", ctypes.c_uint32),
        ("struct_bytes", ctypes.c_uint32),
        ("codebook_kind", ctypes.c_int32),
        ("n", ctypes.c_int64),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("blocksize", ctypes.c_int32),
        ("nested", ctypes.c_int32),
        ("dq_blocksize", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("levels", ctypes.c_float * 16),
        ("codes", ctypes.c_void_p),
        ("absmax", ctypes.c_void_p),
        ("q8", ctypes.c_void_p),
        ("dq_scale", ctypes.c_void_p),
        ("dq_mean", ctypes.c_void_p),
    ]


class QuantTask(ctypes.Structure):
    """qk_quant_task."""
    _fields_ = [("x", ctypes.c_void_p), ("n", ctypes.c_int64), ("codes", ctypes.c_void_p),
                ("absmax", ctypes.c_void_p)]


class DqTask(ctypes.Structure):
    """qk_dq_task."""
    _fields_ = [("absmax", ctypes.c_void_p), ("nblocks", ctypes.c_int64), ("q8", ctypes.c_void_p),
                ("scale", ctypes.c_void_p), ("mean", ctypes.c_void_p)]


class GemvTask(ctypes.Structure):
    """Mirror of qk_gemv_task (include/qk.h)."""
    _fields_ = [("x", ctypes.c_void_p), ("st", ctypes.POINTER(QuantState)), ("y", ctypes.c_void_p)]


class DequantTask(ctypes.Structure):
    """Mirror of qk_dequant_task (include/qk.h)."""
    _fields_ = [("st", ctypes.POINTER(QuantState)), ("out", ctypes.c_void_p)]


class GemmTask(ctypes.Structure):
    """Mirror of qk_gemm_task (include/qk.h)."""
    _fields_ = [("X", ctypes.c_void_p), ("M", ctypes.c_int64), ("st", ctypes.POINTER(QuantState)),
                ("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("r", ctypes.c_int32), ("lora_scale", ctypes.c_float),
                ("Y", ctypes.c_void_p)]


_lib = None
_load_error = None


def lib():
    """The loaded libqk (ctypes), with argument types declared.  Raises QKError
    if the library is missing or cannot be loaded."""
    global _lib, _load_error
    if _lib is not None:
        return _lib
    if _load_error is not None:
        raise QKError(QK_ERR_NO_DEVICE, _load_error)
    if not os.path.exists(LIB_PATH):
        _load_error = f"{LIB_PATH} is not built (run: python -m bit_blockwise_weight_amd.build)"
        raise QKError(QK_ERR_NO_DEVICE, _load_error)
    try:
        L = ctypes.CDLL(LIB_PATH)
    except OSError as e:
        _load_error = f"cannot load {LIB_PATH}: {e}"
        raise QKError(QK_ERR_NO_DEVICE, _load_error) from e
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    st_p = ctypes.POINTER(QuantState)
    sigs = {
        "qk_make_codebook": [i32, ctypes.POINTER(ctypes.c_float)],
        "qk_quantize_blockwise": [vp, i32, i64, i32, ctypes.POINTER(ctypes.c_float), vp, vp, vp],
        "qk_quantize_blockwise_grouped": [ctypes.POINTER(QuantTask), i32, i32, i32, ctypes.POINTER(ctypes.c_float), vp],
        "qk_double_quant_workspace_size": [i64, ctypes.POINTER(ctypes.c_size_t)],
        "qk_double_quant": [vp, i64, i32, vp, vp, vp, vp, ctypes.c_size_t, vp],
        "qk_double_quant_grouped_workspace_size": [ctypes.POINTER(DqTask), i32, ctypes.POINTER(ctypes.c_size_t)],
        "qk_double_quant_grouped": [ctypes.POINTER(DqTask), i32, i32, vp, ctypes.c_size_t, vp],
        "qk_state_init": [st_p, i32, ctypes.POINTER(ctypes.c_float), i64, i64, i32, vp, vp, vp, vp, vp],
        "qk_dequantize": [st_p, vp, i32, vp],
        "qk_gemv_nf4": [vp, i32, st_p, vp, vp],
        "qk_gemv_nf4_grouped": [ctypes.POINTER(GemvTask), i32, i32, vp],
        "qk_gemm_nf4_workspace_size": [i64, i32, ctypes.POINTER(ctypes.c_size_t)],
        "qk_dequantize_grouped": [ctypes.POINTER(DequantTask), i32, i32, vp],
        "qk_gemm_nf4_grouped_workspace_size": [ctypes.POINTER(GemmTask), i32, ctypes.POINTER(ctypes.c_size_t)],
        "qk_gemm_nf4_grouped": [ctypes.POINTER(GemmTask), i32, vp, ctypes.c_size_t, vp],
        "qk_gemm_nf4": [vp, i64, st_p, vp, vp, i32, f32, vp, vp, ctypes.c_size_t, vp],
        "qk_gemm_nf4_noalloc": [vp, i64, st_p, vp, vp, i32, f32, vp, vp],
        "qk_lora_merge": [st_p, vp, vp, i32, f32, vp, vp],
        "qk_qlora_backward_workspace_size": [i64, st_p, i32, ctypes.POINTER(ctypes.c_size_t)],
        "qk_qlora_backward": [vp, i64, st_p, vp, vp, vp, i32, f32, vp, vp, vp, vp, ctypes.c_size_t, vp],
        "qk_make_dynamic_map": [i32, ctypes.POINTER(ctypes.c_float)],
        "qk_int8_quantize_rows": [vp, i32, i64, i64, vp, vp, vp, vp],
        "qk_int8_outlier_columns": [vp, i32, i64, i64, f32, vp, vp, vp, vp, vp],
        "qk_int8_matmul": [vp, vp, vp, vp, i64, i64, i64, vp, vp, vp, vp, vp],
        "qk_quantize_blockwise_8bit": [vp, i32, i64, i32, ctypes.POINTER(ctypes.c_float), vp, vp, vp],
        "qk_dequantize_blockwise_8bit": [vp, vp, i64, i32, ctypes.POINTER(ctypes.c_float), vp, i32, vp],
    }
    for name, args in sigs.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int32
    for name in ("qk_last_error", "qk_version", "qk_backend_info"):
        fn = getattr(L, name)
        fn.argtypes = []
        fn.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int):
    if status != QK_OK:
        raise QKError(status, lib().qk_last_error().decode("utf-8", "replace"))


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _on(dev: torch.device):
    """Makes `dev` current for the call (a no-op when it already is)."""
    if dev.index is None or dev.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(dev)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors passed to libqk must be on a HIP device")
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors passed to libqk must be contiguous")


def _levels_arg(levels, count: int = 16):
    if isinstance(levels, ctypes.Array):      # already a float[count]
        if len(levels) != count:
            raise ValueError(f"a level table has {count} entries")
        return levels, torch.tensor(list(levels), dtype=torch.float32)
    lv = torch.as_tensor(levels, dtype=torch.float32).detach().cpu().contiguous()
    if lv.numel() != count:
        raise ValueError(f"a level table has {count} entries")
    return (ctypes.c_float * count)(*lv.tolist()), lv


def qk_last_error() -> str:
    return lib().qk_last_error().decode("utf-8", "replace")


def qk_version() -> str:
    return lib().qk_version().decode()


def qk_backend_info() -> str:
    return lib().qk_backend_info().decode()


def qk_make_codebook(kind: int = NF4) -> torch.Tensor:
    buf = (ctypes.c_float * 16)()
    _check(lib().qk_make_codebook(int(kind), buf))
    return torch.tensor(list(buf), dtype=torch.float32)


def qk_quantize_blockwise(x: torch.Tensor, blocksize: int = 64, levels=None, codes=None, absmax=None):
    """Returns (codes uint8[ceil(n/2)], absmax fp32[ceil(n/B)]) on x's device."""
    _require_cuda(x)
    if x.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported input dtype {x.dtype}")
    n = x.numel()
    if levels is None:
        levels = qk_make_codebook(NF4)
    lv, _ = _levels_arg(levels)
    if codes is None:
        codes = torch.empty((n + 1) // 2, dtype=torch.uint8, device=x.device)
    if absmax is None:
        absmax = torch.empty((n + blocksize - 1) // blocksize, dtype=torch.float32, device=x.device)
    _require_cuda(codes, absmax)
    with _on(x.device):
        _check(lib().qk_quantize_blockwise(_ptr(x), _DTYPE_CODE[x.dtype], n, int(blocksize), lv, _ptr(codes),
                                           _ptr(absmax), ctypes.c_void_p(_stream(x))))
    return codes, absmax


def qk_quantize_blockwise_grouped(xs, blocksize: int = 64, levels=None, codes=None, absmaxes=None):
    """qk_quantize_blockwise of several tensors of one dtype in one launch per run of
    up to 16; returns [(codes, absmax)] in the order of xs."""
    xs = list(xs)
    if not xs:
        raise ValueError("grouped quantization needs at least one tensor")
    dt = xs[0].dtype
    if dt not in _DTYPE_CODE:
        raise ValueError(f"unsupported input dtype {dt}")
    if levels is None:
        levels = qk_make_codebook(NF4)
    lv, _ = _levels_arg(levels)
    arr = (QuantTask * len(xs))()
    outs = []
    for i, x in enumerate(xs):
        if x.dtype != dt:
            raise ValueError(f"task {i}: every tensor needs the dtype of the first ({dt}), got {x.dtype}")
        _require_cuda(x)
        n = x.numel()
        c = codes[i] if codes is not None else torch.empty((n + 1) // 2, dtype=torch.uint8, device=x.device)
        a = absmaxes[i] if absmaxes is not None else torch.empty((n + blocksize - 1) // blocksize,
                                                                 dtype=torch.float32, device=x.device)
        _require_cuda(c, a)
        if c.dtype != torch.uint8 or c.numel() < (n + 1) // 2:
            raise ValueError(f"task {i}: codes must be uint8 with at least {(n + 1) // 2} elements")
        if a.dtype != torch.float32 or a.numel() < (n + blocksize - 1) // blocksize:
            raise ValueError(f"task {i}: absmax must be fp32 with at least {(n + blocksize - 1) // blocksize} elements")
        arr[i].x, arr[i].n, arr[i].codes, arr[i].absmax = _ptr(x), n, _ptr(c), _ptr(a)
        outs.append((c, a))
    with _on(xs[0].device):
        _check(lib().qk_quantize_blockwise_grouped(arr, len(xs), _DTYPE_CODE[dt], int(blocksize), lv,
                                                   ctypes.c_void_p(_stream(xs[0]))))
    return outs


def qk_make_dynamic_map(signed: bool = True) -> torch.Tensor:
    """The 256-level dynamic map (equal-mass quantiles of N(0,1), or of |N(0,1)|
    when unsigned), float32 on the host."""
    buf = (ctypes.c_float * 256)()
    _check(lib().qk_make_dynamic_map(1 if signed else 0, buf))
    return torch.tensor(list(buf), dtype=torch.float32)


def qk_quantize_blockwise_8bit(x: torch.Tensor, blocksize: int = 2048, levels=None, codes=None, absmax=None):
    """Returns (codes uint8[n], absmax fp32[ceil(n/B)]) on x's device; levels
    defaults to the signed dynamic map."""
    _require_cuda(x)
    if x.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported input dtype {x.dtype}")
    n = x.numel()
    if levels is None:
        levels = qk_make_dynamic_map(True)
    lv, _ = _levels_arg(levels, 256)
    if codes is None:
        codes = torch.empty(n, dtype=torch.uint8, device=x.device)
    if absmax is None:
        absmax = torch.empty((n + blocksize - 1) // blocksize, dtype=torch.float32, device=x.device)
    _require_cuda(codes, absmax)
    with _on(x.device):
        _check(lib().qk_quantize_blockwise_8bit(_ptr(x), _DTYPE_CODE[x.dtype], n, int(blocksize), lv, _ptr(codes),
                                                _ptr(absmax), ctypes.c_void_p(_stream(x))))
    return codes, absmax


def qk_dequantize_blockwise_8bit(codes: torch.Tensor, absmax: torch.Tensor, blocksize: int = 2048, levels=None,
                                 dtype=torch.float32, out=None, n=None) -> torch.Tensor:
    """out[k] = RN(levels[codes[k]] * absmax[k // B]) as fp32 or bf16."""
    _require_cuda(codes, absmax)
    n = codes.numel() if n is None else int(n)
    if levels is None:
        levels = qk_make_dynamic_map(True)
    lv, _ = _levels_arg(levels, 256)
    if dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out dtype must be float32 or bfloat16")
    if out is None:
        out = torch.empty(n, dtype=dtype, device=codes.device)
    _require_cuda(out)
    with _on(codes.device):
        _check(lib().qk_dequantize_blockwise_8bit(_ptr(codes), _ptr(absmax), n, int(blocksize), lv, _ptr(out),
                                                  _DTYPE_CODE[out.dtype], ctypes.c_void_p(_stream(codes))))
    return out


def qk_int8_quantize_rows(x: torch.Tensor, skip_cols=None, q=None, absmax=None):
    """Row-wise int8 quantization of a 2-D tensor: (q int8 [rows, cols], absmax fp32 [rows])."""
    _require_cuda(x, skip_cols)
    if x.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported input dtype {x.dtype}")
    rows, cols = x.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    if absmax is None:
        absmax = torch.empty(rows, dtype=torch.float32, device=x.device)
    _require_cuda(q, absmax)
    with _on(x.device):
        _check(lib().qk_int8_quantize_rows(_ptr(x), _DTYPE_CODE[x.dtype], rows, cols, _ptr(skip_cols), _ptr(q),
                                           _ptr(absmax), ctypes.c_void_p(_stream(x))))
    return q, absmax


def qk_int8_outlier_columns(x: torch.Tensor, threshold: float):
    """(colmax fp32 [K], flags uint8 [K], idx int32 [K], count int32 [1]) for x [M, K];
    the first count entries of idx are the outlier columns in increasing order."""
    _require_cuda(x)
    M, K = x.shape
    dev = x.device
    colmax = torch.empty(K, dtype=torch.float32, device=dev)
    flags = torch.empty(K, dtype=torch.uint8, device=dev)
    idx = torch.empty(K, dtype=torch.int32, device=dev)
    count = torch.empty(1, dtype=torch.int32, device=dev)
    with _on(dev):
        _check(lib().qk_int8_outlier_columns(_ptr(x), _DTYPE_CODE[x.dtype], M, K, float(threshold), _ptr(colmax),
                                             _ptr(flags), _ptr(idx), _ptr(count), ctypes.c_void_p(_stream(x))))
    return colmax, flags, idx, count


def qk_int8_matmul(Xq, SX, CB, SCB, X=None, outlier_idx=None, outlier_count=None, Y=None) -> torch.Tensor:
    """fp16 Y [M, N] of the int8 product plus the fp16 outlier product."""
    _require_cuda(Xq, SX, CB, SCB, X, outlier_idx, outlier_count)
    M, K = Xq.shape
    N = CB.shape[0]
    if CB.shape[1] != K:
        raise ValueError(f"Xq {tuple(Xq.shape)} and CB {tuple(CB.shape)} disagree on K")
    if X is not None and X.dtype != torch.float16:
        raise ValueError("X must be fp16")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=Xq.device)
    _require_cuda(Y)
    with _on(Xq.device):
        _check(lib().qk_int8_matmul(_ptr(Xq), _ptr(SX), _ptr(CB), _ptr(SCB), M, N, K, _ptr(X), _ptr(outlier_idx),
                                    _ptr(outlier_count), _ptr(Y), ctypes.c_void_p(_stream(Xq))))
    return Y


class Int8Weight:
    """A weight [N, K] kept as int8 rows (CB) and their absmax (SCB)."""

    def __init__(self, w: torch.Tensor):
        self.CB, self.SCB = qk_int8_quantize_rows(w)
        self.N, self.K = w.shape

    def forward(self, X: torch.Tensor, threshold: float = 6.0) -> torch.Tensor:
        """Y = X W^T by the mixed-precision decomposition (X fp16 [M, K])."""
        X2 = X.reshape(-1, self.K)
        if threshold > 0:
            _, flags, idx, count = qk_int8_outlier_columns(X2, threshold)
            Xq, SX = qk_int8_quantize_rows(X2, flags)
            return qk_int8_matmul(Xq, SX, self.CB, self.SCB, X2, idx, count)
        Xq, SX = qk_int8_quantize_rows(X2)
        return qk_int8_matmul(Xq, SX, self.CB, self.SCB)


def qk_double_quant_workspace_size(nblocks: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().qk_double_quant_workspace_size(int(nblocks), ctypes.byref(out)))
    return int(out.value)


def qk_double_quant(absmax: torch.Tensor, dq_blocksize: int = QK_DQ_BLOCK, q8=None, scale=None, mean=None,
                    workspace=None):
    """Returns (q8 int8[nb], scale fp32[ceil(nb/256)], mean fp32[1])."""
    _require_cuda(absmax)
    nb = absmax.numel()
    dev = absmax.device
    if q8 is None:
        q8 = torch.empty(nb, dtype=torch.int8, device=dev)
    if scale is None:
        scale = torch.empty((nb + dq_blocksize - 1) // max(1, dq_blocksize), dtype=torch.float32, device=dev)
    if mean is None:
        mean = torch.empty(1, dtype=torch.float32, device=dev)
    wsb = qk_double_quant_workspace_size(nb)
    if workspace is None:
        workspace = torch.empty(max(8, wsb), dtype=torch.uint8, device=dev)
    _require_cuda(q8, scale, mean, workspace)
    with _on(dev):
        _check(lib().qk_double_quant(_ptr(absmax), nb, int(dq_blocksize), _ptr(q8), _ptr(scale), _ptr(mean),
                                     _ptr(workspace), workspace.numel(), ctypes.c_void_p(_stream(absmax))))
    return q8, scale, mean


def _dq_tasks(absmaxes, q8s=None, scales=None, means=None, dq_blocksize=QK_DQ_BLOCK):
    absmaxes = list(absmaxes)
    if not absmaxes:
        raise ValueError("double quantization of a group needs at least one absmax array")
    outs = []
    arr = (DqTask * len(absmaxes))()
    for i, a in enumerate(absmaxes):
        if a.dtype != torch.float32:
            raise ValueError(f"task {i}: absmax must be fp32")
        _require_cuda(a)
        nb = a.numel()
        dev = a.device
        q8 = q8s[i] if q8s is not None else torch.empty(nb, dtype=torch.int8, device=dev)
        scale = scales[i] if scales is not None else torch.empty((nb + dq_blocksize - 1) // max(1, dq_blocksize),
                                                                   dtype=torch.float32, device=dev)
        mean = means[i] if means is not None else torch.empty(1, dtype=torch.float32, device=dev)
        _require_cuda(q8, scale, mean)
        arr[i].absmax, arr[i].nblocks = _ptr(a), nb
        arr[i].q8, arr[i].scale, arr[i].mean = _ptr(q8), _ptr(scale), _ptr(mean)
        outs.append((q8, scale, mean))
    return arr, outs


def qk_double_quant_grouped_workspace_size(nblocks) -> int:
    nblocks = [int(n) for n in nblocks]
    arr = (DqTask * len(nblocks))()
    for i, n in enumerate(nblocks):
        arr[i].nblocks = n
    out = ctypes.c_size_t(0)
    _check(lib().qk_double_quant_grouped_workspace_size(arr, len(nblocks), ctypes.byref(out)))
    return int(out.value)


def qk_double_quant_grouped(absmaxes, dq_blocksize: int = QK_DQ_BLOCK, q8s=None, scales=None, means=None,
                            workspace=None):
    """qk_double_quant of several absmax arrays in two launches per run of up to 16;
    returns [(q8, scale, mean)] in the order of absmaxes."""
    arr, outs = _dq_tasks(absmaxes, q8s, scales, means, dq_blocksize)
    first = list(absmaxes)[0]
    dev = first.device
    if workspace is None:
        workspace = torch.empty(max(8, qk_double_quant_grouped_workspace_size([a.numel() for a in absmaxes])),
                                dtype=torch.uint8, device=dev)
    _require_cuda(workspace)
    with _on(dev):
        _check(lib().qk_double_quant_grouped(arr, len(outs), int(dq_blocksize), _ptr(workspace), workspace.numel(),
                                             ctypes.c_void_p(_stream(first))))
    return outs


def qk_state_init(codebook_kind: int, levels, rows: int, cols: int, blocksize: int, codes: torch.Tensor,
                  absmax=None, q8=None, dq_scale=None, dq_mean=None) -> QuantState:
    st = QuantState()
    lv, lv_t = _levels_arg(levels)
    _check(lib().qk_state_init(ctypes.byref(st), int(codebook_kind), lv, int(rows), int(cols), int(blocksize),
                               _ptr(codes), _ptr(absmax), _ptr(q8), _ptr(dq_scale), _ptr(dq_mean)))
    # keep the device buffers alive as long as the descriptor
    st._keep = (codes, absmax, q8, dq_scale, dq_mean, lv_t)
    return st


def qk_dequantize(state: QuantState, out_dtype=torch.bfloat16, out=None, device=None) -> torch.Tensor:
    dev = device if device is not None else state._keep[0].device
    if out is None:
        out = torch.empty(state.n, dtype=out_dtype, device=dev)
    _require_cuda(out)
    with _on(out.device):
        _check(lib().qk_dequantize(ctypes.byref(state), _ptr(out), _DTYPE_CODE[out.dtype],
                                   ctypes.c_void_p(_stream(out))))
    return out


def qk_dequantize_grouped(states, out_dtype=torch.bfloat16, outs=None):
    """qk_dequantize of several states in as few launches as their level tables
    allow; returns the outputs (given in outs, or allocated)."""
    states = list(states)
    if not states:
        raise ValueError("qk_dequantize_grouped needs at least one state")
    if outs is None:
        outs = [torch.empty(st.n, dtype=out_dtype, device=st._keep[0].device) for st in states]
    outs = list(outs)
    if len(outs) != len(states):
        raise ValueError(f"{len(states)} states but {len(outs)} outputs")
    dts = {o.dtype for o in outs}
    if len(dts) != 1 or next(iter(dts)) not in _DTYPE_CODE:
        raise ValueError(f"every output must have one dtype, float32 or bfloat16 (got {dts})")
    arr = (DequantTask * len(states))()
    for i, (st, o) in enumerate(zip(states, outs)):
        if o.numel() != st.n:
            raise ValueError(f"task {i}: out holds {o.numel()} elements, the state {st.n}")
        _require_cuda(o)
        arr[i].st = ctypes.pointer(st)
        arr[i].out = o.data_ptr()
    with _on(outs[0].device):
        _check(lib().qk_dequantize_grouped(arr, len(states), _DTYPE_CODE[outs[0].dtype],
                                           ctypes.c_void_p(_stream(outs[0]))))
    return outs


def _rows_of(t: torch.Tensor, cols: int, name: str) -> torch.Tensor:
    """t viewed as [M, cols]; a ValueError when its size is not a multiple of cols."""
    if t.numel() % cols != 0 or (t.dim() > 0 and t.shape[-1] != cols):
        raise ValueError(f"{name} {tuple(t.shape)} does not end in the weight's {cols} columns")
    return t.reshape(-1, cols)


def _check_out(t: torch.Tensor, shape, dtype, name: str):
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() != shape[0] * shape[1] or (t.dim() == 2 and tuple(t.shape) != tuple(shape)):
        raise ValueError(f"{name} {tuple(t.shape)} does not hold [{shape[0]}, {shape[1]}]")


def qk_gemv_nf4(x: torch.Tensor, state: QuantState, y=None) -> torch.Tensor:
    if x.dtype != torch.bfloat16:
        raise ValueError("qk_gemv_nf4 takes bf16 activations")
    x2 = _rows_of(x, state.cols, "x")
    M = x2.shape[0]
    if y is not None:
        _check_out(y, (M, state.rows), torch.bfloat16, "y")
    _require_cuda(x, y)
    if y is None:
        y = torch.empty((M, state.rows), dtype=torch.bfloat16, device=x.device)
    with _on(x.device):
        _check(lib().qk_gemv_nf4(_ptr(x2), M, ctypes.byref(state), _ptr(y), ctypes.c_void_p(_stream(x))))
    return y


def qk_gemv_nf4_grouped(tasks, ys=None):
    """y_i = x_i deq(W_i)^T for a list of (x_i, state_i) with the same M, in as few
    launches as the states allow.  Returns the list of y_i (bf16 [M, N_i])."""
    tasks = list(tasks)
    if not tasks:
        raise ValueError("qk_gemv_nf4_grouped needs at least one (x, state)")
    M = None
    xs, outs = [], []
    for i, (x, state) in enumerate(tasks):
        if x.dtype != torch.bfloat16:
            raise ValueError(f"task {i}: x must be bf16")
        x2 = _rows_of(x, state.cols, f"task {i}: x")
        if M is None:
            M = x2.shape[0]
        elif x2.shape[0] != M:
            raise ValueError(f"task {i}: every x needs the same number of rows ({M}), got {x2.shape[0]}")
        y = None if ys is None else ys[i]
        if y is not None:
            _check_out(y, (M, state.rows), torch.bfloat16, f"task {i}: y")
        _require_cuda(x, y)
        if y is None:
            y = torch.empty((M, state.rows), dtype=torch.bfloat16, device=x.device)
        xs.append(x2)
        outs.append(y)
    arr = (GemvTask * len(tasks))()
    for i, ((_, state), x2, y) in enumerate(zip(tasks, xs, outs)):
        arr[i].x = x2.data_ptr()
        arr[i].st = ctypes.pointer(state)
        arr[i].y = y.data_ptr()
    dev = xs[0].device
    with _on(dev):
        _check(lib().qk_gemv_nf4_grouped(arr, len(tasks), int(M), ctypes.c_void_p(_stream(xs[0]))))
    return outs


def qk_gemm_nf4_workspace_size(M: int, r: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().qk_gemm_nf4_workspace_size(int(M), int(r), ctypes.byref(out)))
    return int(out.value)


def qk_gemm_nf4(X: torch.Tensor, state: QuantState, A=None, B=None, lora_scale: float = 0.0, Y=None,
                workspace=None) -> torch.Tensor:
    if (A is None) != (B is None):
        raise ValueError("give both LoRA A and B, or neither")
    for name, t in (("X", X), ("A", A), ("B", B)):
        if t is not None and t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bf16, got {t.dtype}")
    X2 = _rows_of(X, state.cols, "X")
    M = X2.shape[0]
    r = 0 if A is None else A.shape[-1]
    if A is not None and (tuple(A.shape) != (state.cols, r) or tuple(B.shape) != (r, state.rows)):
        raise ValueError(f"shapes A {tuple(A.shape)}, B {tuple(B.shape)} do not match W [{state.rows}, {state.cols}]")
    if Y is not None:
        _check_out(Y, (M, state.rows), torch.bfloat16, "Y")
    _require_cuda(X, A, B, Y)
    if Y is None:
        Y = torch.empty((M, state.rows), dtype=torch.bfloat16, device=X.device)
    wsb = qk_gemm_nf4_workspace_size(M, r)
    if workspace is None and wsb > 0:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=X.device)
    _require_cuda(Y, workspace)
    with _on(X.device):
        _check(lib().qk_gemm_nf4(_ptr(X2), M, ctypes.byref(state), _ptr(A), _ptr(B), int(r), float(lora_scale),
                                 _ptr(Y), _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                 ctypes.c_void_p(_stream(X))))
    return Y


def _gemm_tasks(tasks, ys):
    """ctypes array of qk_gemm_task for a list of (X, state, A, B, lora_scale), with
    the outputs (given in ys, or allocated)."""
    tasks = list(tasks)
    if not tasks:
        raise ValueError("a grouped GEMM needs at least one (X, state, A, B, lora_scale)")
    arr = (GemmTask * len(tasks))()
    keep, outs = [], []
    for i, (X, state, A, B, lora_scale) in enumerate(tasks):
        if (A is None) != (B is None):
            raise ValueError(f"task {i}: give both LoRA A and B, or neither")
        for name, t in (("X", X), ("A", A), ("B", B)):
            if t is not None and t.dtype != torch.bfloat16:
                raise ValueError(f"task {i}: {name} must be bf16, got {t.dtype}")
        X2 = _rows_of(X, state.cols, f"task {i}: X")
        M = X2.shape[0]
        r = 0 if A is None else A.shape[-1]
        if A is not None and (tuple(A.shape) != (state.cols, r) or tuple(B.shape) != (r, state.rows)):
            raise ValueError(f"task {i}: shapes A {tuple(A.shape)}, B {tuple(B.shape)} do not match "
                             f"W [{state.rows}, {state.cols}]")
        Y = None if ys is None else ys[i]
        if Y is not None:
            _check_out(Y, (M, state.rows), torch.bfloat16, f"task {i}: Y")
        _require_cuda(X, A, B, Y)
        if Y is None:
            Y = torch.empty((M, state.rows), dtype=torch.bfloat16, device=X.device)
        arr[i].X = X2.data_ptr()
        arr[i].M = M
        arr[i].st = ctypes.pointer(state)
        arr[i].A = _ptr(A)
        arr[i].B = _ptr(B)
        arr[i].r = int(r)
        arr[i].lora_scale = float(lora_scale)
        arr[i].Y = Y.data_ptr()
        keep.append(X2)
        outs.append(Y)
    return arr, keep, outs


def qk_gemm_nf4_grouped_workspace_size(tasks) -> int:
    """Workspace bytes of qk_gemm_nf4_grouped for a list of (X, state, A, B, lora_scale)."""
    arr, _, _ = _gemm_tasks(tasks, None)
    out = ctypes.c_size_t(0)
    _check(lib().qk_gemm_nf4_grouped_workspace_size(arr, len(arr), ctypes.byref(out)))
    return int(out.value)


def qk_gemm_nf4_grouped(tasks, ys=None, workspace=None):
    """Y_i = X_i deq(W_i)^T + s_i (X_i A_i) B_i for a list of (X_i, state_i, A_i, B_i, s_i),
    in as few launches as their shapes allow; each Y_i equals what qk_gemm_nf4 of that
    task alone writes.  Returns the list of Y_i."""
    arr, keep, outs = _gemm_tasks(tasks, ys)
    out = ctypes.c_size_t(0)
    _check(lib().qk_gemm_nf4_grouped_workspace_size(arr, len(arr), ctypes.byref(out)))
    wsb = int(out.value)
    dev = keep[0].device
    if workspace is None and wsb > 0:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    _require_cuda(workspace)
    with _on(dev):
        _check(lib().qk_gemm_nf4_grouped(arr, len(arr), _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                         ctypes.c_void_p(_stream(keep[0]))))
    return outs


def qk_gemm_nf4_noalloc(X: torch.Tensor, state: QuantState, A=None, B=None, lora_scale: float = 0.0,
                        Y=None) -> torch.Tensor:
    """qk_gemm_nf4 without a workspace: the LoRA partials use the library's static
    device scratch (M * 16 * ceil(r / 16) <= 262144).  Calls that overlap on one
    device race."""
    if (A is None) != (B is None):
        raise ValueError("give both LoRA A and B, or neither")
    for name, t in (("X", X), ("A", A), ("B", B)):
        if t is not None and t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bf16, got {t.dtype}")
    X2 = _rows_of(X, state.cols, "X")
    M = X2.shape[0]
    r = 0 if A is None else A.shape[-1]
    if A is not None and (tuple(A.shape) != (state.cols, r) or tuple(B.shape) != (r, state.rows)):
        raise ValueError(f"shapes A {tuple(A.shape)}, B {tuple(B.shape)} do not match W [{state.rows}, {state.cols}]")
    if Y is not None:
        _check_out(Y, (M, state.rows), torch.bfloat16, "Y")
    _require_cuda(X, A, B, Y)
    if Y is None:
        Y = torch.empty((M, state.rows), dtype=torch.bfloat16, device=X.device)
    with _on(X.device):
        _check(lib().qk_gemm_nf4_noalloc(_ptr(X2), M, ctypes.byref(state), _ptr(A), _ptr(B), int(r),
                                         float(lora_scale), _ptr(Y), ctypes.c_void_p(_stream(X))))
    return Y


def qk_lora_merge(state: QuantState, A: torch.Tensor, B: torch.Tensor, lora_scale: float, out=None,
                  device=None) -> torch.Tensor:
    """bf16 W_new [N, K] = bf16(D + s * (A B)^T) of the quantized weight `state`,
    A [K, r], B [r, N] (bf16)."""
    _require_cuda(A, B)
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise ValueError("A and B must be bf16")
    K, r = A.shape
    if B.shape[0] != r or B.shape[1] != state.rows or K != state.cols:
        raise ValueError(f"shapes A {tuple(A.shape)}, B {tuple(B.shape)} do not match W [{state.rows}, {state.cols}]")
    dev = A.device if device is None else device
    if out is None:
        out = torch.empty((state.rows, state.cols), dtype=torch.bfloat16, device=dev)
    _require_cuda(out)
    with _on(out.device):
        _check(lib().qk_lora_merge(ctypes.byref(state), _ptr(A), _ptr(B), int(r), float(lora_scale), _ptr(out),
                                   ctypes.c_void_p(_stream(out))))
    return out


def qk_qlora_backward_workspace_size(M: int, state: QuantState, r: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().qk_qlora_backward_workspace_size(int(M), ctypes.byref(state), int(r), ctypes.byref(out)))
    return int(out.value)


def qk_qlora_backward(dY: torch.Tensor, state: QuantState, X=None, A=None, B=None, lora_scale: float = 0.0,
                      dX=None, dA=None, dB=None, workspace=None):
    """Gradients of Y = X deq(W)^T + s (X A) B for the upstream gradient dY [M, N]
    (bf16): dX bf16 [M, K] and, with an adapter (A [K, r], B [r, N], X [M, K],
    all bf16), dA fp32 [K, r] and dB fp32 [r, N].  Returns (dX, dA, dB)."""
    _require_cuda(dY, X, A, B)
    if (A is None) != (B is None):
        raise ValueError("give both LoRA A and B, or neither")
    for name, t in (("dY", dY), ("X", X), ("A", A), ("B", B)):
        if t is not None and t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bf16")
    dY2 = dY.reshape(-1, state.rows)
    M = dY2.shape[0]
    dev = dY.device
    r = 0
    X2 = None
    if A is not None:
        if X is None:
            raise ValueError("the adapter gradients need X")
        r = A.shape[1]
        X2 = X.reshape(-1, state.cols)
        if X2.shape[0] != M or tuple(A.shape) != (state.cols, r) or tuple(B.shape) != (r, state.rows):
            raise ValueError(f"shapes X {tuple(X.shape)}, A {tuple(A.shape)}, B {tuple(B.shape)} do not match "
                             f"dY {tuple(dY.shape)} and W [{state.rows}, {state.cols}]")
        if dA is None:
            dA = torch.empty((state.cols, r), dtype=torch.float32, device=dev)
        if dB is None:
            dB = torch.empty((r, state.rows), dtype=torch.float32, device=dev)
    if dX is None:
        dX = torch.empty((M, state.cols), dtype=torch.bfloat16, device=dev)
    need = qk_qlora_backward_workspace_size(M, state, r)
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _require_cuda(dX, dA, dB, workspace)
    with _on(dev):
        _check(lib().qk_qlora_backward(_ptr(dY2), M, ctypes.byref(state), _ptr(X2), _ptr(A), _ptr(B), int(r),
                                       float(lora_scale), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(workspace),
                                       0 if workspace is None else workspace.numel(), ctypes.c_void_p(_stream(dY))))
    return dX, dA, dB


class QuantizedWeight:
    """A weight W[N, K] quantized on the device: its buffers and its descriptor."""

    def __init__(self, state: QuantState, codes, absmax=None, q8=None, scale=None, mean=None):
        self.state = state
        self.codes, self.absmax, self.q8, self.scale, self.mean = codes, absmax, q8, scale, mean

    @property
    def shape(self):
        return (self.state.rows, self.state.cols)

    def dequantize(self, out_dtype=torch.bfloat16, out=None):
        return qk_dequantize(self.state, out_dtype, out, device=self.codes.device)

    def gemv(self, x, y=None):
        return qk_gemv_nf4(x, self.state, y)

    def gemm(self, X, A=None, B=None, lora_scale=0.0, Y=None, workspace=None):
        return qk_gemm_nf4(X, self.state, A, B, lora_scale, Y, workspace)

    def backward(self, dY, X=None, A=None, B=None, lora_scale=0.0, workspace=None):
        return qk_qlora_backward(dY, self.state, X, A, B, lora_scale, workspace=workspace)

    def merge_lora(self, A, B, lora_scale, double_quant=True):
        """Merges the adapter into the weight and quantizes the merged bf16 weight
        again with the same codebook and block size.  Returns (W_new, QuantizedWeight)."""
        w_new = qk_lora_merge(self.state, A, B, lora_scale)
        levels = torch.tensor(list(self.state.levels), dtype=torch.float32)
        return w_new, quantize(w_new, self.state.blocksize, self.state.codebook_kind, double_quant, levels)


def quantize(w: torch.Tensor, blocksize: int = 64, kind: int = NF4, double_quant: bool = True,
             levels=None) -> QuantizedWeight:
    """qk_quantize_blockwise (+ qk_double_quant) of a 2-D weight and the descriptor."""
    if w.dim() != 2:
        raise ValueError("quantize expects a 2-D weight [N, K]")
    if levels is None:
        levels = qk_make_codebook(kind)
    codes, absmax = qk_quantize_blockwise(w, blocksize, levels)
    if double_quant:
        q8, scale, mean = qk_double_quant(absmax)
        st = qk_state_init(kind, levels, w.shape[0], w.shape[1], blocksize, codes, None, q8, scale, mean)
        return QuantizedWeight(st, codes, None, q8, scale, mean)
    st = qk_state_init(kind, levels, w.shape[0], w.shape[1], blocksize, codes, absmax)
    return QuantizedWeight(st, codes, absmax)
