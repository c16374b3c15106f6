"""Python binding of libllmint8 (LLM.int8() linear layer on MI355X / gfx950).

Argument marshalling only: every step of the forward runs in the library's HIP
kernels. Function names are those of the C ABI (include/llmint8.h). PyTorch
provides device memory and the current stream; nothing here computes on the
data, and there is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "LLMINT8_PATH_AUTO", "LLMINT8_PATH_GEMM", "LLMINT8_PATH_GEMV", "LLMINT8_PATH_GEMM_TILES",
    "Llmint8Error",
    "library_path", "load_library", "llmint8_quantize_weight", "llmint8_workspace_bytes",
    "llmint8_workspace_bytes_path", "shared_workspace_bytes",
    "llmint8_linear", "llmint8_linear_debug", "llmint8_linear_timed", "llmint8_gemv_max_rows",
    "llmint8_status_string", "llmint8_backward_workspace_bytes", "llmint8_dequantize_weight_t",
    "llmint8_linear_backward_input", "llmint8_linear_backward_input_timed", "Int8Linear",
    "LLMINT8_DTYPE_F16", "LLMINT8_DTYPE_F32", "llmint8_quantize_blockwise",
    "llmint8_dequantize_blockwise", "EXPORTED_SYMBOLS", "LLMINT8_DTYPE_BF16",
    "llmint8_quantize_weight_ex", "llmint8_linear_ex", "llmint8_linear_debug_ex",
    "LLMINT8_QUANT_NF4", "LLMINT8_QUANT_FP4", "llmint8_code_book_4bit", "llmint8_quantize_4bit",
    "llmint8_dequantize_4bit", "llmint8_linear_4bit", "Linear4bit", "llmint8_linear_timed_ex",
    "llmint8_linear_backward_input_ex", "llmint8_dequantize_weight_t_ex",
    "llmint8_gemm_tile", "llmint8_linear_noalloc", "llmint8_noalloc_scratch_bytes",
]

LLMINT8_PATH_AUTO = 0
LLMINT8_PATH_GEMM = 1
LLMINT8_PATH_GEMV = 2
# the GEMM route with a fixed output tile (N x T), for tests and tuning
LLMINT8_PATH_GEMM_TILES = {"256x256": 16, "192x256": 17, "256x128": 18, "128x128": 19, "352x256": 20}
LLMINT8_DTYPE_F16 = 0
LLMINT8_DTYPE_F32 = 1
LLMINT8_DTYPE_BF16 = 2
LLMINT8_QUANT_NF4 = 0
LLMINT8_QUANT_FP4 = 1

EXPORTED_SYMBOLS = (
    "llmint8_quantize_weight", "llmint8_workspace_bytes", "llmint8_workspace_bytes_path",
    "llmint8_linear",
    "llmint8_linear_debug", "llmint8_linear_timed", "llmint8_gemv_max_rows",
    "llmint8_status_string", "llmint8_last_hip_error", "llmint8_backward_workspace_bytes",
    "llmint8_dequantize_weight_t", "llmint8_linear_backward_input",
    "llmint8_linear_backward_input_timed", "llmint8_quantize_blockwise",
    "llmint8_dequantize_blockwise", "llmint8_quantize_weight_ex", "llmint8_linear_ex",
    "llmint8_linear_debug_ex", "llmint8_code_book_4bit", "llmint8_quantize_4bit",
    "llmint8_dequantize_4bit", "llmint8_linear_4bit", "llmint8_linear_timed_ex",
    "llmint8_linear_backward_input_ex", "llmint8_dequantize_weight_t_ex",
    "llmint8_gemm_tile", "llmint8_linear_noalloc", "llmint8_noalloc_scratch_bytes",
)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64


class Llmint8Error(RuntimeError):
    def __init__(self, status: int, where: str, hip: int = 0):
        self.status = status
        msg = f"{where}: {_status_text(status)} (status {status}"
        if hip:
            msg += f", hipError {hip}"
        super().__init__(msg + ")")


def library_path() -> str:
    return os.path.join(_HERE, "libllmint8.so")


def load_library():
    """Load the built library (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with mixed_precision_int8_amd/build.py "
                           "(or __graft_entry__.build()) before use")
    lib = ctypes.CDLL(path)
    lib.llmint8_quantize_weight.argtypes = [_vp, _i64, _i64, _vp, _vp, _vp]
    lib.llmint8_quantize_weight.restype = ctypes.c_int
    lib.llmint8_workspace_bytes.argtypes = [_i64, _i64, _i64]
    lib.llmint8_workspace_bytes.restype = ctypes.c_size_t
    lib.llmint8_workspace_bytes_path.argtypes = [_i64, _i64, _i64, ctypes.c_int]
    lib.llmint8_workspace_bytes_path.restype = ctypes.c_size_t
    lin = [_vp, _i64, _i64, _vp, _vp, _i64, ctypes.c_float, _vp, _vp, ctypes.c_size_t, _vp]
    lib.llmint8_linear.argtypes = lin
    lib.llmint8_linear.restype = ctypes.c_int
    lib.llmint8_linear_debug.argtypes = lin + [ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.llmint8_linear_debug.restype = ctypes.c_int
    lib.llmint8_linear_timed.argtypes = lin + [ctypes.c_int, ctypes.POINTER(_vp), ctypes.c_int,
                                               ctypes.POINTER(ctypes.c_int)]
    lib.llmint8_linear_timed.restype = ctypes.c_int
    lib.llmint8_backward_workspace_bytes.argtypes = [_i64, _i64, _i64]
    lib.llmint8_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.llmint8_dequantize_weight_t.argtypes = [_vp, _vp, _i64, _i64, _vp, _vp]
    lib.llmint8_dequantize_weight_t.restype = ctypes.c_int
    bwd = [_vp, _i64, _i64, _vp, _vp, _i64, _vp, _vp, ctypes.c_size_t, _vp]
    lib.llmint8_linear_backward_input.argtypes = bwd
    lib.llmint8_linear_backward_input.restype = ctypes.c_int
    lib.llmint8_linear_backward_input_timed.argtypes = bwd + [ctypes.POINTER(_vp), ctypes.c_int,
                                                              ctypes.POINTER(ctypes.c_int)]
    lib.llmint8_linear_backward_input_timed.restype = ctypes.c_int
    lib.llmint8_linear_backward_input_ex.argtypes = [_vp, ctypes.c_int, _i64, _i64, _vp, _vp, _i64,
                                                     _vp, _vp, ctypes.c_size_t, _vp]
    lib.llmint8_linear_backward_input_ex.restype = ctypes.c_int
    lib.llmint8_dequantize_weight_t_ex.argtypes = [_vp, _vp, _i64, _i64, _vp, ctypes.c_int, _vp]
    lib.llmint8_dequantize_weight_t_ex.restype = ctypes.c_int
    lib.llmint8_quantize_blockwise.argtypes = [_vp, ctypes.c_int, _i64, _i64, _vp, _vp, _vp]
    lib.llmint8_quantize_blockwise.restype = ctypes.c_int
    lib.llmint8_dequantize_blockwise.argtypes = [_vp, _vp, _i64, _i64, _vp, ctypes.c_int, _vp]
    lib.llmint8_dequantize_blockwise.restype = ctypes.c_int
    lib.llmint8_quantize_weight_ex.argtypes = [_vp, ctypes.c_int, _i64, _i64, _vp, _vp, _vp]
    lib.llmint8_quantize_weight_ex.restype = ctypes.c_int
    lin_ex = [_vp, ctypes.c_int, _i64, _i64, _vp, _vp, _i64, ctypes.c_float, _vp, _vp, _vp,
              ctypes.c_size_t, _vp]
    lib.llmint8_linear_ex.argtypes = lin_ex
    lib.llmint8_linear_ex.restype = ctypes.c_int
    lib.llmint8_linear_debug_ex.argtypes = lin_ex + [ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.llmint8_linear_timed_ex.argtypes = lin_ex + [ctypes.c_int, ctypes.POINTER(_vp), ctypes.c_int,
                                                     ctypes.POINTER(ctypes.c_int)]
    lib.llmint8_linear_timed_ex.restype = ctypes.c_int
    lib.llmint8_linear_debug_ex.restype = ctypes.c_int
    lib.llmint8_code_book_4bit.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_float)]
    lib.llmint8_code_book_4bit.restype = ctypes.c_int
    lib.llmint8_quantize_4bit.argtypes = [_vp, ctypes.c_int, _i64, _i64, ctypes.c_int, _vp, _vp, _vp]
    lib.llmint8_quantize_4bit.restype = ctypes.c_int
    lib.llmint8_dequantize_4bit.argtypes = [_vp, _vp, _i64, _i64, ctypes.c_int, _vp, ctypes.c_int, _vp]
    lib.llmint8_dequantize_4bit.restype = ctypes.c_int
    lib.llmint8_linear_4bit.argtypes = [_vp, ctypes.c_int, _i64, _i64, _vp, _vp, _i64, ctypes.c_int,
                                        _i64, _vp, _vp, _vp]
    lib.llmint8_linear_4bit.restype = ctypes.c_int
    lib.llmint8_linear_noalloc.argtypes = [_vp, ctypes.c_int, _i64, _i64, _vp, _vp, _i64,
                                           ctypes.c_float, _vp, _vp, _vp]
    lib.llmint8_linear_noalloc.restype = ctypes.c_int
    lib.llmint8_noalloc_scratch_bytes.argtypes = []
    lib.llmint8_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.llmint8_gemm_tile.argtypes = [_i64, _i64]
    lib.llmint8_gemm_tile.restype = ctypes.c_int
    lib.llmint8_gemv_max_rows.argtypes = [_i64]
    lib.llmint8_gemv_max_rows.restype = ctypes.c_int
    lib.llmint8_status_string.argtypes = [ctypes.c_int]
    lib.llmint8_status_string.restype = ctypes.c_char_p
    lib.llmint8_last_hip_error.argtypes = []
    lib.llmint8_last_hip_error.restype = ctypes.c_int
    _LIB = lib
    return lib


def _status_text(status: int) -> str:
    try:
        return load_library().llmint8_status_string(status).decode()
    except Exception:  # noqa: BLE001 - message only
        return "error"


def _check(status: int, where: str):
    if status != 0:
        hip = load_library().llmint8_last_hip_error() if status == -4 else 0
        raise Llmint8Error(status, where, hip)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, dtype, shape, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected contiguous CUDA {dtype} {tuple(shape)}, got "
                         f"{t.dtype} {tuple(t.shape)} on {t.device}")


def llmint8_workspace_bytes(T: int, K: int, N: int) -> int:
    return int(load_library().llmint8_workspace_bytes(T, K, N))


def llmint8_workspace_bytes_path(T: int, K: int, N: int, path: int = LLMINT8_PATH_AUTO) -> int:
    return int(load_library().llmint8_workspace_bytes_path(T, K, N, int(path)))


def llmint8_gemm_tile(T: int, N: int) -> str:
    """Name ("352x256", ...) of the tile the GEMM route picks for T rows and N outputs."""
    code = int(load_library().llmint8_gemm_tile(T, N))
    if code < 0:
        raise Llmint8Error(code, "llmint8_gemm_tile", 0)
    return {v: k for k, v in LLMINT8_PATH_GEMM_TILES.items()}[code]


def llmint8_gemv_max_rows(K: int) -> int:
    return int(load_library().llmint8_gemv_max_rows(K))


def llmint8_status_string(status: int) -> str:
    return _status_text(status)


def llmint8_quantize_weight(W, Wq=None, sW=None, stream=None):
    """W fp16 [N, K] (CUDA) -> (Wq int8 [N, K], sW fp32 [N])."""
    import torch
    lib = load_library()
    N, K = W.shape
    _need(W, torch.float16, (N, K), "W")
    if Wq is None:
        Wq = torch.empty((N, K), dtype=torch.int8, device=W.device)
    if sW is None:
        sW = torch.empty((N,), dtype=torch.float32, device=W.device)
    _need(Wq, torch.int8, (N, K), "Wq")
    _need(sW, torch.float32, (N,), "sW")
    _check(lib.llmint8_quantize_weight(_ptr(W), N, K, _ptr(Wq), _ptr(sW), _stream(stream, W.device)),
           "llmint8_quantize_weight")
    return Wq, sW


def _act_dtype(dtype):
    import torch
    if dtype == torch.float16:
        return LLMINT8_DTYPE_F16
    if dtype == torch.bfloat16:
        return LLMINT8_DTYPE_BF16
    raise ValueError(f"activations: fp16 or bf16 only, got {dtype}")


def llmint8_quantize_weight_ex(W, Wq=None, sW=None, stream=None):
    """W fp16 or bf16 [N, K] (CUDA) -> (Wq int8 [N, K], sW fp32 [N])."""
    import torch
    lib = load_library()
    N, K = W.shape
    code = _act_dtype(W.dtype)
    _need(W, W.dtype, (N, K), "W")
    if Wq is None:
        Wq = torch.empty((N, K), dtype=torch.int8, device=W.device)
    if sW is None:
        sW = torch.empty((N,), dtype=torch.float32, device=W.device)
    _need(Wq, torch.int8, (N, K), "Wq")
    _need(sW, torch.float32, (N,), "sW")
    _check(lib.llmint8_quantize_weight_ex(_ptr(W), code, N, K, _ptr(Wq), _ptr(sW),
                                          _stream(stream, W.device)),
           "llmint8_quantize_weight_ex")
    return Wq, sW


def _workspace(T, K, N, device, workspace, path=LLMINT8_PATH_AUTO):
    """The caller's workspace, or a new one of the size the route needs (None when the
    route needs none: the fused decode kernel keeps everything in LDS)."""
    import torch
    if workspace is None:
        need = llmint8_workspace_bytes_path(T, K, N, path)
        if need > 0:
            workspace = torch.empty((need,), dtype=torch.uint8, device=device)
    return workspace


def _ws_bytes(ws):
    return 0 if ws is None else ws.numel() * ws.element_size()


def _linear_args(X, Wq, sW, threshold, Y, workspace, dtype=None, bias=None, path=LLMINT8_PATH_AUTO):
    import torch
    T, K = X.shape
    N = Wq.shape[0]
    dtype = dtype or torch.float16
    _need(X, dtype, (T, K), "X")
    _need(Wq, torch.int8, (N, K), "Wq")
    _need(sW, torch.float32, (N,), "sW")
    if bias is not None:
        _need(bias, dtype, (N,), "bias")
    if Y is None:
        Y = torch.empty((T, N), dtype=dtype, device=X.device)
    _need(Y, dtype, (T, N), "Y")
    workspace = _workspace(T, K, N, X.device, workspace, path)
    thr = float(threshold)
    if thr == math.inf:
        thr = math.inf
    return T, K, N, Y, workspace, thr


def llmint8_linear(X, Wq, sW, threshold: float = 6.0, Y=None, workspace=None, stream=None):
    """Y fp16 [T, N] = LLM.int8() forward of X fp16 [T, K] with (Wq, sW)."""
    lib = load_library()
    T, K, N, Y, ws, thr = _linear_args(X, Wq, sW, threshold, Y, workspace)
    _check(lib.llmint8_linear(_ptr(X), T, K, _ptr(Wq), _ptr(sW), N, thr, _ptr(Y), _ptr(ws),
                              _ws_bytes(ws), _stream(stream, X.device)),
           "llmint8_linear")
    return Y


def llmint8_linear_ex(X, Wq, sW, threshold: float = 6.0, bias=None, Y=None, workspace=None,
                      stream=None):
    """Y [T, N] = LLM.int8() forward of X [T, K] (fp16 or bf16; Y and the optional
    bias [N] take the type of X) with (Wq, sW)."""
    lib = load_library()
    code = _act_dtype(X.dtype)
    T, K, N, Y, ws, thr = _linear_args(X, Wq, sW, threshold, Y, workspace, X.dtype, bias)
    _check(lib.llmint8_linear_ex(_ptr(X), code, T, K, _ptr(Wq), _ptr(sW), N, thr, _ptr(bias),
                                 _ptr(Y), _ptr(ws), _ws_bytes(ws),
                                 _stream(stream, X.device)),
           "llmint8_linear_ex")
    return Y


def llmint8_linear_noalloc(X, Wq, sW, threshold: float = 6.0, bias=None, Y=None, stream=None):
    """llmint8_linear_ex on the library's static scratch: no workspace and no allocation
    inside the call (pass ``Y`` to allocate nothing at all). For callers that cannot
    allocate; calls that overlap in time on one GPU race on the shared scratch."""
    import torch
    lib = load_library()
    code = _act_dtype(X.dtype)
    T, K = X.shape
    N = Wq.shape[0]
    _need(X, X.dtype, (T, K), "X")
    _need(Wq, torch.int8, (N, K), "Wq")
    _need(sW, torch.float32, (N,), "sW")
    if bias is not None:
        _need(bias, X.dtype, (N,), "bias")
    if Y is None:
        Y = torch.empty((T, N), dtype=X.dtype, device=X.device)
    _need(Y, X.dtype, (T, N), "Y")
    _check(lib.llmint8_linear_noalloc(_ptr(X), code, T, K, _ptr(Wq), _ptr(sW), N, float(threshold),
                                      _ptr(bias), _ptr(Y), _stream(stream, X.device)),
           "llmint8_linear_noalloc")
    return Y


def llmint8_noalloc_scratch_bytes() -> int:
    return int(load_library().llmint8_noalloc_scratch_bytes())


def llmint8_linear_timed_ex(X, Wq, sW, threshold, Y, workspace, events, bias=None,
                            path=LLMINT8_PATH_AUTO, stream=None):
    """llmint8_linear_ex recording ``events`` (created torch.cuda.Event) around each kernel.

    Returns the number of kernels launched.
    """
    lib = load_library()
    code = _act_dtype(X.dtype)
    T, K, N, Y, ws, thr = _linear_args(X, Wq, sW, threshold, Y, workspace, X.dtype, bias, path)
    handles = (_vp * len(events))(*[ctypes.c_void_p(e.cuda_event) for e in events])
    nk = ctypes.c_int(0)
    _check(lib.llmint8_linear_timed_ex(_ptr(X), code, T, K, _ptr(Wq), _ptr(sW), N, thr, _ptr(bias),
                                       _ptr(Y), _ptr(ws), _ws_bytes(ws),
                                       _stream(stream, X.device), int(path), handles, len(events),
                                       ctypes.byref(nk)),
           "llmint8_linear_timed_ex")
    return nk.value


def _debug_outputs(T, K, N, dev, want_C):
    import torch
    KW = (K + 31) // 32
    return {
        "bitmap": torch.zeros((KW,), dtype=torch.int32, device=dev),
        "idx": torch.full((K,), -1, dtype=torch.int32, device=dev),
        "count": torch.full((1,), -1, dtype=torch.int32, device=dev),
        "Xq": torch.zeros((T, K), dtype=torch.int8, device=dev),
        "aX": torch.zeros((T,), dtype=torch.float32, device=dev),
        "C": torch.zeros((T, N), dtype=torch.int32, device=dev) if want_C else None,
    }


def llmint8_linear_debug_ex(X, Wq, sW, threshold: float = 6.0, bias=None,
                            path: int = LLMINT8_PATH_AUTO, Y=None, workspace=None, stream=None,
                            want_C: bool = True):
    """llmint8_linear_ex plus the intermediates of the same kernels: dict of tensors."""
    lib = load_library()
    code = _act_dtype(X.dtype)
    T, K, N, Y, ws, thr = _linear_args(X, Wq, sW, threshold, Y, workspace, X.dtype, bias, path)
    dev = X.device
    out = _debug_outputs(T, K, N, dev, want_C)
    _check(lib.llmint8_linear_debug_ex(_ptr(X), code, T, K, _ptr(Wq), _ptr(sW), N, thr, _ptr(bias),
                                       _ptr(Y), _ptr(ws), _ws_bytes(ws),
                                       _stream(stream, dev), int(path), _ptr(out["bitmap"]),
                                       _ptr(out["idx"]), _ptr(out["count"]), _ptr(out["Xq"]),
                                       _ptr(out["aX"]), _ptr(out["C"])),
           "llmint8_linear_debug_ex")
    out["Y"] = Y
    return out


def llmint8_linear_debug(X, Wq, sW, threshold: float = 6.0, path: int = LLMINT8_PATH_AUTO,
                         Y=None, workspace=None, stream=None, want_C: bool = True):
    """Forward plus the intermediates of the same kernels: dict of tensors."""
    lib = load_library()
    T, K, N, Y, ws, thr = _linear_args(X, Wq, sW, threshold, Y, workspace, path=path)
    dev = X.device
    out = _debug_outputs(T, K, N, dev, want_C)
    _check(lib.llmint8_linear_debug(_ptr(X), T, K, _ptr(Wq), _ptr(sW), N, thr, _ptr(Y), _ptr(ws),
                                    _ws_bytes(ws), _stream(stream, dev), int(path),
                                    _ptr(out["bitmap"]), _ptr(out["idx"]), _ptr(out["count"]),
                                    _ptr(out["Xq"]), _ptr(out["aX"]), _ptr(out["C"])),
           "llmint8_linear_debug")
    out["Y"] = Y
    return out


def llmint8_linear_timed(X, Wq, sW, threshold, Y, workspace, events, path=LLMINT8_PATH_AUTO,
                         stream=None):
    """Forward that records ``events`` (torch.cuda.Event, created) around each kernel.

    Returns the number of kernels launched.
    """
    lib = load_library()
    T, K, N, Y, ws, thr = _linear_args(X, Wq, sW, threshold, Y, workspace, path=path)
    handles = (_vp * len(events))(*[ctypes.c_void_p(e.cuda_event) for e in events])
    nk = ctypes.c_int(0)
    _check(lib.llmint8_linear_timed(_ptr(X), T, K, _ptr(Wq), _ptr(sW), N, thr, _ptr(Y), _ptr(ws),
                                    _ws_bytes(ws), _stream(stream, X.device),
                                    int(path), handles, len(events), ctypes.byref(nk)),
           "llmint8_linear_timed")
    return nk.value


def llmint8_backward_workspace_bytes(T: int, K: int, N: int) -> int:
    return int(load_library().llmint8_backward_workspace_bytes(T, K, N))


def llmint8_dequantize_weight_t(Wq, sW, WdT=None, stream=None):
    """(Wq int8 [N, K], sW fp32 [N]) -> WdT fp16 [K, N], the weight dequantized and transposed."""
    import torch
    lib = load_library()
    N, K = Wq.shape
    _need(Wq, torch.int8, (N, K), "Wq")
    _need(sW, torch.float32, (N,), "sW")
    if WdT is None:
        WdT = torch.empty((K, N), dtype=torch.float16, device=Wq.device)
    _need(WdT, torch.float16, (K, N), "WdT")
    _check(lib.llmint8_dequantize_weight_t(_ptr(Wq), _ptr(sW), N, K, _ptr(WdT),
                                           _stream(stream, Wq.device)),
           "llmint8_dequantize_weight_t")
    return WdT


def _backward_args(dY, Wq, sW, dX, workspace, dtype=None):
    import torch
    T, N = dY.shape
    K = Wq.shape[1]
    dtype = dtype or torch.float16
    _need(dY, dtype, (T, N), "dY")
    _need(Wq, torch.int8, (N, K), "Wq")
    _need(sW, torch.float32, (N,), "sW")
    if dX is None:
        dX = torch.empty((T, K), dtype=dtype, device=dY.device)
    _need(dX, dtype, (T, K), "dX")
    if workspace is None:
        need = llmint8_backward_workspace_bytes(T, K, N)   # 0: the weight is dequantized on the fly
        if need > 0:
            workspace = torch.empty((need,), dtype=torch.uint8, device=dY.device)
    return T, K, N, dX, workspace


def llmint8_linear_backward_input(dY, Wq, sW, dX=None, workspace=None, stream=None):
    """dX fp16 [T, K] = dY fp16 [T, N] . Wdeq, the input gradient of the frozen layer."""
    lib = load_library()
    T, K, N, dX, ws = _backward_args(dY, Wq, sW, dX, workspace)
    _check(lib.llmint8_linear_backward_input(_ptr(dY), T, K, _ptr(Wq), _ptr(sW), N, _ptr(dX),
                                             _ptr(ws), _ws_bytes(ws),
                                             _stream(stream, dY.device)),
           "llmint8_linear_backward_input")
    return dX


def llmint8_linear_backward_input_ex(dY, Wq, sW, dX=None, workspace=None, stream=None):
    """dX [T, K] = dY [T, N] . Wdeq in the type of dY (fp16 or bf16)."""
    lib = load_library()
    code = _act_dtype(dY.dtype)
    T, K, N, dX, ws = _backward_args(dY, Wq, sW, dX, workspace, dY.dtype)
    _check(lib.llmint8_linear_backward_input_ex(_ptr(dY), code, T, K, _ptr(Wq), _ptr(sW), N,
                                                _ptr(dX), _ptr(ws), _ws_bytes(ws),
                                                _stream(stream, dY.device)),
           "llmint8_linear_backward_input_ex")
    return dX


def llmint8_dequantize_weight_t_ex(Wq, sW, dtype=None, WdT=None, stream=None):
    """(Wq int8 [N, K], sW fp32 [N]) -> WdT [K, N] in ``dtype`` (fp16 default, or bf16)."""
    import torch
    lib = load_library()
    N, K = Wq.shape
    dtype = dtype or torch.float16
    _need(Wq, torch.int8, (N, K), "Wq")
    _need(sW, torch.float32, (N,), "sW")
    if WdT is None:
        WdT = torch.empty((K, N), dtype=dtype, device=Wq.device)
    _need(WdT, dtype, (K, N), "WdT")
    _check(lib.llmint8_dequantize_weight_t_ex(_ptr(Wq), _ptr(sW), N, K, _ptr(WdT), _act_dtype(dtype),
                                              _stream(stream, Wq.device)),
           "llmint8_dequantize_weight_t_ex")
    return WdT


def llmint8_linear_backward_input_timed(dY, Wq, sW, events, dX=None, workspace=None, stream=None):
    """Input gradient recording ``events`` (3 created torch.cuda.Event) around its two kernels."""
    lib = load_library()
    T, K, N, dX, ws = _backward_args(dY, Wq, sW, dX, workspace)
    handles = (_vp * len(events))(*[ctypes.c_void_p(e.cuda_event) for e in events])
    nk = ctypes.c_int(0)
    _check(lib.llmint8_linear_backward_input_timed(_ptr(dY), T, K, _ptr(Wq), _ptr(sW), N, _ptr(dX),
                                                   _ptr(ws), _ws_bytes(ws),
                                                   _stream(stream, dY.device), handles, len(events),
                                                   ctypes.byref(nk)),
           "llmint8_linear_backward_input_timed")
    return dX


def _codec_dtype(dtype):
    import torch
    if dtype == torch.float16:
        return LLMINT8_DTYPE_F16
    if dtype == torch.float32:
        return LLMINT8_DTYPE_F32
    raise ValueError(f"blockwise codec: fp16 or fp32 only, got {dtype}")


def llmint8_quantize_blockwise(x, block: int = 4096, q=None, absmax=None, stream=None):
    """Blockwise int8 codes of a contiguous fp16/fp32 tensor (taken flat):
    (q int8 [n], absmax fp32 [ceil(n / block)])."""
    import torch
    lib = load_library()
    if not (isinstance(x, torch.Tensor) and x.is_cuda and x.is_contiguous()):
        raise ValueError("x: expected a contiguous CUDA tensor")
    n = x.numel()
    nb = -(-n // block)
    if q is None:
        q = torch.empty((n,), dtype=torch.int8, device=x.device)
    if absmax is None:
        absmax = torch.empty((nb,), dtype=torch.float32, device=x.device)
    _need(q, torch.int8, (n,), "q")
    _need(absmax, torch.float32, (nb,), "absmax")
    _check(lib.llmint8_quantize_blockwise(_ptr(x), _codec_dtype(x.dtype), n, block, _ptr(q),
                                          _ptr(absmax), _stream(stream, x.device)),
           "llmint8_quantize_blockwise")
    return q, absmax


def llmint8_dequantize_blockwise(q, absmax, block: int = 4096, dtype=None, out=None, stream=None):
    """Inverse of llmint8_quantize_blockwise: fp16 (default) or fp32 [n]."""
    import torch
    lib = load_library()
    n = q.numel()
    nb = -(-n // block)
    _need(q, torch.int8, (n,), "q")
    _need(absmax, torch.float32, (nb,), "absmax")
    if out is None:
        out = torch.empty((n,), dtype=dtype or torch.float16, device=q.device)
    if not (out.is_cuda and out.is_contiguous() and out.numel() == n):
        raise ValueError("out: expected a contiguous CUDA tensor of n elements")
    _check(lib.llmint8_dequantize_blockwise(_ptr(q), _ptr(absmax), n, block, _ptr(out),
                                            _codec_dtype(out.dtype), _stream(stream, q.device)),
           "llmint8_dequantize_blockwise")
    return out


def _quant_type(q):
    if isinstance(q, str):
        codes = {"nf4": LLMINT8_QUANT_NF4, "fp4": LLMINT8_QUANT_FP4}
        if q.lower() not in codes:
            raise ValueError(f"4-bit type: 'nf4' or 'fp4', got {q!r}")
        return codes[q.lower()]
    return int(q)


def llmint8_code_book_4bit(quant_type="nf4"):
    """The 16 fp32 levels of a 4-bit type, indexed by code (a host list)."""
    vals = (ctypes.c_float * 16)()
    _check(load_library().llmint8_code_book_4bit(_quant_type(quant_type), vals),
           "llmint8_code_book_4bit")
    return list(vals)


def llmint8_quantize_4bit(W, block: int = 64, quant_type="nf4", packed=None, absmax=None,
                          stream=None):
    """Blockwise 4-bit codes of a contiguous fp16/bf16 tensor taken flat:
    (packed uint8 [n / 2], absmax fp32 [ceil(n / block)])."""
    import torch
    lib = load_library()
    if not (isinstance(W, torch.Tensor) and W.is_cuda and W.is_contiguous()):
        raise ValueError("W: expected a contiguous CUDA tensor")
    n = W.numel()
    nb = -(-n // block)
    if packed is None:
        packed = torch.empty((n // 2,), dtype=torch.uint8, device=W.device)
    if absmax is None:
        absmax = torch.empty((nb,), dtype=torch.float32, device=W.device)
    _need(packed, torch.uint8, (n // 2,), "packed")
    _need(absmax, torch.float32, (nb,), "absmax")
    _check(lib.llmint8_quantize_4bit(_ptr(W), _act_dtype(W.dtype), n, block, _quant_type(quant_type),
                                     _ptr(packed), _ptr(absmax), _stream(stream, W.device)),
           "llmint8_quantize_4bit")
    return packed, absmax


def llmint8_dequantize_4bit(packed, absmax, block: int = 64, quant_type="nf4", dtype=None,
                            out=None, stream=None):
    """Inverse of llmint8_quantize_4bit: fp16 (default) or bf16 [2 * packed.numel()]."""
    import torch
    lib = load_library()
    n = 2 * packed.numel()
    nb = -(-n // block)
    _need(packed, torch.uint8, (n // 2,), "packed")
    _need(absmax, torch.float32, (nb,), "absmax")
    if out is None:
        out = torch.empty((n,), dtype=dtype or torch.float16, device=packed.device)
    if not (out.is_cuda and out.is_contiguous() and out.numel() == n):
        raise ValueError("out: expected a contiguous CUDA tensor of n elements")
    _check(lib.llmint8_dequantize_4bit(_ptr(packed), _ptr(absmax), n, block, _quant_type(quant_type),
                                       _ptr(out), _act_dtype(out.dtype), _stream(stream, packed.device)),
           "llmint8_dequantize_4bit")
    return out


def llmint8_linear_4bit(X, packed, absmax, N: int, block: int = 64, quant_type="nf4", bias=None,
                        Y=None, stream=None):
    """Y [T, N] = X [T, K] . Wdeq^T (+ bias) with the 4-bit weight [N, K] dequantized on the fly.
    X, bias and Y share one type (fp16 or bf16)."""
    import torch
    lib = load_library()
    T, K = X.shape
    _need(X, X.dtype, (T, K), "X")
    _need(packed, torch.uint8, (N * K // 2,), "packed")
    _need(absmax, torch.float32, (-(-N * K // block),), "absmax")
    if bias is not None:
        _need(bias, X.dtype, (N,), "bias")
    if Y is None:
        Y = torch.empty((T, N), dtype=X.dtype, device=X.device)
    _need(Y, X.dtype, (T, N), "Y")
    _check(lib.llmint8_linear_4bit(_ptr(X), _act_dtype(X.dtype), T, K, _ptr(packed), _ptr(absmax),
                                   block, _quant_type(quant_type), N, _ptr(bias), _ptr(Y),
                                   _stream(stream, X.device)),
           "llmint8_linear_4bit")
    return Y


class Linear4bit:
    """Drop-in 4-bit (NF4 by default, or FP4) replacement of an fp16 or bf16 linear layer.

    The weight is quantized blockwise once at construction ("bitsandbytes: GPU-
    Accelerated Inference ...", introduction: the 4-bit layer keeps the weight
    in blocks with their own scaling factors and computes in a 16-bit type with
    the weight dequantized per operation); ``forward`` streams the codes and
    never stores the dequantized weight. Activations, bias and output take the
    weight's type.
    """

    def __init__(self, weight, bias=None, block: int = 64, quant_type="nf4"):
        self.out_features, self.in_features = weight.shape
        self.block, self.quant_type = int(block), quant_type
        self.dtype = weight.dtype
        self.packed, self.absmax = llmint8_quantize_4bit(weight.contiguous(), self.block, quant_type)
        self.bias = None if bias is None else bias.detach().to(weight.dtype).contiguous()

    def memory_bytes(self) -> int:
        extra = 0 if self.bias is None else self.bias.numel() * 2
        return self.packed.numel() + self.absmax.numel() * 4 + extra

    def forward(self, X):
        shape = X.shape
        X2 = X.reshape(-1, self.in_features).contiguous()
        Y = llmint8_linear_4bit(X2, self.packed, self.absmax, self.out_features, self.block,
                                self.quant_type, bias=self.bias)
        return Y.reshape(*shape[:-1], self.out_features)

    __call__ = forward


def _autograd_function():
    import torch

    class _Int8LinearFn(torch.autograd.Function):
        """Forward through llmint8_linear; backward gives the input gradient only
        (the int8 weight is frozen; an adapter trained on top needs dX)."""

        @staticmethod
        def forward(ctx, X2, layer):
            ctx.layer = layer
            return layer._forward(X2)

        @staticmethod
        def backward(ctx, dY):
            layer = ctx.layer
            dY = dY.contiguous().to(layer.dtype)
            if layer.dtype == torch.float16:
                dX = llmint8_linear_backward_input(dY, layer.Wq, layer.sW)
            else:
                dX = llmint8_linear_backward_input_ex(dY, layer.Wq, layer.sW)
            return dX, None

    return _Int8LinearFn


_FN = None


def _fp16():
    import torch
    return torch.float16


# One forward workspace per (device, stream), shared by every Int8Linear: calls on one
# stream run one after another, so layers never use it at the same time.
_SHARED_WS = {}


def _shared_workspace(need, device):
    import torch
    if need == 0:
        return None
    key = (device.index if device.index is not None else torch.cuda.current_device(),
           torch.cuda.current_stream(device).cuda_stream)
    ws = _SHARED_WS.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty((need,), dtype=torch.uint8, device=device)
        _SHARED_WS[key] = ws
    return ws


def shared_workspace_bytes() -> int:
    """Device bytes held by the forward workspaces that Int8Linear layers share."""
    return sum(ws.numel() for ws in _SHARED_WS.values())


class Int8Linear:
    """Drop-in int8 replacement of an fp16 or bf16 linear layer, with or without bias.

    The weight is quantized once at construction ("bitsandbytes" glossary,
    introduction: quantization happens when the model loads); ``forward`` runs
    the LLM.int8() forward ("Hugging Face Quantization with bitsandbytes",
    sections 2 and 3; section 5 for bf16 as the compute type) with the bias
    added before the output's rounding, and, for inputs that require a
    gradient, registers the input-gradient kernels (fp16 or bf16) as its backward
    (same page, section 6: the int8 weights stay frozen while an adapter on top
    is trained).
    Activations, bias and output take the weight's type.
    """

    def __init__(self, weight, threshold: float = 6.0, bias=None):
        self.threshold = float(threshold)
        self.out_features, self.in_features = weight.shape
        self.dtype = weight.dtype
        self.Wq, self.sW = llmint8_quantize_weight_ex(weight.contiguous())
        self.bias = None if bias is None else bias.detach().to(weight.dtype).contiguous()

    def memory_bytes(self) -> int:
        """Device bytes this layer holds: the int8 weight, its scales and the bias. The
        forward's scratch is not per layer: every Int8Linear on a device and stream shares
        one workspace (``shared_workspace_bytes()``), and the fused decode route needs none."""
        extra = 0 if self.bias is None else self.bias.numel() * 2
        return self.Wq.numel() + self.sW.numel() * 4 + extra

    def _forward(self, X2):
        ws = _shared_workspace(llmint8_workspace_bytes(X2.shape[0], self.in_features,
                                                       self.out_features), X2.device)
        if self.dtype == _fp16() and self.bias is None:
            return llmint8_linear(X2, self.Wq, self.sW, self.threshold, workspace=ws)
        return llmint8_linear_ex(X2, self.Wq, self.sW, self.threshold, bias=self.bias,
                                 workspace=ws)

    def forward(self, X):
        """Y = the LLM.int8() forward of X. When X requires a gradient, the
        backward pass gives dX = dY . Wdeq (the weight itself stays frozen)."""
        global _FN
        shape = X.shape
        X2 = X.reshape(-1, self.in_features).contiguous()
        if X2.requires_grad:
            if _FN is None:
                _FN = _autograd_function()
            Y = _FN.apply(X2, self)
        else:
            Y = self._forward(X2)
        return Y.reshape(*shape[:-1], self.out_features)

    __call__ = forward
