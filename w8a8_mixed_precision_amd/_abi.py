"""ctypes declarations of libw8mp.so (the C ABI in include/w8mp.h).

Loading fails loudly: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw8mp.so")

W8_OK, W8_ERR_INVALID_ARGUMENT, W8_ERR_UNSUPPORTED, W8_ERR_WORKSPACE, W8_ERR_HIP = range(5)
W8_DT_F16, W8_DT_BF16, W8_DT_F32 = range(3)
W8_Q_INT8, W8_Q_FP8_E4M3, W8_Q_INT4_G128 = range(3)
W8_INT8_MAX_K = 133144
W8_PRODUCER_NONE, W8_PRODUCER_RMSNORM, W8_PRODUCER_GELU_TANH = range(3)

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_size = ctypes.c_size_t
_f = ctypes.c_float


class Producer(ctypes.Structure):
    """struct w8_producer of include/w8mp.h."""
    _fields_ = [("kind", ctypes.c_int), ("gamma", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("shift", ctypes.c_void_p), ("eps", ctypes.c_float)]


class DitBlock(ctypes.Structure):
    """struct w8_dit_block of include/w8mp.h."""
    _fields_ = [("D", ctypes.c_int64), ("F", ctypes.c_int64), ("threshold", ctypes.c_float)] + [
        (f"{k}_{n}", ctypes.c_void_p) for n in ("qkv", "o", "up", "down") for k in ("w", "s", "b")] + [
        ("w_down16", ctypes.c_void_p), ("norm1", Producer), ("norm2", Producer)]


# name -> (restype, argtypes)
SIGNATURES = {
    "quantize_weight_rowwise": (_int, [_p, _int, _i64, _i64, _int, _p, _p, _p]),
    "int8_mixed_linear_workspace_size": (_size, [_i64, _i64, _i64]),
    "int8_mixed_linear": (_int, [_p, _int, _i64, _i64, _p, _p, _i64, _f, _p, _int, _p, _size, _p]),
    "int8_mixed_linear_noalloc": (_int, [_p, _int, _i64, _i64, _p, _p, _i64, _f, _p, _int, _p]),
    "int8_mixed_linear_fused": (_int, [_p, _int, _i64, _i64, _p, _p, _p, _p, _i64, _f, _p, _int, _p, _size, _p]),
    "fp8_w8a8_linear_workspace_size": (_size, [_i64, _i64, _i64]),
    "fp8_w8a8_linear": (_int, [_p, _int, _i64, _i64, _p, _p, _i64, _p, _p, _int, _p, _size, _p]),
    "fp8_w8a16_linear_workspace_size": (_size, [_i64, _i64, _i64]),
    "w4a8_linear_workspace_size": (_size, [_i64, _i64, _i64]),
    "w8_dit_block_workspace_size": (_size, [_i64, _i64, _i64]),
    "w8_dit_block_forward": (_int, [_p, _p, _i64, _p, _p, _size, _p]),
    "w8dbg_linear16_workspace_size": (_size, [_i64, _i64, _i64, _int, _int]),
    "w8dbg_linear16": (_int, [_p, _int, _i64, _i64, _p, _i64, _int, _int, _p, _int, _p, _size, _p]),
    "w4a8_linear": (_int, [_p, _int, _i64, _i64, _p, _p, _i64, _p, _int, _p, _size, _p]),
    "w8dbg_w4a8_linear_workspace_size": (_size, [_i64, _i64, _i64, _int]),
    "w8dbg_w4a8_linear": (_int, [_p, _int, _i64, _i64, _p, _p, _i64, _int, _p, _int, _p, _size, _p]),
    "fp8_w8a16_linear": (_int, [_p, _int, _i64, _i64, _p, _p, _i64, _p, _int, _p, _size, _p]),
    "w8_status_string": (ctypes.c_char_p, [_int]),
    "w8_last_error": (ctypes.c_char_p, []),
    "w8dbg_int8_quantize_activations_workspace_size": (_size, [_i64, _i64]),
    "w8dbg_int8_quantize_activations": (_int, [_p, _int, _i64, _i64, _p, _f, _p, _p, _p, _p, _p, _size, _p]),
    "w8dbg_produce": (_int, [_p, _int, _i64, _i64, _p, _p, _p]),
    "w8dbg_int8_gemm_i32_workspace_size": (_size, [_i64, _i64, _i64, _int, _int]),
    "w8dbg_int8_gemm_i32": (_int, [_p, _p, _i64, _i64, _i64, _int, _int, _p, _p, _size, _p]),
    "w8dbg_fp8_quantize_activations": (_int, [_p, _int, _i64, _i64, _p, _p, _p, _p]),
    "w8dbg_fp8_gemm_workspace_size": (_size, [_i64, _i64, _i64, _int, _int]),
    "w8dbg_fp8_gemm": (_int, [_p, _p, _p, _p, _i64, _i64, _i64, _int, _int, _p, _int, _p, _size, _p]),
    "w8dbg_fp8_w8a16_linear_workspace_size": (_size, [_i64, _i64, _i64, _int, _int]),
    "w8dbg_fp8_w8a16_linear": (_int, [_p, _int, _i64, _i64, _p, _p, _i64, _int, _int, _p, _int, _p, _size, _p]),
    "w8dbg_cvt_f16_pair_check": (_int, [_p, _p]),
    "w8dbg_int8_mixed_linear_plan_workspace_size": (_size, [_i64, _i64, _i64, _int]),
    "w8dbg_int8_mixed_linear_plan": (_int, [_p, _int, _i64, _i64, _p, _p, _p, _p, _i64, _f, _p, _int, _p, _size,
                                            _int, _p]),
    "w8dbg_int8_mixed_linear_events": (_int, [_p, _int, _i64, _i64, _p, _p, _p, _p, _i64, _f, _p, _int, _p, _size,
                                               _p, _p]),
    "w8dbg_fp8_w8a8_linear_events": (_int, [_p, _int, _i64, _i64, _p, _p, _i64, _p, _p, _int, _p, _size, _p, _p]),
    "w8dbg_int8_gemm_timeline": (_int, [_p, _int, _i64, _i64, _p, _p, _i64, _f, _p, _int, _p, _size, _p, _size,
                                         ctypes.POINTER(ctypes.c_int), _p]),
    "w8dbg_int8_workspace_layout": (_int, [_i64, _i64, _i64, ctypes.POINTER(_size)]),
    "w8dbg_dit_block_layout": (_int, [_i64, _i64, _i64, ctypes.POINTER(_size)]),
    "w8dbg_mfma_peak": (_int, [_int, _int, _int, _p, ctypes.POINTER(ctypes.c_double), _p]),
    "w8dbg_lds_stream": (_int, [_p, _size, _int, _int, _int, _int, _int, _p, ctypes.POINTER(ctypes.c_double), _p]),
}


class W8Error(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_string(status)}: {detail}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m w8a8_mixed_precision_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().w8_status_string(status).decode()


def check(status: int) -> None:
    if status != W8_OK:
        raise W8Error(status, lib().w8_last_error().decode())
