"""ctypes view of libw8a8.so, the C ABI declared in include/w8a8.h.

Loading fails loudly when the library has not been built: there is no
Python or CPU fallback for any step of the layer.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libw8a8.so")

W8A8_OK = 0
W8A8_ERR_NULL = 1
W8A8_ERR_SHAPE = 2
W8A8_ERR_ALIGN = 3
W8A8_ERR_DEVICE = 4
W8A8_ERR_MODE = 5
W8A8_ERR_HIP = 6
W8A8_OUT_BF16 = 0
W8A8_OUT_I32 = 1
W8A8_OUT_F16 = 2
W8A8_MAX_K = 131056
W8A8_MAX_LDQ = 4194304

# name -> (restype, argtypes), in the order of include/w8a8.h
_i64, _vp, _int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
SIGNATURES = {
    "int8_quant_per_token": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp]),
    "int8_quant_per_token_f16": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp]),
    "int8_quant_per_channel": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp]),
    "int8_prepack_weight_bytes": (ctypes.c_size_t, [_i64, _i64]),
    "int8_prepack_weight": (_int, [_vp, _i64, _i64, _i64, _vp, _vp]),
    "int8_unpack_weight": (_int, [_vp, _i64, _i64, _vp, _i64, _vp]),
    "int8_quant_prepack_weight": (_int, [_vp, _int, _i64, _i64, _i64, _vp, _vp, _vp]),
    "int8_scaled_mm": (_int, [_vp, _i64, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _vp, _i64,
                              _vp]),
    "int8_scaled_mm_tile": (_int, [_vp, _i64, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _vp,
                                   _i64, _vp, _int]),
    "int8_quant_scaled_mm": (_int, [_vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                    _int, _vp, _i64, _vp]),
    "int8_quant_scaled_mm_tile": (_int, [_vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _i64,
                                         _i64, _int, _vp, _i64, _vp, _int]),
    "int8_scaled_mm_workspace_bytes": (ctypes.c_size_t, [_i64, _i64, _i64]),
    "int8_scaled_mm_ws": (_int, [_vp, _i64, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _vp, _i64,
                                 _vp, ctypes.c_size_t, _vp]),
    "int8_quant_scaled_mm_ws": (_int, [_vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                       _int, _vp, _i64, _vp, ctypes.c_size_t, _vp]),
    "int8_quant_scaled_mm_noalloc": (_int, [_vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _i64,
                                            _i64, _int, _vp, _i64, _vp]),
    "int8_quant_scaled_mm_f16": (_int, [_vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                        _int, _vp, _i64, _vp]),
    "int8_quant_scaled_mm_f16_tile": (_int, [_vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _i64,
                                             _i64, _int, _vp, _i64, _vp, _int]),
    "fp8_quant_per_token": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp]),
    "fp8_quant_per_channel": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp]),
    "fp8_quant_prepack_weight": (_int, [_vp, _int, _i64, _i64, _i64, _vp, _vp, _vp]),
    "fp8_scaled_mm": (_int, [_vp, _i64, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _vp, _i64,
                             _vp]),
    "fp8_scaled_mm_tile": (_int, [_vp, _i64, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _vp,
                                  _i64, _vp, _int]),
    "fp8_quant_scaled_mm": (_int, [_vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                   _int, _vp, _i64, _vp]),
    "fp8_quant_scaled_mm_tile": (_int, [_vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _i64,
                                        _i64, _int, _vp, _i64, _vp, _int]),
    "w8a8_fp8_tile_count": (_int, []),
    "w8a8_fused_wait_limit": (_int, [_int]),
    "w8a8_fp8_tile_auto": (_int, [_i64, _i64, _i64]),
    "w8a8_mm_tile_count": (_int, []),
    "w8a8_mm_tile_name": (ctypes.c_char_p, [_int]),
    "w8a8_mm_tile_auto": (_int, [_i64, _i64, _i64]),
    "w8a8_device_supported": (_int, [_int]),
    "w8a8_status_string": (ctypes.c_char_p, [_int]),
    "w8a8_last_error": (ctypes.c_char_p, []),
}


class W8A8Error(RuntimeError):
    """A libw8a8 entry point returned a non-zero status."""

    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        self.func = func
        super().__init__(f"{func}: {detail or status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(
                f"{LIBRARY} is missing: build it with `python -m w8a8_int8_dynamic_amd.build` "
                "(there is no fallback implementation)")
        # torch ships its own HIP runtime. Load it first so that libw8a8 binds
        # to that same runtime (one HIP context per process) instead of
        # pulling in a second copy from the ROCm install.
        import torch  # noqa: F401
        handle = ctypes.CDLL(LIBRARY)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().w8a8_status_string(status).decode()


def last_error() -> str:
    return lib().w8a8_last_error().decode()


def call(name: str, *args) -> int:
    """Call entry point ``name``; raise W8A8Error unless it returns W8A8_OK."""
    rc = getattr(lib(), name)(*args)
    if rc != W8A8_OK:
        raise W8A8Error(rc, name, last_error())
    return rc
