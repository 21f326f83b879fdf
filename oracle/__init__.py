"""CPU oracle for W8A8 int8-dynamic linear layers (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never does, and this package never imports the product.

The arithmetic lives in ``oracle.c`` (plain C loops, OpenMP across rows);
this module compiles it with gcc on first use and wraps it for NumPy arrays.
What each function computes, and the passage of the pages it follows, is
stated in ``oracle.c``.

Every array crossing this boundary is C-contiguous; bf16 and fp16 values are
carried as ``uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-std=c11", "-Wall", "-Wextra", "-Wno-unused-parameter"]

__all__ = ["build", "Oracle", "load", "LIBRARY", "SOURCE", "CFLAGS"]


def build(source: str = SOURCE, output: str = LIBRARY, extra_flags=()) -> str:
    """Compile ``source`` into a shared library with gcc; returns its path."""
    cmd = ["gcc", *CFLAGS, *extra_flags, source, "-o", output + ".tmp", "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(output + ".tmp", output)
    return output


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: str):
        self.path = path
        lib = ctypes.CDLL(path)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        for name, args in {
            "oracle_quant_rows_bf16": [vp, i64, i64, i64, vp, i64, vp],
            "oracle_quant_rows_f32": [vp, i64, i64, i64, vp, i64, vp],
            "oracle_gemm_i32_rows": [vp, i64, vp, i64, vp, i64, i64, i64, vp, i64],
            "oracle_epilogue_f32": [vp, i64, i64, i64, vp, vp, vp, vp, i64],
            "oracle_epilogue_f64": [vp, i64, i64, i64, vp, vp, vp, vp, i64],
            "oracle_quant_rows_f16": [vp, i64, i64, i64, vp, i64, vp],
            "oracle_epilogue_f32_f16": [vp, i64, i64, i64, vp, vp, vp, vp, i64],
            "oracle_epilogue_f64_f16": [vp, i64, i64, i64, vp, vp, vp, vp, i64],
            "oracle_fp8_quant_rows_bf16": [vp, i64, i64, i64, vp, i64, vp],
            "oracle_fp8_quant_rows_f32": [vp, i64, i64, i64, vp, i64, vp],
            "oracle_fp8_gemm_rows": [vp, i64, vp, i64, vp, i64, i64, i64, vp, i64],
            "oracle_fp8_epilogue": [vp, i64, i64, i64, vp, vp, vp, vp, vp, i64, ctypes.c_int],
        }.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.oracle_float_to_bf16.argtypes = [ctypes.c_float]
        lib.oracle_float_to_bf16.restype = ctypes.c_uint16
        lib.oracle_double_to_bf16.argtypes = [ctypes.c_double]
        lib.oracle_double_to_bf16.restype = ctypes.c_uint16
        lib.oracle_double_to_f16.argtypes = [ctypes.c_double]
        lib.oracle_double_to_f16.restype = ctypes.c_uint16
        lib.oracle_f16_to_float.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_float.restype = ctypes.c_float
        lib.oracle_double_to_e4m3.argtypes = [ctypes.c_double]
        lib.oracle_double_to_e4m3.restype = ctypes.c_uint8
        lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_to_double.restype = ctypes.c_double
        self.lib = lib

    @staticmethod
    def _check(rc: int, what: str):
        if rc == 2:
            raise OverflowError(f"{what}: an int8 dot product left the int32 range")
        if rc != 0:
            raise ValueError(f"{what}: bad arguments (code {rc})")

    # -- step 1: per-token activation quantization -------------------------
    def quant_per_token(self, x_bf16: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
        M, K = x.shape
        q = np.empty((M, K), dtype=np.int8)
        s = np.empty(M, dtype=np.float32)
        self._check(self.lib.oracle_quant_rows_bf16(_p(x), M, K, K, _p(q), K, _p(s)),
                    "quant_per_token")
        return q, s

    def quant_per_token_f16(self, x_f16: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        """Step 1 on fp16 activations (uint16 bit patterns)."""
        x = np.ascontiguousarray(x_f16, dtype=np.uint16)
        M, K = x.shape
        q = np.empty((M, K), dtype=np.int8)
        s = np.empty(M, dtype=np.float32)
        self._check(self.lib.oracle_quant_rows_f16(_p(x), M, K, K, _p(q), K, _p(s)),
                    "quant_per_token_f16")
        return q, s

    # -- step 2: per-output-channel weight quantization --------------------
    def quant_per_channel(self, w_f32: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        w = np.ascontiguousarray(w_f32, dtype=np.float32)
        N, K = w.shape
        q = np.empty((N, K), dtype=np.int8)
        s = np.empty(N, dtype=np.float32)
        self._check(self.lib.oracle_quant_rows_f32(_p(w), N, K, K, _p(q), K, _p(s)),
                    "quant_per_channel")
        return q, s

    # -- step 3: exact int32 accumulators ----------------------------------
    def gemm_i32(self, xq: np.ndarray, wq: np.ndarray,
                 rows: Optional[np.ndarray] = None) -> np.ndarray:
        a = np.ascontiguousarray(xq, dtype=np.int8)
        b = np.ascontiguousarray(wq, dtype=np.int8)
        M, K = a.shape
        N, K2 = b.shape
        if K != K2:
            raise ValueError("inner dimensions differ")
        r = None
        if rows is not None:
            r = np.ascontiguousarray(rows, dtype=np.int64)
            if r.size and (r.min() < 0 or r.max() >= M):
                raise IndexError("row index out of range")
            M = r.size
        acc = np.empty((M, N), dtype=np.int32)
        self._check(self.lib.oracle_gemm_i32_rows(_p(a), K, _p(r), M, _p(b), K, N, K,
                                                  _p(acc), N), "gemm_i32")
        return acc

    # -- step 4: scale epilogue --------------------------------------------
    def _epilogue(self, fn, acc, xs, ws, bias):
        acc = np.ascontiguousarray(acc, dtype=np.int32)
        xs = np.ascontiguousarray(xs, dtype=np.float32)
        ws = np.ascontiguousarray(ws, dtype=np.float32)
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.uint16)
        M, N = acc.shape
        if xs.shape != (M,) or ws.shape != (N,) or (b is not None and b.shape != (N,)):
            raise ValueError("scale/bias shapes do not match the accumulators")
        out = np.empty((M, N), dtype=np.uint16)
        self._check(fn(_p(acc), N, M, N, _p(xs), _p(ws), _p(b), _p(out), N), "epilogue")
        return out

    def epilogue_f32(self, acc, xs, ws, bias=None) -> np.ndarray:
        """bf16 bits of fl(fl(fl(acc)*xs)*ws) (+bias), fixed fp32 order."""
        return self._epilogue(self.lib.oracle_epilogue_f32, acc, xs, ws, bias)

    def epilogue_f64(self, acc, xs, ws, bias=None) -> np.ndarray:
        """bf16 bits of acc*xs*ws (+bias) evaluated in fp64, rounded once."""
        return self._epilogue(self.lib.oracle_epilogue_f64, acc, xs, ws, bias)

    def epilogue_f32_f16(self, acc, xs, ws, bias=None) -> np.ndarray:
        """fp16 bits of fl(fl(fl(acc)*xs)*ws) (+fp16 bias), fixed fp32 order."""
        return self._epilogue(self.lib.oracle_epilogue_f32_f16, acc, xs, ws, bias)

    def epilogue_f64_f16(self, acc, xs, ws, bias=None) -> np.ndarray:
        """fp16 bits of acc*xs*ws (+fp16 bias) evaluated in fp64, rounded once."""
        return self._epilogue(self.lib.oracle_epilogue_f64_f16, acc, xs, ws, bias)

    def double_to_f16(self, d: float) -> int:
        return int(self.lib.oracle_double_to_f16(d))

    def f16_to_float(self, h: int) -> float:
        return float(self.lib.oracle_f16_to_float(h))

    def float_to_bf16(self, f: float) -> int:
        return int(self.lib.oracle_float_to_bf16(f))

    def double_to_bf16(self, d: float) -> int:
        return int(self.lib.oracle_double_to_bf16(d))

    # -- the FP8 (e4m3) twin -------------------------------------------------
    def fp8_quant_per_token(self, x_bf16: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
        M, K = x.shape
        q = np.empty((M, K), dtype=np.uint8)
        s = np.empty(M, dtype=np.float32)
        self._check(self.lib.oracle_fp8_quant_rows_bf16(_p(x), M, K, K, _p(q), K, _p(s)),
                    "fp8_quant_per_token")
        return q, s

    def fp8_quant_per_channel(self, w_f32: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        w = np.ascontiguousarray(w_f32, dtype=np.float32)
        N, K = w.shape
        q = np.empty((N, K), dtype=np.uint8)
        s = np.empty(N, dtype=np.float32)
        self._check(self.lib.oracle_fp8_quant_rows_f32(_p(w), N, K, K, _p(q), K, _p(s)),
                    "fp8_quant_per_channel")
        return q, s

    def fp8_gemm(self, xq: np.ndarray, wq: np.ndarray,
                 rows: Optional[np.ndarray] = None) -> np.ndarray:
        """Exact (float64) sums of products of the decoded e4m3 codes."""
        a = np.ascontiguousarray(xq, dtype=np.uint8)
        b = np.ascontiguousarray(wq, dtype=np.uint8)
        M, K = a.shape
        N, K2 = b.shape
        if K != K2:
            raise ValueError("inner dimensions differ")
        r = None
        if rows is not None:
            r = np.ascontiguousarray(rows, dtype=np.int64)
            M = r.size
        acc = np.empty((M, N), dtype=np.float64)
        self._check(self.lib.oracle_fp8_gemm_rows(_p(a), K, _p(r), M, _p(b), K, N, K, _p(acc), N),
                    "fp8_gemm")
        return acc

    def fp8_epilogue(self, acc, xs, ws, bias=None, f16: bool = False
                     ) -> Tuple[np.ndarray, np.ndarray]:
        """(bits of the fp32-order epilogue on fl32(acc), bits of the fp64 value
        rounded once): bf16, or fp16 (with an fp16 bias) when f16."""
        acc = np.ascontiguousarray(acc, dtype=np.float64)
        xs = np.ascontiguousarray(xs, dtype=np.float32)
        ws = np.ascontiguousarray(ws, dtype=np.float32)
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.uint16)
        M, N = acc.shape
        o32 = np.empty((M, N), dtype=np.uint16)
        o64 = np.empty((M, N), dtype=np.uint16)
        self._check(self.lib.oracle_fp8_epilogue(_p(acc), N, M, N, _p(xs), _p(ws), _p(b), _p(o32),
                                                 _p(o64), N, int(f16)), "fp8_epilogue")
        return o32, o64

    def double_to_e4m3(self, d: float) -> int:
        return int(self.lib.oracle_double_to_e4m3(d))

    def e4m3_to_double(self, c: int) -> float:
        return float(self.lib.oracle_e4m3_to_double(c))

    # -- the whole layer ----------------------------------------------------
    def linear(self, x_bf16, wq, ws, bias=None, rows=None, f64=False):
        """Quantize X per token, multiply by int8 W, apply the epilogue.

        Returns (xq, xs, acc, out_bf16) with acc/out restricted to ``rows``
        when given (xq/xs always cover every row).
        """
        xq, xs = self.quant_per_token(x_bf16)
        acc = self.gemm_i32(xq, wq, rows)
        xs_r = xs if rows is None else xs[np.asarray(rows, dtype=np.int64)]
        out = (self.epilogue_f64 if f64 else self.epilogue_f32)(acc, xs_r, ws, bias)
        return xq, xs, acc, out


_default: Optional[Oracle] = None


def load(rebuild: bool = False) -> Oracle:
    """The oracle built from ``oracle.c`` (compiled if missing or stale)."""
    global _default
    if _default is not None and not rebuild:
        return _default
    stale = (not os.path.exists(LIBRARY)
             or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE))
    if rebuild or stale:
        build()
    _default = Oracle(LIBRARY)
    return _default
