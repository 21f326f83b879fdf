"""Torch-tensor wrappers over the libw8a8 C ABI (argument marshalling only).

Every step of the layer runs in the HIP kernels; these functions only check
dtypes and devices, allocate outputs with torch, and pass raw device
pointers, leading dimensions and torch's current HIP stream to the library.
Tensors must be on a CUDA (HIP) device; the last dimension must be
contiguous (stride 1); the row stride becomes the leading dimension.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import W8A8_OUT_BF16, W8A8_OUT_F16, W8A8_OUT_I32, call

__all__ = ["quant_per_token", "quant_per_channel", "prepack_weight", "quant_prepack_weight", "unpack_weight",
           "prepack_weight_bytes", "scaled_mm", "quant_scaled_mm", "tile_count", "tile_name",
           "workspace_bytes", "new_workspace",
           "tile_auto", "device_supported", "fp8_quant_per_token", "fp8_quant_per_channel",
           "fp8_quant_prepack_weight", "fp8_scaled_mm", "fp8_quant_scaled_mm", "fp8_tile_count"]


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _matrix(t: torch.Tensor, name: str, dtype: torch.dtype) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if t.stride(1) != 1 and t.shape[1] > 1:
        raise ValueError(f"{name} must have a contiguous last dimension")
    return t


def _ld(t: torch.Tensor) -> int:
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])


def _vector(t: Optional[torch.Tensor], n: int, name: str, dtype: torch.dtype):
    if t is None:
        return None
    if not t.is_cuda or t.dtype != dtype or t.shape != (n,) or (n > 1 and t.stride(0) != 1):
        raise ValueError(f"{name} must be a contiguous {dtype} device vector of length {n}")
    return t


def _same_device(ref: torch.Tensor, *others: Optional[torch.Tensor]) -> None:
    for t in others:
        if t is not None and t.device != ref.device:
            raise ValueError(f"all tensors must be on {ref.device}, got one on {t.device}")


def _packed(w_packed: torch.Tensor, N: int, K: int) -> None:
    if not w_packed.is_cuda or w_packed.dtype != torch.uint8 or \
            w_packed.numel() < prepack_weight_bytes(N, K):
        raise ValueError("w_packed must be a uint8 device buffer of the packed layout (N, K)")


def _round_up(a: int, b: int) -> int:
    return -(-a // b) * b


def _rows_aligned(t: torch.Tensor, elems: int) -> torch.Tensor:
    """t itself when its rows start on 16-byte boundaries (row stride a multiple of
    ``elems``), else a copy into a row-padded buffer, viewed back to t's shape."""
    if t.data_ptr() % 16 == 0 and _ld(t) % elems == 0:
        return t
    M, K = t.shape
    buf = torch.empty((M, _round_up(K, elems)), dtype=t.dtype, device=t.device)
    buf[:, :K].copy_(t)
    return buf[:, :K]


def _codes(M: int, K: int, device) -> torch.Tensor:
    """int8 [M, K] view of a buffer whose rows are padded to 16 bytes, the row
    stride int8_scaled_mm requires."""
    return torch.empty((M, _round_up(K, 16)), dtype=torch.int8, device=device)[:, :K]


_ACT_ENTRY = {torch.bfloat16: "", torch.float16: "_f16"}
_OUT_MODE = {torch.bfloat16: W8A8_OUT_BF16, torch.float16: W8A8_OUT_F16, torch.int32: W8A8_OUT_I32}


def _act_dtype(x: torch.Tensor) -> torch.dtype:
    if x.dtype not in _ACT_ENTRY:
        raise TypeError(f"x must be bfloat16 or float16, got {x.dtype}")
    return x.dtype


def _out_mode(out_dtype: torch.dtype) -> int:
    if out_dtype not in _OUT_MODE:
        raise TypeError("out_dtype must be torch.bfloat16, torch.float16 or torch.int32")
    return _OUT_MODE[out_dtype]


def quant_per_token(x: torch.Tensor, xq: Optional[torch.Tensor] = None,
                    xs: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-token dynamic quantization of bf16 or fp16 x [M, K] -> (int8 [M, K], fp32 [M])."""
    _matrix(x, "x", _act_dtype(x))
    M, K = x.shape
    x = _rows_aligned(x, 8)
    if xq is None:
        xq = _codes(M, K, x.device)
    if xs is None:
        xs = torch.empty((M,), dtype=torch.float32, device=x.device)
    _matrix(xq, "xq", torch.int8)
    if xq.shape != (M, K):
        raise ValueError(f"xq must have shape {(M, K)}")
    _vector(xs, M, "xs", torch.float32)
    _same_device(x, xq, xs)
    with torch.cuda.device(x.device):
        call("int8_quant_per_token" + _ACT_ENTRY[x.dtype], x.data_ptr(), M, K, _ld(x),
             xq.data_ptr(), _ld(xq), xs.data_ptr(), _stream(x))
    return xq, xs


def quant_per_channel(w: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-output-channel quantization of fp32 w [N, K] -> (int8 [N, K], fp32 [N])."""
    _matrix(w, "w", torch.float32)
    N, K = w.shape
    w = _rows_aligned(w, 4)
    wq = _codes(N, K, w.device)
    ws = torch.empty((N,), dtype=torch.float32, device=w.device)
    with torch.cuda.device(w.device):
        call("int8_quant_per_channel", w.data_ptr(), N, K, _ld(w), wq.data_ptr(), _ld(wq),
             ws.data_ptr(), _stream(w))
    return wq, ws


def prepack_weight_bytes(N: int, K: int) -> int:
    n = _lib.lib().int8_prepack_weight_bytes(N, K)
    if n == 0:
        raise ValueError(f"no prepacked size for N={N}, K={K}")
    return n


def prepack_weight(wq: torch.Tensor) -> torch.Tensor:
    """Repack int8 wq [N, K] into the fragment layout int8_scaled_mm reads (uint8 bytes)."""
    _matrix(wq, "wq", torch.int8)
    N, K = wq.shape
    packed = torch.empty((prepack_weight_bytes(N, K),), dtype=torch.uint8, device=wq.device)
    with torch.cuda.device(wq.device):
        call("int8_prepack_weight", wq.data_ptr(), N, K, _ld(wq), packed.data_ptr(), _stream(wq))
    return packed


def quant_prepack_weight(w: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Online per-output-channel quantization of a bf16 or fp32 weight [N, K],
    written straight into the prepacked layout: (packed uint8 bytes, fp32 [N]).
    The same bytes and scales as prepack_weight(quant_per_channel(w))."""
    if w.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"w must be bfloat16 or float32, got {w.dtype}")
    _matrix(w, "w", w.dtype)
    N, K = w.shape
    f32 = w.dtype == torch.float32
    w = _rows_aligned(w, 4 if f32 else 8)
    packed = torch.empty((prepack_weight_bytes(N, K),), dtype=torch.uint8, device=w.device)
    ws = torch.empty((N,), dtype=torch.float32, device=w.device)
    with torch.cuda.device(w.device):
        call("int8_quant_prepack_weight", w.data_ptr(), 0 if f32 else 1, N, K, _ld(w),
             packed.data_ptr(), ws.data_ptr(), _stream(w))
    return packed, ws


def unpack_weight(packed: torch.Tensor, N: int, K: int) -> torch.Tensor:
    """Inverse of prepack_weight: int8 [N, K]."""
    if not packed.is_cuda or packed.dtype != torch.uint8 or packed.numel() < prepack_weight_bytes(N, K):
        raise ValueError("packed must be a uint8 device buffer from prepack_weight")
    wq = torch.empty((N, K), dtype=torch.int8, device=packed.device)
    with torch.cuda.device(packed.device):
        call("int8_unpack_weight", packed.data_ptr(), N, K, wq.data_ptr(), K, _stream(packed))
    return wq


def workspace_bytes(M: int, N: int, K: int) -> int:
    """Bytes of workspace the split of K uses for an M x N x K product (0: none)."""
    return int(_lib.lib().int8_scaled_mm_workspace_bytes(M, N, K))


def new_workspace(N: int, K: int, max_rows: int = 32, device=None) -> Optional[torch.Tensor]:
    """A zeroed workspace large enough for every M up to max_rows against an
    N x K weight (None when no such shape splits K). Give each stream (or
    each concurrently replayed graph) its own."""
    need = max(workspace_bytes(m, N, K) for m in range(1, max_rows + 1))
    if need == 0:
        return None
    if device is None:
        device = torch.device("cuda", torch.cuda.current_device())
    return torch.zeros((need,), dtype=torch.uint8, device=device)


def _workspace(workspace: Optional[torch.Tensor]):
    if workspace is None:
        return None, 0
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def scaled_mm(xq: torch.Tensor, xs: Optional[torch.Tensor], w_packed: torch.Tensor,
              ws: Optional[torch.Tensor], N: int, bias: Optional[torch.Tensor] = None,
              out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
              tile: int = -1, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[m, n] = acc * xs[m] * ws[n] (+ bias[n]) rounded to out_dtype (bf16 or fp16;
    the bias in the same type), or the int32 accumulators when out_dtype=int32.
    With a workspace (from new_workspace; automatic tile only) decode-shaped
    products may split K over workgroups; results are bit-identical."""
    _matrix(xq, "xq", torch.int8)
    M, K = xq.shape
    mode = _out_mode(out_dtype)
    if mode != W8A8_OUT_I32:
        _vector(xs, M, "xs", torch.float32)
        _vector(ws, N, "ws", torch.float32)
        _vector(bias, N, "bias", out_dtype)
    _packed(w_packed, N, K)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=xq.device)
    _matrix(out, "out", out_dtype)
    if out.shape != (M, N):
        raise ValueError(f"out must have shape {(M, N)}")

    def ptr(t):
        return None if t is None or mode == W8A8_OUT_I32 else t.data_ptr()

    _same_device(xq, w_packed, out, *((xs, ws, bias) if mode != W8A8_OUT_I32 else ()))
    if workspace is not None:
        if tile != -1:
            raise ValueError("a workspace goes with the automatic tile (tile=-1)")
        _same_device(xq, workspace)
        wp, wb = _workspace(workspace)
        with torch.cuda.device(xq.device):
            call("int8_scaled_mm_ws", xq.data_ptr(), _ld(xq), ptr(xs), w_packed.data_ptr(), ptr(ws),
                 ptr(bias), M, N, K, mode, out.data_ptr(), _ld(out), wp, wb, _stream(xq))
        return out
    with torch.cuda.device(xq.device):
        call("int8_scaled_mm_tile", xq.data_ptr(), _ld(xq), ptr(xs), w_packed.data_ptr(), ptr(ws),
             ptr(bias), M, N, K, mode, out.data_ptr(), _ld(out), _stream(xq), tile)
    return out


def quant_scaled_mm(x: torch.Tensor, w_packed: torch.Tensor, ws: Optional[torch.Tensor], N: int,
                    bias: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                    out: Optional[torch.Tensor] = None, tile: int = -1,
                    xq: Optional[torch.Tensor] = None, xs: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None
                    ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Per-token quant of bf16 or fp16 x [M, K] and the scaled matmul in one call.

    out_dtype defaults to x's type. Returns (out, xq, xs): out as scaled_mm
    returns it, and the int8 codes and fp32 scales the quant produced
    (bit-identical to quant_per_token). A workspace (bf16 x, automatic tile)
    lets decode-shaped products split K, as in scaled_mm."""
    _matrix(x, "x", _act_dtype(x))
    if out_dtype is None:
        out_dtype = x.dtype
    M, K = x.shape
    x = _rows_aligned(x, 8)
    mode = _out_mode(out_dtype)
    if mode != W8A8_OUT_I32:
        _vector(ws, N, "ws", torch.float32)
        _vector(bias, N, "bias", out_dtype)
    _packed(w_packed, N, K)
    if xq is None:
        xq = _codes(M, K, x.device)
    if xs is None:
        xs = torch.empty((M,), dtype=torch.float32, device=x.device)
    _matrix(xq, "xq", torch.int8)
    if xq.shape != (M, K):
        raise ValueError(f"xq must have shape {(M, K)}")
    _vector(xs, M, "xs", torch.float32)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    _matrix(out, "out", out_dtype)
    if out.shape != (M, N):
        raise ValueError(f"out must have shape {(M, N)}")

    def ptr(t):
        return None if t is None or mode == W8A8_OUT_I32 else t.data_ptr()

    _same_device(x, w_packed, xq, xs, out, *((ws, bias) if mode != W8A8_OUT_I32 else ()))
    if workspace is not None:
        if tile != -1 or x.dtype != torch.bfloat16:
            raise ValueError("a workspace goes with bf16 activations and the automatic tile")
        _same_device(x, workspace)
        wp, wb = _workspace(workspace)
        with torch.cuda.device(x.device):
            call("int8_quant_scaled_mm_ws", x.data_ptr(), _ld(x), xq.data_ptr(), _ld(xq),
                 xs.data_ptr(), w_packed.data_ptr(), ptr(ws), ptr(bias), M, N, K, mode,
                 out.data_ptr(), _ld(out), wp, wb, _stream(x))
        return out, xq, xs
    with torch.cuda.device(x.device):
        call("int8_quant_scaled_mm" + _ACT_ENTRY[x.dtype] + "_tile", x.data_ptr(), _ld(x),
             xq.data_ptr(), _ld(xq), xs.data_ptr(), w_packed.data_ptr(), ptr(ws), ptr(bias), M,
             N, K, mode, out.data_ptr(), _ld(out), _stream(x), tile)
    return out, xq, xs


# ---- the FP8 (e4m3) twin ------------------------------------------------
_FP8_OUT_MODE = {torch.bfloat16: W8A8_OUT_BF16, torch.float16: W8A8_OUT_F16,
                 torch.float32: W8A8_OUT_I32}


def _fp8_codes(M: int, K: int, device) -> torch.Tensor:
    return torch.empty((M, _round_up(K, 16)), dtype=torch.uint8, device=device)[:, :K]


def fp8_quant_per_token(x: torch.Tensor, xq: Optional[torch.Tensor] = None,
                        xs: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-token dynamic e4m3 quantization of bf16 x [M, K] -> (uint8 codes [M, K], fp32 [M])."""
    _matrix(x, "x", torch.bfloat16)
    M, K = x.shape
    x = _rows_aligned(x, 8)
    xq = _fp8_codes(M, K, x.device) if xq is None else xq
    xs = torch.empty((M,), dtype=torch.float32, device=x.device) if xs is None else xs
    _matrix(xq, "xq", torch.uint8)
    if xq.shape != (M, K):
        raise ValueError(f"xq must have shape {(M, K)}")
    _vector(xs, M, "xs", torch.float32)
    _same_device(x, xq, xs)
    with torch.cuda.device(x.device):
        call("fp8_quant_per_token", x.data_ptr(), M, K, _ld(x), xq.data_ptr(), _ld(xq),
             xs.data_ptr(), _stream(x))
    return xq, xs


def fp8_quant_per_channel(w: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-output-channel e4m3 quantization of fp32 w [N, K] -> (uint8 [N, K], fp32 [N])."""
    _matrix(w, "w", torch.float32)
    N, K = w.shape
    w = _rows_aligned(w, 4)
    wq = _fp8_codes(N, K, w.device)
    ws = torch.empty((N,), dtype=torch.float32, device=w.device)
    with torch.cuda.device(w.device):
        call("fp8_quant_per_channel", w.data_ptr(), N, K, _ld(w), wq.data_ptr(), _ld(wq),
             ws.data_ptr(), _stream(w))
    return wq, ws


def fp8_quant_prepack_weight(w: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Online e4m3 quantization of a bf16 or fp32 weight [N, K] into the packed layout."""
    if w.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"w must be bfloat16 or float32, got {w.dtype}")
    _matrix(w, "w", w.dtype)
    N, K = w.shape
    f32 = w.dtype == torch.float32
    w = _rows_aligned(w, 4 if f32 else 8)
    packed = torch.empty((prepack_weight_bytes(N, K),), dtype=torch.uint8, device=w.device)
    ws = torch.empty((N,), dtype=torch.float32, device=w.device)
    with torch.cuda.device(w.device):
        call("fp8_quant_prepack_weight", w.data_ptr(), 0 if f32 else 1, N, K, _ld(w),
             packed.data_ptr(), ws.data_ptr(), _stream(w))
    return packed, ws


def fp8_scaled_mm(xq: torch.Tensor, xs: Optional[torch.Tensor], w_packed: torch.Tensor,
                  ws: Optional[torch.Tensor], N: int, bias: Optional[torch.Tensor] = None,
                  out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
                  tile: int = -1) -> torch.Tensor:
    """The e4m3 twin of scaled_mm: xq uint8 e4m3 codes; out_dtype bf16 or fp16 (bias
    of that type), or float32 for the raw fp32 accumulators."""
    _matrix(xq, "xq", torch.uint8)
    M, K = xq.shape
    if out_dtype not in _FP8_OUT_MODE:
        raise TypeError("out_dtype must be torch.bfloat16, torch.float16 or torch.float32")
    mode = _FP8_OUT_MODE[out_dtype]
    if mode != W8A8_OUT_I32:
        _vector(xs, M, "xs", torch.float32)
        _vector(ws, N, "ws", torch.float32)
        _vector(bias, N, "bias", out_dtype)
    _packed(w_packed, N, K)
    out = torch.empty((M, N), dtype=out_dtype, device=xq.device) if out is None else out
    _matrix(out, "out", out_dtype)
    if out.shape != (M, N):
        raise ValueError(f"out must have shape {(M, N)}")

    def ptr(t):
        return None if t is None or mode == W8A8_OUT_I32 else t.data_ptr()

    _same_device(xq, w_packed, out, *((xs, ws, bias) if mode != W8A8_OUT_I32 else ()))
    with torch.cuda.device(xq.device):
        call("fp8_scaled_mm_tile", xq.data_ptr(), _ld(xq), ptr(xs), w_packed.data_ptr(), ptr(ws),
             ptr(bias), M, N, K, mode, out.data_ptr(), _ld(out), _stream(xq), tile)
    return out


def fp8_quant_scaled_mm(x: torch.Tensor, w_packed: torch.Tensor, ws: Optional[torch.Tensor],
                        N: int, bias: Optional[torch.Tensor] = None,
                        out_dtype: torch.dtype = torch.bfloat16,
                        out: Optional[torch.Tensor] = None, tile: int = -1,
                        xq: Optional[torch.Tensor] = None, xs: Optional[torch.Tensor] = None
                        ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """e4m3 per-token quant of bf16 x and the e4m3 scaled matmul: (out, xq, xs).
    out_dtype bf16 or fp16, or float32 for the raw fp32 accumulators."""
    _matrix(x, "x", torch.bfloat16)
    M, K = x.shape
    x = _rows_aligned(x, 8)
    if out_dtype not in _FP8_OUT_MODE:
        raise TypeError("out_dtype must be torch.bfloat16, torch.float16 or torch.float32")
    mode = _FP8_OUT_MODE[out_dtype]
    if mode != W8A8_OUT_I32:
        _vector(ws, N, "ws", torch.float32)
        _vector(bias, N, "bias", out_dtype)
    _packed(w_packed, N, K)
    xq = _fp8_codes(M, K, x.device) if xq is None else xq
    xs = torch.empty((M,), dtype=torch.float32, device=x.device) if xs is None else xs
    _matrix(xq, "xq", torch.uint8)
    if xq.shape != (M, K):
        raise ValueError(f"xq must have shape {(M, K)}")
    _vector(xs, M, "xs", torch.float32)
    out = torch.empty((M, N), dtype=out_dtype, device=x.device) if out is None else out
    _matrix(out, "out", out_dtype)
    if out.shape != (M, N):
        raise ValueError(f"out must have shape {(M, N)}")

    def ptr(t):
        return None if t is None or mode == W8A8_OUT_I32 else t.data_ptr()

    _same_device(x, w_packed, xq, xs, out, *((ws, bias) if mode != W8A8_OUT_I32 else ()))
    with torch.cuda.device(x.device):
        call("fp8_quant_scaled_mm_tile", x.data_ptr(), _ld(x), xq.data_ptr(), _ld(xq),
             xs.data_ptr(), w_packed.data_ptr(), ptr(ws), ptr(bias), M, N, K, mode,
             out.data_ptr(), _ld(out), _stream(x), tile)
    return out, xq, xs


def fp8_tile_count() -> int:
    return _lib.lib().w8a8_fp8_tile_count()


def tile_count() -> int:
    return _lib.lib().w8a8_mm_tile_count()


def tile_name(tile: int) -> str:
    return _lib.lib().w8a8_mm_tile_name(tile).decode()


def tile_auto(M: int, N: int, K: int) -> int:
    return _lib.lib().w8a8_mm_tile_auto(M, N, K)


def device_supported(device: int = 0) -> bool:
    return bool(_lib.lib().w8a8_device_supported(device))
