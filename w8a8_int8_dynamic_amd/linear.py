"""W8A8Linear: a linear layer whose forward pass runs the W8A8 int8-dynamic path.

Shape handling follows the page "Diffusion Quantization Reference": its GGUF
rules flatten N-D activations around the matmul and restore the shape, and
its "Common Failures" table lists an output rank collapsing from 3-D to 2-D
as a bug. Inputs [..., K] are viewed as [M, K] (no copy when the last
dimension is contiguous) and outputs come back as [..., N].
"""
from __future__ import annotations

import fnmatch
from typing import Optional, Sequence

import torch

from . import ops

__all__ = ["W8A8Linear", "quantize_linear_layers"]


class W8A8Linear(torch.nn.Module):
    """y = q(x) @ q(W)^T * x_scale * w_scale (+ bias), in x's type.

    scheme "int8" (the default): int8 codes, bf16 or fp16 activations.
    scheme "fp8": the e4m3 twin (page "Online Quantization": FP8 W8A8 with
    dynamic per-token activation scales), bf16 activations.

    Build with ``from_float`` (online per-channel weight quantization on the
    GPU, written straight into the load-time layout) or ``from_quantized``
    (int8 weights and fp32 scales already made offline).
    """

    def __init__(self, w_packed: torch.Tensor, w_scale: torch.Tensor, out_features: int,
                 in_features: int, bias: Optional[torch.Tensor] = None, scheme: str = "int8"):
        super().__init__()
        if scheme not in ("int8", "fp8"):
            raise ValueError(f"scheme must be 'int8' or 'fp8', got {scheme!r}")
        self.scheme = scheme
        self.in_features = in_features
        self.out_features = out_features
        self.register_buffer("w_packed", w_packed)
        self.register_buffer("w_scale", w_scale)
        # The bias in each output type, rounded once from what was given.
        self.register_buffer("bias", None if bias is None else bias.to(torch.bfloat16).contiguous())
        self.register_buffer("bias_f16", None if bias is None else bias.to(torch.float16).contiguous())
        # The layer's own workspace for decode-shaped calls (a handful of
        # tokens against a weight with few column blocks), allocated once
        # here so that forward never allocates it.
        self.register_buffer(
            "workspace",
            ops.new_workspace(out_features, in_features, device=w_packed.device)
            if scheme == "int8" and w_packed.is_cuda else None,
            persistent=False)

    @classmethod
    def from_quantized(cls, wq: torch.Tensor, w_scale: torch.Tensor,
                       bias: Optional[torch.Tensor] = None) -> "W8A8Linear":
        N, K = wq.shape
        if not torch.isfinite(w_scale).all():
            raise ValueError("weight scales must be finite")
        packed = ops.prepack_weight(wq.contiguous())
        return cls(packed, w_scale.to(torch.float32).contiguous(), N, K, bias)

    @classmethod
    def from_float(cls, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
                   scheme: str = "int8") -> "W8A8Linear":
        """bf16 and fp32 weights are quantized as they are. Other float types
        are converted to fp32 first: exact for fp16, rounded for fp64 (the
        quant rule works on fp32 values)."""
        w = weight if weight.dtype in (torch.bfloat16, torch.float32) else weight.to(torch.float32)
        N, K = w.shape
        quant = ops.fp8_quant_prepack_weight if scheme == "fp8" else ops.quant_prepack_weight
        packed, ws = quant(w.contiguous())
        if not torch.isfinite(ws).all():
            raise ValueError("weight scales must be finite")
        return cls(packed, ws, N, K, bias, scheme)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.shape[-1] != self.in_features:
            raise ValueError(f"expected last dimension {self.in_features}, got {x.shape[-1]}")
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features)
        if x2.stride(-1) != 1:
            x2 = x2.contiguous()
        # The per-token quant and the scaled matmul, as one library call; the
        # output (and bias) type is x's.
        bias = self.bias_f16 if x2.dtype == torch.float16 else self.bias
        if self.scheme == "fp8":
            if x2.dtype != torch.bfloat16:
                raise TypeError(f"the fp8 scheme takes bfloat16 activations, got {x2.dtype}")
            out, _, _ = ops.fp8_quant_scaled_mm(x2, self.w_packed, self.w_scale,
                                                self.out_features, bias)
        else:
            wsp = self.workspace if x2.dtype == torch.bfloat16 else None
            out, _, _ = ops.quant_scaled_mm(x2, self.w_packed, self.w_scale, self.out_features,
                                            bias, workspace=wsp)
        return out.reshape(*lead, self.out_features)

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"bias={self.bias is not None}, scheme={self.scheme}")


def quantize_linear_layers(module: torch.nn.Module, method: str = "int8",
                           activation_scheme: str = "dynamic",
                           ignored_layers: Sequence[str] = ()) -> torch.nn.Module:
    """Replace the torch.nn.Linear layers of `module` by W8A8Linear layers.

    The selection follows the page "Online Quantization" (Parameters table):
    `method` is "int8" or "fp8"; `activation_scheme` must be "dynamic"
    (activation scales computed per token at run time, the only scheme
    implemented); `ignored_layers` holds name patterns of layers to keep in
    their float type. A layer is kept when its qualified name (as in
    module.named_modules()) matches a pattern by fnmatch or contains it.
    Weights are quantized online on their device (W8A8Linear.from_float).
    Anything the path cannot run raises ValueError naming the layer: a layer
    on the CPU, or in_features not a multiple of 16. Returns `module`, or the
    replacement when `module` is itself a Linear."""
    if method not in ("int8", "fp8"):
        raise ValueError(f"method must be 'int8' or 'fp8', got {method!r}")
    if activation_scheme != "dynamic":
        raise ValueError(f"only activation_scheme='dynamic' is implemented, got {activation_scheme!r}")
    patterns = [p for p in ignored_layers if p]

    def kept(name: str) -> bool:
        return any(fnmatch.fnmatchcase(name, p) or p in name for p in patterns)

    def convert(name: str, lin: torch.nn.Linear) -> W8A8Linear:
        if not lin.weight.is_cuda:
            raise ValueError(f"layer {name!r} is on {lin.weight.device}; move the model to the GPU first")
        if lin.in_features % 16 != 0:
            raise ValueError(f"layer {name!r}: in_features {lin.in_features} is not a multiple of 16")
        bias = None if lin.bias is None else lin.bias.detach()
        return W8A8Linear.from_float(lin.weight.detach(), bias, scheme=method)

    if isinstance(module, torch.nn.Linear):
        return module if kept("") else convert("", module)
    for parent_name, parent in list(module.named_modules()):
        for child_name, child in list(parent.named_children()):
            name = f"{parent_name}.{child_name}" if parent_name else child_name
            if isinstance(child, torch.nn.Linear) and not kept(name):
                setattr(parent, child_name, convert(name, child))
    return module
