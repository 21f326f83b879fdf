"""Seeded synthetic inputs for W8A8 int8-dynamic linear layers.

This module only draws random numbers. It holds none of the method's
arithmetic (no absmax, no scales, no quantization, no matmul), so both the
CPU oracle and the GPU path can take their inputs from here without sharing
any step of the computation.

The five workloads mirror the layer geometries measured on the page
"Issue 5 probe: int8 quantized DiT serve paths on the RTX 3090 (24 GB)":
the three raw-op shapes of its "Round two" kernel-path verification
paragraph, and the attention out-projection, fused QKV, FFN-up and FFN-down
rows of its "Kernel isolation" table.

Recipe (fixed, so a result record can name it):

* RNG: ``numpy.random.default_rng(seed)`` (PCG64).
* Draw order: X, outlier columns, per-row magnitudes, W, bias.
* X is drawn in float32, post-processed, then rounded to bfloat16 (RNE) and
  returned as raw ``uint16`` bit patterns.
* "1 % of columns" means ``round(0.01 * K)`` distinct columns drawn without
  replacement; each is multiplied by the outlier factor.
* "per-row magnitudes log-uniform in [0.1, 10]" means row m is multiplied by
  ``10 ** U(-1, 1)``.
* GELU is the exact erf form.
* ``N(0, s)`` means standard deviation ``s``.
* W is float32 ``[N, K]`` (out x in, the layer computes ``x @ W^T``); it is
  quantized per output channel by whichever side consumes it.
* Bias, when present, is ``bf16(0.01 * N(0, 1))`` of length N.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "by_name", "generate", "Inputs",
           "f32_to_bf16_bits", "bf16_bits_to_f32", "random_case"]


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    seed: int
    x_kind: str             # "normal" | "gelu"
    outlier_cols: int       # number of outlier columns (0 = none)
    outlier_factor: float
    row_loguniform: bool    # per-row magnitudes 10**U(-1,1)
    w_sigma: float
    w_blocks: int           # W drawn as this many stacked [N/blocks, K] blocks
    bias: bool
    description: str

    @property
    def ops(self) -> int:
        """Integer multiply-adds counted as 2 ops each: 2*M*N*K."""
        return 2 * self.M * self.N * self.K


WORKLOADS = (
    Workload("tiny", 64, 256, 128, 2301, "normal", 2, 20.0, False, 0.02, 1, False,
             "tiny W8A8 linear M64 K256 N128"),
    Workload("attn_out", 512, 4096, 4096, 2302, "normal", 41, 30.0, False, 0.02, 1, True,
             "DiT attention out-projection M512 K4096 N4096"),
    Workload("fused_qkv", 512, 4096, 12288, 2303, "normal", 41, 30.0, False, 0.02, 3, False,
             "fused-QKV W8A8 linear M512 K4096 N12288"),
    Workload("ffn_up", 4096, 3072, 12288, 2304, "normal", 0, 1.0, True, 0.02, 1, True,
             "DiT FFN up-projection M4096 K3072 N12288"),
    Workload("ffn_down", 8192, 12288, 3072, 2305, "gelu", 0, 1.0, True, 0.01, 1, False,
             "DiT FFN down-projection M8192 K12288 N3072"),
)


def by_name(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(f"unknown workload {name!r}; known: {[w.name for w in WORKLOADS]}")


@dataclass
class Inputs:
    x_bf16: np.ndarray            # uint16 [M, K] bf16 bit patterns
    w_f32: np.ndarray             # float32 [N, K]
    bias_bf16: Optional[np.ndarray]  # uint16 [N] or None
    outlier_cols: np.ndarray      # int64 indices (may be empty)
    row_mag: Optional[np.ndarray]  # float32 [M] or None


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even) via torch's CPU cast.

    Used only to shape synthetic inputs; returns uint16 bit patterns.
    """
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _gelu_erf(x: np.ndarray) -> np.ndarray:
    import torch
    return torch.nn.functional.gelu(torch.from_numpy(x), approximate="none").numpy()


def _draw(rng: np.random.Generator, M: int, K: int, N: int, x_kind: str,
          outlier_cols: int, outlier_factor: float, row_loguniform: bool,
          w_sigma: float, w_blocks: int, bias: bool) -> Inputs:
    x = rng.standard_normal((M, K), dtype=np.float32)
    if x_kind == "gelu":
        x = _gelu_erf(x)
    elif x_kind != "normal":
        raise ValueError(x_kind)
    cols = np.zeros(0, dtype=np.int64)
    if outlier_cols:
        cols = np.sort(rng.choice(K, size=outlier_cols, replace=False)).astype(np.int64)
        x[:, cols] *= np.float32(outlier_factor)
    mag = None
    if row_loguniform:
        mag = (10.0 ** rng.uniform(-1.0, 1.0, size=M)).astype(np.float32)
        x *= mag[:, None]
    if N % w_blocks:
        raise ValueError("N must split into w_blocks equal blocks")
    nb = N // w_blocks
    w = np.concatenate([rng.standard_normal((nb, K), dtype=np.float32) for _ in range(w_blocks)],
                       axis=0)
    w *= np.float32(w_sigma)
    b = None
    if bias:
        b = f32_to_bf16_bits(np.float32(0.01) * rng.standard_normal(N, dtype=np.float32))
    return Inputs(f32_to_bf16_bits(x), np.ascontiguousarray(w), b, cols, mag)


def generate(w: Workload, seed: Optional[int] = None) -> Inputs:
    """Draw the inputs of workload ``w`` (its own seed unless one is given)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    return _draw(rng, w.M, w.K, w.N, w.x_kind, w.outlier_cols, w.outlier_factor,
                 w.row_loguniform, w.w_sigma, w.w_blocks, w.bias)


def random_case(M: int, K: int, N: int, seed: int, *, x_kind: str = "normal",
                outlier_frac: float = 0.01, outlier_factor: float = 30.0,
                row_loguniform: bool = False, w_sigma: float = 0.02,
                bias: bool = True) -> Inputs:
    """A smaller case with the same value distributions, for parity tests."""
    rng = np.random.default_rng(seed)
    n_out = int(round(outlier_frac * K)) if outlier_frac else 0
    return _draw(rng, M, K, N, x_kind, n_out, outlier_factor, row_loguniform,
                 w_sigma, 1, bias)
