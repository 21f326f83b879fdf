"""A seeded sweep of random shapes through every tile and entry point.

Each case draws M, N and K (K a multiple of 16, often not of 64), padded
leading dimensions for the codes and the output, bias or none, and the
value mix of the workloads (normal or GELU rows, outlier columns, per-row
log-uniform magnitudes). Shapes lean towards tile edges: M and N near
multiples of 16, 32, 64, 128 and 192 as well as arbitrary values, and M
of one to four token rows (the small-M kernel and its fused quant).

Per case, against the oracle:
- int8_scaled_mm on every tile: int32 accumulators bit-exact, bf16 outputs
  bit-exact to the fp32 epilogue, nothing written past N in a padded row;
- int8_quant_scaled_mm on every tile: codes and scales bit-exact, outputs
  bit-exact (the single-launch main and small-M paths and the two-launch
  path, whichever the shape takes);
- fp16 output with an fp16 bias on one tile: bit-exact to the oracle's fp16
  epilogue;
- the e4m3 twin on one tile: codes and scales bit-exact, accumulators within
  the measured-precision bound, outputs bit-exact to the epilogue on them.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wl
from tests import test_gpu_fp8 as F
from tests.test_gpu_parity import bf16_dev, bits_np

pytestmark = pytest.mark.gpu

DEV = "cuda"
CASES = 64


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w8a8_int8_dynamic_amd import ops as _ops
    from w8a8_int8_dynamic_amd import _lib
    assert _ops.device_supported(torch.cuda.current_device()), _lib.last_error()
    return _ops


def _edge_size(rng, hi: int) -> int:
    if rng.random() < 0.5:
        base = int(rng.choice([16, 32, 64, 128, 192])) * int(rng.integers(1, 4))
        v = base + int(rng.integers(-1, 2))
    else:
        v = int(rng.integers(1, hi + 1))
    return max(1, min(hi, v))


def _case(i: int):
    rng = np.random.default_rng(20000 + i)
    M = _edge_size(rng, 300) if rng.random() < 0.8 else int(rng.integers(1, 5))   # decode rows too
    N = _edge_size(rng, 420)
    K = 16 * int(rng.integers(1, 76))                      # 16 .. 1200
    ldq = K + 16 * int(rng.integers(0, 3))
    ldo = N + int(rng.integers(0, 5))
    kind = str(rng.choice(["normal", "gelu"]))
    inp = wl.random_case(M, K, N, 21000 + i, x_kind=kind,
                         outlier_frac=float(rng.choice([0.0, 0.01, 0.05])),
                         row_loguniform=bool(rng.random() < 0.5), bias=bool(rng.random() < 0.6))
    return rng, M, N, K, ldq, ldo, inp


def _padded(t: torch.Tensor, ld: int, fill: int) -> torch.Tensor:
    """A view of t's values inside a buffer whose rows are ld long, the rest
    set to `fill` bytes."""
    M, K = t.shape
    raw = torch.full((M, ld * t.element_size()), fill, dtype=torch.uint8, device=DEV)
    big = raw.view(t.dtype)
    big[:, :K] = t
    return big[:, :K]


@pytest.mark.parametrize("i", range(CASES))
def test_sweep_case(ops, orc, i):
    rng, M, N, K, ldq, ldo, inp = _case(i)
    what = f"case {i}: M={M} N={N} K={K} ldq={ldq} ldo={ldo} bias={inp.bias_bf16 is not None}"
    print(what, flush=True)
    wq, ws = orc.quant_per_channel(inp.w_f32)
    xq, xs = orc.quant_per_token(inp.x_bf16)
    acc = orc.gemm_i32(xq, wq)
    ref32 = orc.epilogue_f32(acc, xs, ws, inp.bias_bf16)

    packed = ops.prepack_weight(torch.from_numpy(wq).to(DEV))
    ws_d, xs_d = torch.from_numpy(ws).to(DEV), torch.from_numpy(xs).to(DEV)
    b_d = None if inp.bias_bf16 is None else bf16_dev(inp.bias_bf16)
    xq_d = _padded(torch.from_numpy(xq).to(DEV), ldq, 0x55)
    x_d = bf16_dev(inp.x_bf16)

    for t in range(ops.tile_count()):
        name = f"{what} tile {ops.tile_name(t)}"
        got = ops.scaled_mm(xq_d, None, packed, None, N, out_dtype=torch.int32, tile=t)
        assert np.array_equal(got.cpu().numpy(), acc), name
        out = _padded(torch.zeros((M, N), dtype=torch.bfloat16, device=DEV), ldo, 0xEE)
        ops.scaled_mm(xq_d, xs_d, packed, ws_d, N, b_d, out=out, tile=t)
        full = out.view(torch.int16).as_strided((M, ldo), (ldo, 1)).cpu().numpy().view(np.uint16)
        assert np.array_equal(full[:, :N], ref32), name
        assert np.all(full[:, N:] == 0xEEEE), f"{name}: wrote past N"
        fout, fq, fs = ops.quant_scaled_mm(x_d, packed, ws_d, N, b_d, tile=t)
        assert np.array_equal(fs.cpu().numpy(), xs) and np.array_equal(fq.cpu().numpy(), xq), name
        assert np.array_equal(bits_np(fout), ref32), f"{name} (fused)"

    # fp16 output with an fp16 bias on one tile
    t = int(rng.integers(0, ops.tile_count()))
    b16 = None if inp.bias_bf16 is None else \
        wl.bf16_bits_to_f32(inp.bias_bf16).astype(np.float16).view(np.uint16)
    ref16 = orc.epilogue_f32_f16(acc, xs, ws, b16)
    b16_d = None if b16 is None else torch.from_numpy(b16.view(np.int16)).view(torch.float16).to(DEV)
    out16 = ops.scaled_mm(xq_d, xs_d, packed, ws_d, N, b16_d, out_dtype=torch.float16, tile=t)
    assert np.array_equal(bits_np(out16), ref16), f"{what} fp16 tile {ops.tile_name(t)}"

    # the e4m3 twin on one tile
    t = int(rng.integers(0, ops.fp8_tile_count()))
    wq8, ws8 = orc.fp8_quant_per_channel(inp.w_f32)
    xq8, xs8 = orc.fp8_quant_per_token(inp.x_bf16)
    packed8, ws8_d = ops.fp8_quant_prepack_weight(torch.from_numpy(inp.w_f32).to(DEV))
    assert np.array_equal(ws8_d.cpu().numpy(), ws8), what
    acc8, q8, s8 = ops.fp8_quant_scaled_mm(x_d, packed8, None, N, out_dtype=torch.float32, tile=t)
    assert np.array_equal(q8.cpu().numpy(), xq8) and np.array_equal(s8.cpu().numpy(), xs8), what
    acc8 = acc8.cpu().numpy()
    F.check_acc(orc, acc8, xq8, wq8, orc.fp8_gemm(xq8, wq8), f"{what} fp8 tile {t}")
    own32, _ = orc.fp8_epilogue(acc8.astype(np.float64), xs8, ws8, inp.bias_bf16)
    out8, _, _ = ops.fp8_quant_scaled_mm(x_d, packed8, ws8_d, N, b_d, tile=t)
    assert np.array_equal(bits_np(out8), own32), f"{what} fp8 out tile {t}"
