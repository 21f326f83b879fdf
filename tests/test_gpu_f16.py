"""GPU parity of the fp16 twin: fp16 activations in, fp16 bias and output.

The pages run the layer with bf16 and with fp16 activations (page "Issue 5
probe ...", the isolation table's two activation columns). The HIP path,
through the C ABI, against the oracle's fp16 functions: int8 codes, fp32
scales and int32 accumulators bit-exact; fp16 outputs bit-identical to the
oracle's fixed-order fp32 epilogue rounded to fp16, and within
|g - r| <= 1e-2*|r| + 1e-4*rms(r[m,:]) of its fp64 epilogue.

Inputs: the workloads' seeded values (and the random cases' recipe) rounded
to fp16 nearest-even; all of them lie inside fp16's range.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

RTOL, ATOL_RMS = 1e-2, 1e-4
DEV = "cuda"


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w8a8_int8_dynamic_amd import ops as _ops
    from w8a8_int8_dynamic_amd import _lib
    assert _ops.device_supported(torch.cuda.current_device()), _lib.last_error()
    return _ops


def to_f16_bits(bf16_bits: np.ndarray) -> np.ndarray:
    """fp16 bit patterns of bf16 values (nearest-even)."""
    return wl.bf16_bits_to_f32(bf16_bits).astype(np.float16).view(np.uint16)


def f16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16).to(DEV)


def bits_np(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def f64_16(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def check_out16(got: np.ndarray, ref32: np.ndarray, ref64: np.ndarray, what: str) -> float:
    """Tolerance bar against the fp64 epilogue; returns the bit-exact fraction vs fp32."""
    g, r = f64_16(got), f64_16(ref64)
    assert np.all(np.isfinite(g)) and np.all(np.isfinite(r)), what
    rms = np.sqrt(np.mean(r * r, axis=1, keepdims=True))
    bad = np.abs(g - r) > RTOL * np.abs(r) + ATOL_RMS * rms
    assert not bad.any(), f"{what}: {bad.sum()} outputs outside tolerance"
    return float(np.mean(got == ref32))


def case(M, N, K, seed, bias=True):
    inp = wl.random_case(M, K, N, seed, bias=bias)
    x16 = to_f16_bits(inp.x_bf16)
    b16 = None if inp.bias_bf16 is None else to_f16_bits(inp.bias_bf16)
    return inp, x16, b16


@pytest.mark.parametrize("name", [w.name for w in wl.WORKLOADS])
def test_quant_f16_workload(ops, orc, name):
    x16 = to_f16_bits(wl.generate(wl.by_name(name)).x_bf16)
    xq, xs = ops.quant_per_token(f16_dev(x16))
    q_ref, s_ref = orc.quant_per_token_f16(x16)
    assert np.array_equal(xs.cpu().numpy(), s_ref)
    assert np.array_equal(xq.cpu().numpy(), q_ref)


@pytest.mark.parametrize("M,K,pad", [(1, 1, 0), (3, 7, 9), (65, 200, 0), (130, 1000, 24),
                                     (7, 40000, 0)])
def test_quant_f16_edges(ops, orc, M, K, pad):
    """Ragged K, padded rows, the two-pass kernel (K = 40000), a zero row, a
    row of fp16 subnormals and rows with exact ties."""
    rng = np.random.default_rng(7100 + M + K)
    x = (rng.standard_normal((M, K)) * 10.0 ** rng.uniform(-3, 3, (M, 1))).astype(np.float16)
    if M > 2:
        x[1] = 0
        x[2] = np.float16(3e-7)
        x[2, 0] = np.float16(-6e-8)
    bits = x.view(np.uint16)
    x_big = torch.zeros((M, K + pad), dtype=torch.float16, device=DEV)
    x_big[:, :K] = f16_dev(bits)
    xq, xs = ops.quant_per_token(x_big[:, :K])
    q_ref, s_ref = orc.quant_per_token_f16(bits)
    assert np.array_equal(xs.cpu().numpy(), s_ref)
    assert np.array_equal(xq.cpu().numpy(), q_ref)


SHAPES = [(1, 1, 16), (37, 45, 80), (130, 200, 336), (257, 300, 1040), (5, 1000, 2064)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("bias", [False, True])
def test_scaled_mm_f16_every_tile(ops, orc, M, N, K, bias):
    inp, x16, b16 = case(M, N, K, 7200 + M + N + K, bias)
    wq, ws = orc.quant_per_channel(inp.w_f32)
    xq, xs = orc.quant_per_token_f16(x16)
    acc = orc.gemm_i32(xq, wq)
    ref32 = orc.epilogue_f32_f16(acc, xs, ws, b16)
    ref64 = orc.epilogue_f64_f16(acc, xs, ws, b16)
    packed = ops.prepack_weight(torch.from_numpy(wq).to(DEV))
    xq_d, xs_d = torch.from_numpy(xq).to(DEV), torch.from_numpy(xs).to(DEV)
    ws_d = torch.from_numpy(ws).to(DEV)
    b_d = None if b16 is None else f16_dev(b16)
    for t in range(ops.tile_count()):
        out = ops.scaled_mm(xq_d, xs_d, packed, ws_d, N, b_d, out_dtype=torch.float16, tile=t)
        assert out.dtype == torch.float16
        exact = check_out16(bits_np(out), ref32, ref64, f"tile {ops.tile_name(t)}")
        assert exact == 1.0, f"tile {ops.tile_name(t)}: {exact:.6f} bit-exact vs fp32 epilogue"


QMM_SHAPES = [(1, 48, 64), (2, 1000, 4112), (37, 45, 80), (257, 300, 1040), (512, 520, 576),
              (64, 128, 256)]


@pytest.mark.parametrize("M,N,K", QMM_SHAPES)
@pytest.mark.parametrize("bias", [False, True])
def test_quant_scaled_mm_f16_every_tile(ops, orc, M, N, K, bias):
    """fp16 x through int8_quant_scaled_mm_f16 for every tile (single-launch
    main and small-M paths and the two-launch fallback), twice per tile: fp16
    out bit-exact to the oracle, codes and scales too; int32 out exact."""
    inp, x16, b16 = case(M, N, K, 7300 + M + N + K, bias)
    x = f16_dev(x16)
    wq, ws_ref = orc.quant_per_channel(inp.w_f32)
    packed = ops.prepack_weight(torch.from_numpy(wq).to(DEV))
    ws = torch.from_numpy(ws_ref).to(DEV)
    b = None if b16 is None else f16_dev(b16)
    xq_ref, xs_ref = orc.quant_per_token_f16(x16)
    acc = orc.gemm_i32(xq_ref, wq)
    ref32 = orc.epilogue_f32_f16(acc, xs_ref, ws_ref, b16)
    ref64 = orc.epilogue_f64_f16(acc, xs_ref, ws_ref, b16)
    for t in range(ops.tile_count()):
        for _ in range(2):
            out, xq, xs = ops.quant_scaled_mm(x, packed, ws, N, b, tile=t)
            torch.cuda.synchronize()
            assert out.dtype == torch.float16
            assert np.array_equal(xs.cpu().numpy(), xs_ref), ops.tile_name(t)
            assert np.array_equal(xq.cpu().numpy(), xq_ref), ops.tile_name(t)
            exact = check_out16(bits_np(out), ref32, ref64, f"fused f16 {ops.tile_name(t)}")
            assert exact == 1.0, ops.tile_name(t)
        got, _, _ = ops.quant_scaled_mm(x, packed, None, N, out_dtype=torch.int32, tile=t)
        assert np.array_equal(got.cpu().numpy(), acc), ops.tile_name(t)


def test_quant_scaled_mm_mixed_types(ops, orc):
    """fp16 activations with bf16 output, and bf16 activations with fp16
    output: each quantizes in the activation's type and rounds the output to
    its own (two launches); results match the oracle's pairing."""
    M, N, K = 70, 300, 576
    inp, x16, b16 = case(M, N, K, 7400)
    wq, ws_ref = orc.quant_per_channel(inp.w_f32)
    packed = ops.prepack_weight(torch.from_numpy(wq).to(DEV))
    ws = torch.from_numpy(ws_ref).to(DEV)
    # fp16 in, bf16 out (bf16 bias)
    xq_ref, xs_ref = orc.quant_per_token_f16(x16)
    acc = orc.gemm_i32(xq_ref, wq)
    out, xq, xs = ops.quant_scaled_mm(f16_dev(x16), packed, ws, N,
                                      torch.from_numpy(inp.bias_bf16.view(np.int16)).view(
                                          torch.bfloat16).to(DEV), out_dtype=torch.bfloat16)
    assert np.array_equal(xq.cpu().numpy(), xq_ref) and np.array_equal(xs.cpu().numpy(), xs_ref)
    assert np.array_equal(bits_np(out), orc.epilogue_f32(acc, xs_ref, ws_ref, inp.bias_bf16))
    # bf16 in, fp16 out (fp16 bias)
    xq_ref, xs_ref = orc.quant_per_token(inp.x_bf16)
    acc = orc.gemm_i32(xq_ref, wq)
    x_bf = torch.from_numpy(inp.x_bf16.view(np.int16)).view(torch.bfloat16).to(DEV)
    out, xq, xs = ops.quant_scaled_mm(x_bf, packed, ws, N, f16_dev(b16), out_dtype=torch.float16)
    assert np.array_equal(xq.cpu().numpy(), xq_ref) and np.array_equal(xs.cpu().numpy(), xs_ref)
    assert np.array_equal(bits_np(out), orc.epilogue_f32_f16(acc, xs_ref, ws_ref, b16))


def test_linear_f16(ops, orc):
    """W8A8Linear on fp16 activations: fp16 out with the bias rounded to
    fp16, leading dimensions kept, bit-identical to the oracle."""
    from w8a8_int8_dynamic_amd import W8A8Linear
    N, K = 200, 320
    inp, x16, b16 = case(2 * 37, N, K, 7500)
    bias_f32 = wl.bf16_bits_to_f32(inp.bias_bf16)
    layer = W8A8Linear.from_float(torch.from_numpy(inp.w_f32).to(DEV),
                                  torch.from_numpy(bias_f32).to(DEV))
    x = f16_dev(x16).view(2, 37, K)
    out = layer(x)
    assert out.shape == (2, 37, N) and out.dtype == torch.float16
    wq, ws = orc.quant_per_channel(inp.w_f32)
    xq, xs = orc.quant_per_token_f16(x16)
    ref = orc.epilogue_f32_f16(orc.gemm_i32(xq, wq), xs, ws, b16)
    assert np.array_equal(bits_np(out).reshape(2 * 37, N), ref)


def test_fused_qkv_full_size_f16(ops, orc):
    """The fused-QKV workload at full size in fp16: codes and scales exact,
    sampled rows bit-exact to the fp32 epilogue."""
    w = wl.by_name("fused_qkv")
    inp = wl.generate(w)
    x16 = to_f16_bits(inp.x_bf16)
    b16 = None if inp.bias_bf16 is None else to_f16_bits(inp.bias_bf16)
    wq, ws_ref = orc.quant_per_channel(inp.w_f32)
    packed = ops.prepack_weight(torch.from_numpy(wq).to(DEV))
    out, xq, xs = ops.quant_scaled_mm(f16_dev(x16), packed, torch.from_numpy(ws_ref).to(DEV), w.N,
                                      None if b16 is None else f16_dev(b16))
    xq_ref, xs_ref = orc.quant_per_token_f16(x16)
    assert np.array_equal(xq.cpu().numpy(), xq_ref) and np.array_equal(xs.cpu().numpy(), xs_ref)
    rows = np.unique(np.concatenate([np.random.default_rng(w.seed).choice(w.M, 40, replace=False),
                                     [0, w.M - 1]])).astype(np.int64)
    acc = orc.gemm_i32(xq_ref, wq, rows)
    ref32 = orc.epilogue_f32_f16(acc, xs_ref[rows], ws_ref, b16)
    ref64 = orc.epilogue_f64_f16(acc, xs_ref[rows], ws_ref, b16)
    exact = check_out16(bits_np(out)[rows], ref32, ref64, "fused_qkv f16")
    assert exact == 1.0


def test_f16_output_range_edges(ops, orc):
    """fp16 outputs across the whole range on every tile: row scales from
    1e-14 to 1e4 put outputs in fp16's subnormal range, around its largest
    finite value and past it (infinity from 65520). Bit-exact to the
    oracle's fp16 epilogue, infinities and signed zeros included."""
    M, N, K = 80, 136, 320
    rng = np.random.default_rng(8800)
    xq = rng.integers(-127, 128, (M, K), dtype=np.int8)
    wq = rng.integers(-127, 128, (N, K), dtype=np.int8)
    xs = (10.0 ** np.linspace(-14, 4, M)).astype(np.float32)
    ws = (rng.uniform(0.5, 2.0, N) * 1e-2).astype(np.float32)
    bias = np.where(np.arange(N) % 3 == 0, 0.0, rng.standard_normal(N) * 1e-6).astype(np.float16)
    b16 = bias.view(np.uint16)
    acc = orc.gemm_i32(xq, wq)
    ref = orc.epilogue_f32_f16(acc, xs, ws, b16)
    assert np.isinf(ref.view(np.float16)).any()              # the cases are there
    assert ((ref & 0x7C00) == 0).any() and ((ref & 0x03FF) != 0).any()
    xq_d = torch.from_numpy(xq).to(DEV)
    packed = ops.prepack_weight(torch.from_numpy(wq).to(DEV))
    xs_d, ws_d = torch.from_numpy(xs).to(DEV), torch.from_numpy(ws).to(DEV)
    b_d = torch.from_numpy(bias).to(DEV)
    for t in range(ops.tile_count()):
        out = ops.scaled_mm(xq_d, xs_d, packed, ws_d, N, b_d, out_dtype=torch.float16, tile=t)
        assert np.array_equal(bits_np(out), ref), ops.tile_name(t)
