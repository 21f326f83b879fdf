"""GPU parity of the FP8 (e4m3) W8A8 twin against the oracle's e4m3 functions.

Bar: e4m3 codes, fp32 scales and packed bytes bit-exact. The fp32
accumulators of the fp8 MFMA are not exact sums: measured on MI355X, the
MFMA sums each 64-product k-block to about 12 bits relative to the block's
largest product (error up to 2^-11.4 of it, never zero on random codes),
then adds the block sums in fp32. So they are checked against the oracle's
exact sums within
  |acc - exact| <= 2^-9 * sum_blocks max|x| * max|w|  +  (K/64 + 4) * 2^-23 * sum_k |x_k w_k|
(the per-block maxima taken over each 64-element block of the row and the
column: four times and more the measured error, and far below the error of
a wrong operand layout, which is of the order of the sum itself). The 16-bit outputs
must equal the epilogue applied to the GPU's own accumulators bit for bit
(the raw-accumulator mode returns them), and lie within
|g - r| <= 1e-2*|r| + 1e-4*rms(r[m,:]) + xs*ws*bound of the fp64 epilogue on
the exact sums (the last term carries the accumulator bound through the
scales).

Inputs follow the workloads' recipe (seeded; bf16 activations, fp32
weights).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wl
from tests.test_gpu_parity import packed_reference

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


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def bits_np(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def f64(bits: np.ndarray) -> np.ndarray:
    return wl.bf16_bits_to_f32(bits).astype(np.float64)


_E4M3 = None


def dec(orc, codes: np.ndarray) -> np.ndarray:
    global _E4M3
    if _E4M3 is None:
        _E4M3 = np.array([orc.e4m3_to_double(c) for c in range(256)])
    return _E4M3[codes]


def _block_max(v: np.ndarray) -> np.ndarray:
    """max |v| over each 64-element k-block of each row (zero-padded)."""
    R, K = v.shape
    nb = (K + 63) // 64
    p = np.zeros((R, nb * 64))
    p[:, :K] = np.abs(v)
    return p.reshape(R, nb, 64).max(-1)


def check_acc(orc, got, xq, wq, exact, what):
    K = xq.shape[1]
    a, w = dec(orc, xq), dec(orc, wq)
    S = np.abs(a) @ np.abs(w).T
    bound = 2.0 ** -9 * (_block_max(a) @ _block_max(w).T) + (K / 64 + 4) * 2.0 ** -23 * S
    err = np.abs(got.astype(np.float64) - exact)
    assert np.all(err <= bound), f"{what}: {int((err > bound).sum())} accumulators outside the bound"
    return bound


def check_out(got, ref64, what, acc_slack=0.0):
    """Tolerance against the fp64 epilogue on exact sums; acc_slack is the
    accumulator bound carried through the scales (xs * ws * bound)."""
    g, r = f64(got), f64(ref64)
    assert np.all(np.isfinite(g)), what
    rms = np.sqrt(np.mean(r * r, axis=1, keepdims=True))
    bad = np.abs(g - r) > RTOL * np.abs(r) + ATOL_RMS * rms + acc_slack
    assert not bad.any(), f"{what}: {bad.sum()} outputs outside tolerance"


@pytest.mark.parametrize("name", [w.name for w in wl.WORKLOADS])
def test_fp8_quant_per_token_workload(ops, orc, name):
    inp = wl.generate(wl.by_name(name))
    xq, xs = ops.fp8_quant_per_token(bf16_dev(inp.x_bf16))
    q_ref, s_ref = orc.fp8_quant_per_token(inp.x_bf16)
    assert np.array_equal(xs.cpu().numpy(), s_ref)
    assert np.array_equal(xq.cpu().numpy(), q_ref)


def test_fp8_quant_edges(ops, orc):
    """Rows built to land x*inv on e4m3 ties, subnormal codes, signed zeros,
    fp32-subnormal products and the 448 edge; ragged K; the two-pass kernel
    (K = 40000)."""
    rng = np.random.default_rng(8100)
    rows = []
    # absmax 448 -> inv = 1: the row's values are scaled codes directly
    ties = np.array([448.0, 1.0 + 2 ** -4, 1.0 + 3 * 2 ** -4, -(1.0 + 2 ** -4), 2 ** -10,
                     3 * 2 ** -10, -2 ** -11, 2 ** -6 - 2 ** -10, 447.0, 440.0, 0.0, -0.0],
                    np.float32)
    rows.append(np.resize(ties, 50))
    rows.append(np.resize(-ties, 50))
    rows.append(np.zeros(50, np.float32))
    rows.append((rng.standard_normal(50) * 1e-3).astype(np.float32))
    # absmax near the bf16 maximum: small entries give fp32-subnormal x*inv
    # (codes +-0, sign kept) next to ordinary codes
    rows.append(np.resize(np.array([3e38, -1e-3, 1e-3, -1e-36, 2e-36, -3e35, 1e35, 0.0],
                                   np.float32), 50))
    x = wl.f32_to_bf16_bits(np.stack(rows))
    for arr in (x, wl.f32_to_bf16_bits((rng.standard_normal((7, 40000)) * 3).astype(np.float32)),
                wl.f32_to_bf16_bits((rng.standard_normal((65, 200)) * 10).astype(np.float32))):
        xq, xs = ops.fp8_quant_per_token(bf16_dev(arr))
        q_ref, s_ref = orc.fp8_quant_per_token(arr)
        assert np.array_equal(xs.cpu().numpy(), s_ref)
        assert np.array_equal(xq.cpu().numpy(), q_ref)


@pytest.mark.parametrize("N,K", [(1, 1), (17, 65), (40, 200), (256, 4096)])
def test_fp8_weight_quant_and_prepack(ops, orc, N, K):
    rng = np.random.default_rng(8200 + N + K)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    if N > 3:
        w[1] = 0
        w[2] = 1e-32
    wq_ref, ws_ref = orc.fp8_quant_per_channel(w)
    wq, ws = ops.fp8_quant_per_channel(torch.from_numpy(w).to(DEV))
    assert np.array_equal(ws.cpu().numpy(), ws_ref) and np.array_equal(wq.cpu().numpy(), wq_ref)
    for dt in (torch.float32, torch.bfloat16):
        w_d = torch.from_numpy(w).to(DEV).to(dt)
        q_ref, s_ref = orc.fp8_quant_per_channel(w_d.to(torch.float32).cpu().numpy())
        packed, s = ops.fp8_quant_prepack_weight(w_d)
        assert np.array_equal(s.cpu().numpy(), s_ref)
        assert np.array_equal(packed.cpu().numpy(), packed_reference(q_ref.view(np.int8)))


SHAPES = [(1, 1, 16), (37, 45, 80), (130, 200, 336), (257, 300, 1040), (300, 520, 4096)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("bias", [False, True])
def test_fp8_scaled_mm_every_tile(ops, orc, M, N, K, bias):
    inp = wl.random_case(M, K, N, 8300 + M + N + K, bias=bias)
    wq, ws = orc.fp8_quant_per_channel(inp.w_f32)
    xq, xs = orc.fp8_quant_per_token(inp.x_bf16)
    exact = orc.fp8_gemm(xq, wq)
    _, ref64 = orc.fp8_epilogue(exact, xs, ws, inp.bias_bf16)
    packed = ops.prepack_weight(torch.from_numpy(wq.view(np.int8)).to(DEV))
    xq_d, xs_d, ws_d = (torch.from_numpy(a).to(DEV) for a in (xq, xs, ws))
    b_d = None if inp.bias_bf16 is None else bf16_dev(inp.bias_bf16)
    for t in range(ops.fp8_tile_count()):
        name = ops.tile_name(t)
        acc = ops.fp8_scaled_mm(xq_d, None, packed, None, N, out_dtype=torch.float32, tile=t)
        acc = acc.cpu().numpy()
        bound = check_acc(orc, acc, xq, wq, exact, name)
        out = ops.fp8_scaled_mm(xq_d, xs_d, packed, ws_d, N, b_d, tile=t)
        own32, _ = orc.fp8_epilogue(acc.astype(np.float64), xs, ws, inp.bias_bf16)
        assert np.array_equal(bits_np(out), own32), f"{name}: epilogue differs on its own sums"
        check_out(bits_np(out), ref64, name, xs.astype(np.float64)[:, None] * ws[None, :] * bound)


def test_fp8_quant_scaled_mm_and_f16_out(ops, orc):
    M, N, K = 200, 384, 1024
    inp = wl.random_case(M, K, N, 8400, bias=True)
    wq, ws_ref = orc.fp8_quant_per_channel(inp.w_f32)
    packed, ws = ops.fp8_quant_prepack_weight(torch.from_numpy(inp.w_f32).to(DEV))
    assert np.array_equal(ws.cpu().numpy(), ws_ref)
    out, xq, xs = ops.fp8_quant_scaled_mm(bf16_dev(inp.x_bf16), packed, ws, N,
                                          bf16_dev(inp.bias_bf16))
    xq_ref, xs_ref = orc.fp8_quant_per_token(inp.x_bf16)
    assert np.array_equal(xq.cpu().numpy(), xq_ref) and np.array_equal(xs.cpu().numpy(), xs_ref)
    exact = orc.fp8_gemm(xq_ref, wq)
    _, ref64 = orc.fp8_epilogue(exact, xs_ref, ws_ref, inp.bias_bf16)
    acc = ops.fp8_scaled_mm(xq, None, packed, None, N, out_dtype=torch.float32).cpu().numpy()
    bound = check_acc(orc, acc, xq_ref, wq, exact, "fp8_quant_scaled_mm")
    check_out(bits_np(out), ref64, "fp8_quant_scaled_mm",
              xs_ref.astype(np.float64)[:, None] * ws_ref[None, :] * bound)
    # fp16 output: the GPU's own fp32 sums through the oracle's fp16 epilogue
    b16 = wl.bf16_bits_to_f32(inp.bias_bf16).astype(np.float16).view(np.uint16)
    out16 = ops.fp8_scaled_mm(xq, xs, packed, ws, N,
                              torch.from_numpy(b16.view(np.int16)).view(torch.float16).to(DEV),
                              out_dtype=torch.float16)
    own16, _ = orc.fp8_epilogue(acc.astype(np.float64), xs_ref, ws_ref, b16, f16=True)
    assert np.array_equal(bits_np(out16), own16)


QMM_SHAPES = [(1, 48, 64), (2, 1000, 4112), (37, 45, 80), (257, 300, 1040), (512, 1536, 512)]


@pytest.mark.parametrize("M,N,K", QMM_SHAPES)
def test_fp8_quant_scaled_mm_every_tile(ops, orc, M, N, K):
    """fp8_quant_scaled_mm for every tile (the single-launch main and small-M
    paths with e4m3 producers, and the two-launch fallback), twice per tile:
    codes and scales bit-exact, raw accumulators within the bound, bf16
    outputs bit-exact to the epilogue on those accumulators."""
    inp = wl.random_case(M, K, N, 8500 + M + N + K, bias=True)
    x = bf16_dev(inp.x_bf16)
    wq, ws_ref = orc.fp8_quant_per_channel(inp.w_f32)
    packed, ws = ops.fp8_quant_prepack_weight(torch.from_numpy(inp.w_f32).to(DEV))
    b = bf16_dev(inp.bias_bf16)
    xq_ref, xs_ref = orc.fp8_quant_per_token(inp.x_bf16)
    exact = orc.fp8_gemm(xq_ref, wq)
    for t in range(ops.fp8_tile_count()):
        name = ops.tile_name(t)
        acc, xq, xs = ops.fp8_quant_scaled_mm(x, packed, None, N, out_dtype=torch.float32, tile=t)
        assert np.array_equal(xq.cpu().numpy(), xq_ref) and np.array_equal(xs.cpu().numpy(), xs_ref), name
        acc = acc.cpu().numpy()
        check_acc(orc, acc, xq_ref, wq, exact, name)
        own32, _ = orc.fp8_epilogue(acc.astype(np.float64), xs_ref, ws_ref, inp.bias_bf16)
        for _ in range(2):
            out, xq, xs = ops.fp8_quant_scaled_mm(x, packed, ws, N, b, tile=t)
            torch.cuda.synchronize()
            assert np.array_equal(xq.cpu().numpy(), xq_ref), name
            assert np.array_equal(bits_np(out), own32), name


def test_fp8_quant_scaled_mm_graph_replays_new_inputs(ops, orc):
    """The main-tile fp8_quant_scaled_mm captured in a HIP graph and replayed
    with a different input copied into the captured x before each replay:
    codes and scales bit-exact to the oracle for the input of that replay;
    raw accumulators within the bound; bf16 outputs bit-exact to the
    epilogue on those accumulators."""
    M, N, K = 512, 1536, 512
    inps = [wl.random_case(M, K, N, 8600 + i, bias=True) for i in range(2)]
    wq, ws_ref = orc.fp8_quant_per_channel(inps[0].w_f32)
    packed, ws = ops.fp8_quant_prepack_weight(torch.from_numpy(inps[0].w_f32).to(DEV))
    b = bf16_dev(inps[0].bias_bf16)
    refs = []
    for inp in inps:
        xq_ref, xs_ref = orc.fp8_quant_per_token(inp.x_bf16)
        xq_dev = torch.from_numpy(xq_ref.view(np.uint8)).to(DEV)
        acc = ops.fp8_scaled_mm(xq_dev, None, packed, None, N, out_dtype=torch.float32)
        acc = acc.cpu().numpy()
        check_acc(orc, acc, xq_ref, wq, orc.fp8_gemm(xq_ref, wq), "graph case")
        own32, _ = orc.fp8_epilogue(acc.astype(np.float64), xs_ref, ws_ref, inps[0].bias_bf16)
        refs.append((xq_ref, xs_ref, own32))
    xs_dev = [bf16_dev(inp.x_bf16) for inp in inps]
    x = xs_dev[0].clone()
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ops.fp8_quant_scaled_mm(x, packed, ws, N, b, out=out)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _, xq, xs = ops.fp8_quant_scaled_mm(x, packed, ws, N, b, out=out)
    for i in range(6):
        c = i % 2
        x.copy_(xs_dev[c])
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        xq_ref, xs_ref, own32 = refs[c]
        assert np.array_equal(xs.cpu().numpy(), xs_ref), f"replay {i}"
        assert np.array_equal(xq.cpu().numpy(), xq_ref), f"replay {i}"
        assert np.array_equal(bits_np(out), own32), f"replay {i}"
        ops.fp8_quant_scaled_mm(xs_dev[1 - c], packed, ws, N, b)   # eager call between


def test_fp8_full_size_fused_qkv(ops, orc):
    """The fused-QKV workload at full size through the e4m3 twin: codes and
    scales exact; sampled rows' accumulators within the bound and outputs
    within tolerance."""
    w = wl.by_name("fused_qkv")
    inp = wl.generate(w)
    wq, ws_ref = orc.fp8_quant_per_channel(inp.w_f32)
    packed, ws = ops.fp8_quant_prepack_weight(torch.from_numpy(inp.w_f32).to(DEV))
    x = bf16_dev(inp.x_bf16)
    out, xq, xs = ops.fp8_quant_scaled_mm(x, packed, ws, w.N)
    xq_ref, xs_ref = orc.fp8_quant_per_token(inp.x_bf16)
    assert np.array_equal(xq.cpu().numpy(), xq_ref) and np.array_equal(xs.cpu().numpy(), xs_ref)
    rows = np.unique(np.concatenate([np.random.default_rng(w.seed).choice(w.M, 24, replace=False),
                                     [0, w.M - 1]])).astype(np.int64)
    exact = orc.fp8_gemm(xq_ref, wq, rows)
    acc = ops.fp8_scaled_mm(xq, None, packed, None, w.N, out_dtype=torch.float32).cpu().numpy()
    bound = check_acc(orc, acc[rows], xq_ref[rows], wq, exact, "fused_qkv fp8")
    _, ref64 = orc.fp8_epilogue(exact, xs_ref[rows], ws_ref, inp.bias_bf16)
    check_out(bits_np(out)[rows], ref64, "fused_qkv fp8",
              xs_ref[rows].astype(np.float64)[:, None] * ws_ref[None, :] * bound)


def test_fp8_linear_layer(ops, orc):
    """W8A8Linear with scheme "fp8": the weight quantized online to e4m3, the
    forward equal to fp8_quant_scaled_mm bit for bit and within tolerance of
    the oracle's exact pipeline; leading dimensions kept; fp16 activations
    refused."""
    from w8a8_int8_dynamic_amd import W8A8Linear
    M, N, K = 96, 200, 640
    inp = wl.random_case(M, K, N, 8700, bias=True)
    layer = W8A8Linear.from_float(torch.from_numpy(inp.w_f32).to(DEV), bf16_dev(inp.bias_bf16),
                                  scheme="fp8")
    x = bf16_dev(inp.x_bf16)
    y = layer(x.view(2, M // 2, K))
    assert y.shape == (2, M // 2, N) and y.dtype == torch.bfloat16
    ref, _, _ = ops.fp8_quant_scaled_mm(x, layer.w_packed, layer.w_scale, N, layer.bias)
    assert torch.equal(y.reshape(M, N).view(torch.int16), ref.view(torch.int16))
    wq, ws_ref = orc.fp8_quant_per_channel(inp.w_f32)
    assert np.array_equal(layer.w_scale.cpu().numpy(), ws_ref)
    xq, xs = orc.fp8_quant_per_token(inp.x_bf16)
    exact = orc.fp8_gemm(xq, wq)
    _, ref64 = orc.fp8_epilogue(exact, xs, ws_ref, inp.bias_bf16)
    acc = ops.fp8_scaled_mm(torch.from_numpy(xq).to(DEV), None, layer.w_packed, None, N,
                            out_dtype=torch.float32).cpu().numpy()
    bound = check_acc(orc, acc, xq, wq, exact, "fp8 layer")
    check_out(bits_np(y.reshape(M, N)), ref64, "fp8 layer",
              xs.astype(np.float64)[:, None] * ws_ref[None, :] * bound)
    with pytest.raises(TypeError):
        layer(x.to(torch.float16))
    assert "scheme=fp8" in repr(layer)
