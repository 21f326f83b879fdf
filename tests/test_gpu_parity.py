"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: int8 codes, fp32 scales, prepacked bytes and int32 accumulators are
bit-exact; bf16 outputs satisfy |g - r| <= 1e-2*|r| + 1e-4*rms(r[m,:])
against the oracle's fp64 epilogue, and are expected to equal the oracle's
fixed-order fp32 epilogue bit for bit.

Sizes: small and mid shapes span several tiles with ragged M/N/K tails and
run the oracle in full; the five workload shapes run at full size in the
launch configuration the benchmark times, every element compared.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

RTOL, ATOL_RMS = 1e-2, 1e-4


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w8a8_int8_dynamic_amd import ops as _ops
    from w8a8_int8_dynamic_amd import _lib
    assert _ops.device_supported(torch.cuda.current_device()), _lib.last_error()
    return _ops


DEV = "cuda"


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def bits_np(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def f64(bits: np.ndarray) -> np.ndarray:
    return wl.bf16_bits_to_f32(bits).astype(np.float64)


def check_out(got: np.ndarray, ref32: np.ndarray, ref64: np.ndarray, what: str) -> float:
    """Tolerance bar against the fp64 epilogue; returns the bit-exact fraction vs fp32."""
    g, r = f64(got), f64(ref64)
    assert np.all(np.isfinite(g)), what
    rms = np.sqrt(np.mean(r * r, axis=1, keepdims=True))
    bad = np.abs(g - r) > RTOL * np.abs(r) + ATOL_RMS * rms
    assert not bad.any(), f"{what}: {bad.sum()} outputs outside tolerance"
    return float(np.mean(got == ref32))


def rand_i8(rng, shape, lo=-127):
    return rng.integers(lo, 128, shape, dtype=np.int8)


# ---------------------------------------------------------------------------
# Quantization
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", [w.name for w in wl.WORKLOADS])
def test_quant_per_token_workload(ops, orc, name):
    inp = wl.generate(wl.by_name(name))
    xq, xs = ops.quant_per_token(bf16_dev(inp.x_bf16))
    q_ref, s_ref = orc.quant_per_token(inp.x_bf16)
    assert np.array_equal(xs.cpu().numpy(), s_ref)
    assert np.array_equal(xq.cpu().numpy(), q_ref)


@pytest.mark.parametrize("name", [w.name for w in wl.WORKLOADS])
def test_quant_per_channel_workload(ops, orc, name):
    inp = wl.generate(wl.by_name(name))
    wq, ws = ops.quant_per_channel(torch.from_numpy(inp.w_f32).to(DEV))
    q_ref, s_ref = orc.quant_per_channel(inp.w_f32)
    assert np.array_equal(ws.cpu().numpy(), s_ref)
    assert np.array_equal(wq.cpu().numpy(), q_ref)


def _edge_rows(rng, M, K):
    x = (rng.standard_normal((M, K)) * 10.0 ** rng.uniform(-3, 3, (M, 1))).astype(np.float32)
    if M > 4:
        x[1] = 0.0                                   # all-zero row
        x[2] = 0.0
        x[2, K // 2] = 2.0 ** -101                   # below the zero-row threshold
        x[3] = np.round(x[3])                        # integers: many exact ties below
        x[3, 0] = 127.0 * np.sign(x[3, 0] or 1.0)
        x[3, 1:] = np.clip(x[3, 1:], -126, 126) + 0.5
    return x


@pytest.mark.parametrize("M,K,pad", [(1, 1, 0), (3, 3, 8), (5, 8, 0), (7, 9, 0), (33, 100, 8),
                                     (64, 511, 0), (130, 513, 16), (9, 4097, 0), (600, 4096, 0),
                                     (17, 12288, 0), (5, 20000, 8), (3, 40000, 0)])
def test_quant_per_token_edges(ops, orc, M, K, pad):
    rng = np.random.default_rng(1000 + M + K)
    bits = wl.f32_to_bf16_bits(_edge_rows(rng, M, K))
    ldx = -(-K // 8) * 8 + pad
    xpad = np.zeros((M, ldx), np.uint16)
    xpad[:, :K] = bits
    xpad[:, K:] = 0x4780                             # large values beyond K must be ignored
    ldq = -(-K // 8) * 8 + 8
    x_d = bf16_dev(xpad)
    xq = torch.full((M, ldq), 0x5A, dtype=torch.int8, device=DEV)
    xs = torch.empty(M, dtype=torch.float32, device=DEV)
    ops.quant_per_token(x_d[:, :K], xq[:, :K], xs)
    q_ref, s_ref = orc.quant_per_token(bits)
    got = xq.cpu().numpy()
    assert np.array_equal(xs.cpu().numpy(), s_ref)
    assert np.array_equal(got[:, :K], q_ref)
    assert np.all(got[:, K:] == 0x5A), "wrote past K"


@pytest.mark.parametrize("N,K", [(1, 1), (3, 5), (17, 64), (40, 1000), (2, 40000)])
def test_quant_per_channel_edges(ops, orc, N, K):
    rng = np.random.default_rng(2000 + N + K)
    w = _edge_rows(rng, N, K)
    wq, ws = ops.quant_per_channel(torch.from_numpy(w).to(DEV))
    q_ref, s_ref = orc.quant_per_channel(w)
    assert np.array_equal(ws.cpu().numpy(), s_ref)
    assert np.array_equal(wq.cpu().numpy(), q_ref)


def test_quant_empty(ops):
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    xq, xs = ops.quant_per_token(x)
    assert xq.shape == (0, 64) and xs.shape == (0,)


# ---------------------------------------------------------------------------
# Prepack
# ---------------------------------------------------------------------------
def packed_reference(wq: np.ndarray) -> np.ndarray:
    """The byte layout stated in include/w8a8.h, built with NumPy indexing."""
    N, K = wq.shape
    Np, Kp = -(-N // 16) * 16, -(-K // 64) * 64
    w = np.zeros((Np, Kp), np.int8)
    w[:N, :K] = wq
    # F[nb][kb] byte 16*l + j = w[16*nb + l%16, 64*kb + 16*(l//16) + j]
    f = w.reshape(Np // 16, 16, Kp // 64, 4, 16)          # nb, l%16, kb, l//16, j
    f = f.transpose(0, 2, 3, 1, 4)                        # nb, kb, l//16, l%16, j
    return np.ascontiguousarray(f).reshape(-1).view(np.uint8)


@pytest.mark.parametrize("N,K", [(1, 1), (17, 65), (40, 200), (256, 4096), (3072, 12288)])
def test_prepack_layout_and_roundtrip(ops, N, K):
    rng = np.random.default_rng(3000 + N)
    wq = rand_i8(rng, (N, K), lo=-128)
    w_d = torch.from_numpy(wq).to(DEV)
    packed = ops.prepack_weight(w_d)
    assert np.array_equal(packed.cpu().numpy(), packed_reference(wq))
    assert np.array_equal(ops.unpack_weight(packed, N, K).cpu().numpy(), wq)


@pytest.mark.parametrize("N,K", [(1, 1), (17, 65), (40, 200), (33, 1000), (256, 4096),
                                 (3072, 12288)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quant_prepack_weight(ops, orc, N, K, dtype):
    """Online weight quant from fp32 or bf16 straight into the packed layout:
    the packed bytes are the layout of the oracle's per-channel codes, the
    scales are the oracle's, bit for bit (zero rows, a row below 2^-100 and a
    row of exact ties included)."""
    rng = np.random.default_rng(3100 + N + K)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    if N > 3:
        w[1] = 0.0
        w[2] = 1e-32
        w[3] = (np.arange(K) % 5 - 2).astype(np.float32) * 0.5 * (127.0 / 254.0)
    w_d = torch.from_numpy(w).to(DEV).to(dtype)
    w_exact = w_d.to(torch.float32).cpu().numpy()            # bf16 widens exactly
    wq_ref, ws_ref = orc.quant_per_channel(w_exact)
    packed, ws = ops.quant_prepack_weight(w_d)
    assert np.array_equal(ws.cpu().numpy(), ws_ref)
    assert np.array_equal(packed.cpu().numpy(), packed_reference(wq_ref))


# ---------------------------------------------------------------------------
# Scaled matmul on small and mid shapes, every tile configuration
# ---------------------------------------------------------------------------
SHAPES = [(1, 1, 16), (37, 45, 80), (130, 200, 336), (257, 300, 1040), (64, 128, 256),
          (300, 520, 576), (5, 1000, 2064), (61, 777, 1104)]


def _mm_case(seed, M, N, K, bias=True):
    inp = wl.random_case(M, K, N, seed, bias=bias)
    return inp


def _ntiles(ops):
    return list(range(ops.tile_count()))


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_scaled_mm_i32_every_tile(ops, orc, M, N, K):
    rng = np.random.default_rng(4000 + M + N + K)
    xq = rand_i8(rng, (M, K), lo=-128)
    wq = rand_i8(rng, (N, K), lo=-128)
    ref = orc.gemm_i32(xq, wq)
    xq_d = torch.from_numpy(xq).to(DEV)
    packed = ops.prepack_weight(torch.from_numpy(wq).to(DEV))
    for t in _ntiles(ops):
        acc = ops.scaled_mm(xq_d, None, packed, None, N, out_dtype=torch.int32, tile=t)
        assert np.array_equal(acc.cpu().numpy(), ref), f"tile {ops.tile_name(t)}"


# K values giving every number of LDS stages from 1 to 20 on the tiles with one
# k-group (a stage is one 64-deep k-block) and 1 to 10 on those with two (two
# k-blocks per stage), with a partial last k-block in between: the main
# kernel's LDS ring holds four stages, and loads for stages past the end are
# still issued (to clamped addresses) when K is short.
RING_KS = [64 * s for s in range(1, 21)] + [16, 208, 464, 720]


@pytest.mark.parametrize("K", RING_KS)
def test_scaled_mm_i32_ring_depths_every_tile(ops, orc, K):
    M, N = 97, 130
    rng = np.random.default_rng(4500 + K)
    xq = rand_i8(rng, (M, K), lo=-128)
    wq = rand_i8(rng, (N, K), lo=-128)
    ref = orc.gemm_i32(xq, wq)
    xq_d = torch.from_numpy(xq).to(DEV)
    packed = ops.prepack_weight(torch.from_numpy(wq).to(DEV))
    for t in _ntiles(ops):
        acc = ops.scaled_mm(xq_d, None, packed, None, N, out_dtype=torch.int32, tile=t)
        assert np.array_equal(acc.cpu().numpy(), ref), f"tile {ops.tile_name(t)} K {K}"


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("bias", [False, True])
def test_scaled_mm_bf16_every_tile(ops, orc, M, N, K, bias):
    inp = _mm_case(5000 + M + N + K, M, N, K, bias)
    wq, ws = orc.quant_per_channel(inp.w_f32)
    xq, xs = orc.quant_per_token(inp.x_bf16)
    acc = orc.gemm_i32(xq, wq)
    ref32 = orc.epilogue_f32(acc, xs, ws, inp.bias_bf16)
    ref64 = orc.epilogue_f64(acc, xs, ws, inp.bias_bf16)
    xq_d, xs_d = torch.from_numpy(xq).to(DEV), torch.from_numpy(xs).to(DEV)
    ws_d = torch.from_numpy(ws).to(DEV)
    b_d = None if inp.bias_bf16 is None else bf16_dev(inp.bias_bf16)
    packed = ops.prepack_weight(torch.from_numpy(wq).to(DEV))
    for t in _ntiles(ops):
        out = ops.scaled_mm(xq_d, xs_d, packed, ws_d, N, b_d, tile=t)
        got = bits_np(out)
        exact = check_out(got, ref32, ref64, f"tile {ops.tile_name(t)}")
        assert exact == 1.0, f"tile {ops.tile_name(t)}: {exact:.6f} bit-exact vs fp32 epilogue"


@pytest.mark.parametrize("M", [1, 3, 16, 32])
def test_scaled_mm_decode_shapes_auto(ops, orc, M):
    """A few token rows against a full-size weight (the decode case), through
    the automatic tile choice (the small-M kernel): exact against the oracle
    on every output, with a ragged N and K not a multiple of 64."""
    N, K = 3000, 4112
    inp = _mm_case(5500 + M, M, N, K, True)
    wq, ws = orc.quant_per_channel(inp.w_f32)
    xq, xs = orc.quant_per_token(inp.x_bf16)
    acc = orc.gemm_i32(xq, wq)
    ref32 = orc.epilogue_f32(acc, xs, ws, inp.bias_bf16)
    ref64 = orc.epilogue_f64(acc, xs, ws, inp.bias_bf16)
    assert ops.tile_name(ops.tile_auto(M, N, K)).startswith("s")
    packed = ops.prepack_weight(torch.from_numpy(wq).to(DEV))
    xq_d, xs_d = torch.from_numpy(xq).to(DEV), torch.from_numpy(xs).to(DEV)
    out = ops.scaled_mm(xq_d, xs_d, packed, torch.from_numpy(ws).to(DEV), N, bf16_dev(inp.bias_bf16))
    exact = check_out(bits_np(out), ref32, ref64, f"decode M={M}")
    assert exact == 1.0
    got = ops.scaled_mm(xq_d, None, packed, None, N, out_dtype=torch.int32)
    assert np.array_equal(got.cpu().numpy(), acc)


def test_scaled_mm_max_k_extremes(ops, orc):
    """K = W8A8_MAX_K with codes of magnitude 127 and mostly aligned signs:
    accumulators reach +-127^2 K (just inside int32) in every tile,
    main and small-M, exact in int32 and in the bf16 epilogue."""
    from w8a8_int8_dynamic_amd import _lib
    K = _lib.W8A8_MAX_K
    M, N = 33, 40
    rng = np.random.default_rng(4400)
    xq = np.where(rng.random((M, K)) < 0.999, 127, -127).astype(np.int8)
    wq = np.where(rng.random((N, K)) < 0.999, 127, -127).astype(np.int8)
    xq[0] = 127
    wq[0] = 127                                  # acc[0, 0] = 127^2 K
    wq[1] = -127                                 # acc[0, 1] = -127^2 K
    acc = orc.gemm_i32(xq, wq)
    assert acc[0, 0] == 127 * 127 * K and acc[0, 1] == -127 * 127 * K
    xs = rng.uniform(1e-3, 1e-2, M).astype(np.float32)
    ws = rng.uniform(1e-4, 1e-3, N).astype(np.float32)
    ref32 = orc.epilogue_f32(acc, xs, ws)
    ref64 = orc.epilogue_f64(acc, xs, ws)
    xq_d = torch.from_numpy(xq).to(DEV)
    packed = ops.prepack_weight(torch.from_numpy(wq).to(DEV))
    xs_d, ws_d = torch.from_numpy(xs).to(DEV), torch.from_numpy(ws).to(DEV)
    for t in range(ops.tile_count()):
        got = ops.scaled_mm(xq_d, None, packed, None, N, out_dtype=torch.int32, tile=t)
        assert np.array_equal(got.cpu().numpy(), acc), ops.tile_name(t)
        out = ops.scaled_mm(xq_d, xs_d, packed, ws_d, N, tile=t)
        assert check_out(bits_np(out), ref32, ref64, ops.tile_name(t)) == 1.0, ops.tile_name(t)


def test_scaled_mm_strided_output_and_unaligned_rows(ops, orc):
    """Leading dimensions larger than the row, odd ldo (scalar store path)."""
    M, N, K = 70, 37, 96
    inp = _mm_case(6001, M, N, K)
    wq, ws = orc.quant_per_channel(inp.w_f32)
    xq, xs = orc.quant_per_token(inp.x_bf16)
    acc = orc.gemm_i32(xq, wq)
    ref32 = orc.epilogue_f32(acc, xs, ws, inp.bias_bf16)
    xq_big = torch.zeros((M, K + 32), dtype=torch.int8, device=DEV)
    xq_big[:, :K] = torch.from_numpy(xq).to(DEV)
    packed = ops.prepack_weight(torch.from_numpy(wq).to(DEV))
    for ldo in (N, N + 3, 64):
        out_big = torch.full((M, ldo), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        ops.scaled_mm(xq_big[:, :K], torch.from_numpy(xs).to(DEV), packed,
                      torch.from_numpy(ws).to(DEV), N, bf16_dev(inp.bias_bf16), out=out_big[:, :N])
        got = bits_np(out_big)
        assert np.array_equal(got[:, :N], ref32)
        assert np.all(got[:, N:] == 0xFFFF), "wrote past N"


def test_scaled_mm_empty_and_determinism(ops, orc):
    packed = ops.prepack_weight(torch.zeros((16, 64), dtype=torch.int8, device=DEV))
    out = ops.scaled_mm(torch.empty((0, 64), dtype=torch.int8, device=DEV),
                        torch.empty(0, device=DEV), packed, torch.ones(16, device=DEV), 16)
    assert out.shape == (0, 16)
    M, N, K = 300, 520, 576
    inp = _mm_case(6002, M, N, K)
    wq, ws = orc.quant_per_channel(inp.w_f32)
    x_d = bf16_dev(inp.x_bf16)
    xq, xs = ops.quant_per_token(x_d)
    packed = ops.prepack_weight(torch.from_numpy(wq).to(DEV))
    ws_d, b_d = torch.from_numpy(ws).to(DEV), bf16_dev(inp.bias_bf16)
    first = ops.scaled_mm(xq, xs, packed, ws_d, N, b_d)
    for _ in range(50):
        again = ops.scaled_mm(xq, xs, packed, ws_d, N, b_d)
        assert torch.equal(first.view(torch.int16), again.view(torch.int16))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        other = ops.scaled_mm(xq, xs, packed, ws_d, N, b_d)
    s.synchronize()
    assert torch.equal(first.view(torch.int16), other.view(torch.int16))


# ---------------------------------------------------------------------------
# The five workloads at full size, in the benchmark's launch configuration
# ---------------------------------------------------------------------------
def full_size_parity(ops, orc, w) -> dict:
    """Run workload w at full size through the product path (W8A8Linear: the
    per-token quant and scaled matmul in one call) and compare every element
    with the oracle: codes, token and channel scales, the unpacked weight,
    the int32 accumulators (I32 mode) and the bf16 outputs (against the
    fp32 epilogue bit for bit and the fp64 epilogue within the tolerance
    bar). Also the rel-L2 of the outputs against fp64 matmuls of the
    dequantized operands (the pages' 0.17 % statistic) and of the raw bf16 X
    and fp32 W. Returns the counts; the caller asserts."""
    inp = wl.generate(w)
    from w8a8_int8_dynamic_amd import W8A8Linear
    layer = W8A8Linear.from_float(torch.from_numpy(inp.w_f32).to(DEV),
                                  None if inp.bias_bf16 is None else bf16_dev(inp.bias_bf16))
    x_d = bf16_dev(inp.x_bf16)
    out = layer(x_d)
    xq, xs = ops.quant_per_token(x_d)
    acc = ops.scaled_mm(xq, None, layer.w_packed, None, w.N, out_dtype=torch.int32)
    torch.cuda.synchronize()
    assert out.shape == (w.M, w.N) and out.dtype == torch.bfloat16
    r = {"name": w.name, "shape": (w.M, w.K, w.N)}
    wq_ref, ws_ref = orc.quant_per_channel(inp.w_f32)
    xq_ref, xs_ref = orc.quant_per_token(inp.x_bf16)
    r["ws_equal"] = int((layer.w_scale.cpu().numpy() == ws_ref).sum())
    r["wq_equal"] = int((ops.unpack_weight(layer.w_packed, w.N, w.K).cpu().numpy() == wq_ref).sum())
    r["xs_equal"] = int((xs.cpu().numpy() == xs_ref).sum())
    r["xq_equal"] = int((xq.cpu().numpy() == xq_ref).sum())
    acc_ref = orc.gemm_i32(xq_ref, wq_ref)
    r["acc_equal"] = int((acc.cpu().numpy() == acc_ref).sum())
    del acc
    got = bits_np(out)
    del out
    ref32 = orc.epilogue_f32(acc_ref, xs_ref, ws_ref, inp.bias_bf16)
    ref64 = orc.epilogue_f64(acc_ref, xs_ref, ws_ref, inp.bias_bf16)
    del acc_ref
    r["out_equal_f32_epilogue"] = int((got == ref32).sum())
    g, ref = f64(got), f64(ref64)
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    r["finite"] = bool(np.all(np.isfinite(g)))
    r["outside_tolerance"] = int((np.abs(g - ref) > RTOL * np.abs(ref) + ATOL_RMS * rms).sum())
    nz = ref != 0
    r["max_rel_vs_f64_epilogue"] = float(np.max(np.abs(g - ref)[nz] / np.abs(ref)[nz]))
    r["rel_l2_vs_f64_epilogue"] = float(np.linalg.norm(g - ref) / np.linalg.norm(ref))
    del ref, ref32, ref64
    b64 = 0.0 if inp.bias_bf16 is None else f64(inp.bias_bf16)[None, :]
    deq = (xq_ref.astype(np.float64) * xs_ref.astype(np.float64)[:, None]) @ \
          (wq_ref.astype(np.float64) * ws_ref.astype(np.float64)[:, None]).T + b64
    r["rel_l2_vs_f64_dequantized"] = float(np.linalg.norm(g - deq) / np.linalg.norm(deq))
    del deq
    raw = f64(inp.x_bf16) @ inp.w_f32.astype(np.float64).T + b64
    r["rel_l2_vs_f64_raw"] = float(np.linalg.norm(g - raw) / np.linalg.norm(raw))
    return r


def parity_table_row(r: dict) -> str:
    M, K, N = r["shape"]
    return (f"| {r['name']} | {M} x {K} x {N} | {r['xq_equal']:,} / {M * K:,} | "
            f"{r['xs_equal'] + r['ws_equal']:,} / {M + N:,} | {r['wq_equal']:,} / {N * K:,} | "
            f"{r['acc_equal']:,} / {M * N:,} | {r['out_equal_f32_epilogue']:,} / {M * N:,} | "
            f"{r['outside_tolerance']} | {r['max_rel_vs_f64_epilogue']:.2e} | "
            f"{100 * r['rel_l2_vs_f64_epilogue']:.4f} % | "
            f"{100 * r['rel_l2_vs_f64_dequantized']:.3f} % | {100 * r['rel_l2_vs_f64_raw']:.2f} % |")


PARITY_TABLE_HEAD = (
    "| workload | M x K x N | codes equal | scales equal (xs, ws) | weight codes equal | "
    "int32 acc equal | bf16 out equal to fp32 epilogue | outside tolerance | "
    "max rel err vs fp64 epilogue | rel-L2 vs fp64 epilogue | rel-L2 vs fp64 dequantized "
    "matmul | rel-L2 vs fp64 raw X W |\n|---|---|---|---|---|---|---|---|---|---|---|---|")


@pytest.mark.parametrize("name", [w.name for w in wl.WORKLOADS])
def test_workload_full_size(ops, orc, name):
    """Every element of every workload at full size, bit-exact (codes,
    scales, weight codes, int32 accumulators, bf16 outputs against the fp32
    epilogue) and within the tolerance bar of the fp64 epilogue."""
    w = wl.by_name(name)
    r = full_size_parity(ops, orc, w)
    print("\n" + parity_table_row(r))
    M, K, N = r["shape"]
    assert r["xq_equal"] == M * K and r["xs_equal"] == M
    assert r["wq_equal"] == N * K and r["ws_equal"] == N
    assert r["acc_equal"] == M * N
    assert r["finite"] and r["outside_tolerance"] == 0
    assert r["out_equal_f32_epilogue"] == M * N
    # bf16 rounding against fp64 on the dequantized operands: ~0.17 %
    assert r["rel_l2_vs_f64_dequantized"] < 0.0025


# ---------------------------------------------------------------------------
# Per-token quant and scaled matmul in one call (one launch where the grid
# fits the device, two launches otherwise)
# ---------------------------------------------------------------------------
QMM_SHAPES = [(1, 48, 64), (37, 45, 80), (130, 200, 336), (257, 300, 1040), (512, 520, 576),
              (512, 1536, 512), (2, 1000, 4112), (1, 300, 16384), (97, 130, 192), (66, 200, 448)]


@pytest.mark.parametrize("M,N,K", QMM_SHAPES)
@pytest.mark.parametrize("bias", [False, True])
def test_quant_scaled_mm_matches_two_calls_and_oracle(ops, orc, M, N, K, bias):
    inp = wl.random_case(M, K, N, 9100 + M + N + K, bias=bias)
    x = bf16_dev(inp.x_bf16)
    wq_ref, ws_ref = orc.quant_per_channel(inp.w_f32)
    packed = ops.prepack_weight(torch.from_numpy(wq_ref).to(DEV))
    ws = torch.from_numpy(ws_ref).to(DEV)
    b = bf16_dev(inp.bias_bf16) if bias else None
    xq_ref, xs_ref = orc.quant_per_token(inp.x_bf16)
    acc_ref = orc.gemm_i32(xq_ref, wq_ref)
    ref32 = orc.epilogue_f32(acc_ref, xs_ref, ws_ref, inp.bias_bf16 if bias else None)
    ref64 = orc.epilogue_f64(acc_ref, xs_ref, ws_ref, inp.bias_bf16 if bias else None)
    for t in range(ops.tile_count()):
        for _ in range(2):                     # the second call reuses reset counters
            out, xq, xs = ops.quant_scaled_mm(x, packed, ws, N, b, tile=t)
            torch.cuda.synchronize()
            assert np.array_equal(xs.cpu().numpy(), xs_ref), ops.tile_name(t)
            assert np.array_equal(xq.cpu().numpy(), xq_ref), ops.tile_name(t)
            got = bits_np(out)
            exact = check_out(got, ref32, ref64, f"fused {ops.tile_name(t)} {M}x{N}x{K}")
            assert exact == 1.0, ops.tile_name(t)
        acc, _, _ = ops.quant_scaled_mm(x, packed, None, N, out_dtype=torch.int32, tile=t)
        assert np.array_equal(acc.cpu().numpy(), acc_ref), ops.tile_name(t)


@pytest.mark.parametrize("M", [1, 2, 5])
def test_quant_scaled_mm_decode_graph_replays(ops, orc, M):
    """The decode-shaped fused call captured in a HIP graph: several replays,
    with eager work and synchronizations between them, each checked against
    the oracle (M 1 and 2 take the single-launch small-M path, 5 the two
    launches)."""
    N, K = 1000, 4112
    inp = wl.random_case(M, K, N, 9300 + M, bias=True)
    x = bf16_dev(inp.x_bf16)
    wq_ref, ws_ref = orc.quant_per_channel(inp.w_f32)
    packed = ops.prepack_weight(torch.from_numpy(wq_ref).to(DEV))
    ws, b = torch.from_numpy(ws_ref).to(DEV), bf16_dev(inp.bias_bf16)
    xq_ref, xs_ref = orc.quant_per_token(inp.x_bf16)
    acc = orc.gemm_i32(xq_ref, wq_ref)
    ref32 = orc.epilogue_f32(acc, xs_ref, ws_ref, inp.bias_bf16)
    ref64 = orc.epilogue_f64(acc, xs_ref, ws_ref, inp.bias_bf16)
    xq = torch.empty((M, K), dtype=torch.int8, device=DEV)
    xs = torch.empty((M,), dtype=torch.float32, device=DEV)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ops.quant_scaled_mm(x, packed, ws, N, b, out=out, xq=xq, xs=xs)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.quant_scaled_mm(x, packed, ws, N, b, out=out, xq=xq, xs=xs)
    for i in range(4):
        out.fill_(0)
        xq.fill_(0)
        xs.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(xq.cpu().numpy(), xq_ref) and np.array_equal(xs.cpu().numpy(), xs_ref)
        exact = check_out(bits_np(out), ref32, ref64, f"replay {i}")
        assert exact == 1.0, f"replay {i}"
        ops.scaled_mm(xq, xs, packed, ws, N, b)    # eager work between replays


def test_quant_scaled_mm_main_graph_replays_new_inputs(ops, orc):
    """A main-tile call (eagerly the one-launch path with producer flags)
    captured in a HIP graph, replayed with a different input copied into
    the captured x before each replay. Each replay must match the oracle
    for the input it saw: a replay must never take an earlier replay's
    quantized rows."""
    M, N, K = 512, 1536, 512
    cases = []
    for i in range(2):
        inp = wl.random_case(M, K, N, 9400 + i, bias=True)
        xq_ref, xs_ref = orc.quant_per_token(inp.x_bf16)
        cases.append((inp, xq_ref, xs_ref))
    w_inp = cases[0][0]
    wq_ref, ws_ref = orc.quant_per_channel(w_inp.w_f32)
    packed = ops.prepack_weight(torch.from_numpy(wq_ref).to(DEV))
    ws, b = torch.from_numpy(ws_ref).to(DEV), bf16_dev(w_inp.bias_bf16)
    refs = []
    for inp, xq_ref, xs_ref in cases:
        acc = orc.gemm_i32(xq_ref, wq_ref)
        refs.append((orc.epilogue_f32(acc, xs_ref, ws_ref, w_inp.bias_bf16),
                     orc.epilogue_f64(acc, xs_ref, ws_ref, w_inp.bias_bf16)))
    xs_dev = [bf16_dev(inp.x_bf16) for inp, _, _ in cases]
    x = xs_dev[0].clone()
    xq = torch.empty((M, K), dtype=torch.int8, device=DEV)
    xs = torch.empty((M,), dtype=torch.float32, device=DEV)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ops.quant_scaled_mm(x, packed, ws, N, b, out=out, xq=xq, xs=xs)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.quant_scaled_mm(x, packed, ws, N, b, out=out, xq=xq, xs=xs)
    for i in range(6):
        c = i % 2
        x.copy_(xs_dev[c])
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _, xq_ref, xs_ref = cases[c]
        assert np.array_equal(xs.cpu().numpy(), xs_ref), f"replay {i}"
        assert np.array_equal(xq.cpu().numpy(), xq_ref), f"replay {i}"
        exact = check_out(bits_np(out), refs[c][0], refs[c][1], f"replay {i}")
        assert exact == 1.0, f"replay {i}"
        ops.quant_scaled_mm(xs_dev[1 - c], packed, ws, N, b)    # eager one-launch call between


def test_quant_scaled_mm_alternating_shapes(ops, orc):
    """Calls of different shapes back to back on one stream, each checked."""
    cases = []
    for i, (M, N, K) in enumerate([(512, 1536, 512), (64, 128, 256), (300, 520, 576)] * 2):
        inp = wl.random_case(M, K, N, 9300 + i)
        wq_ref, ws_ref = orc.quant_per_channel(inp.w_f32)
        packed = ops.prepack_weight(torch.from_numpy(wq_ref).to(DEV))
        out, _, _ = ops.quant_scaled_mm(bf16_dev(inp.x_bf16), packed,
                                        torch.from_numpy(ws_ref).to(DEV), N)
        cases.append((inp, wq_ref, ws_ref, out))
    torch.cuda.synchronize()
    for inp, wq_ref, ws_ref, out in cases:
        xq_ref, xs_ref = orc.quant_per_token(inp.x_bf16)
        ref32 = orc.epilogue_f32(orc.gemm_i32(xq_ref, wq_ref), xs_ref, ws_ref)
        assert np.array_equal(bits_np(out), ref32)


def test_quant_scaled_mm_reused_buffers(ops, orc):
    """Back-to-back calls that write new codes into the same xq / xs / out
    buffers: every call must read the codes of its own input, never a copy
    left in a cache by the previous call."""
    M, N, K = 512, 1536, 512
    inps = [wl.random_case(M, K, N, 9400 + i) for i in range(2)]
    wq_ref, ws_ref = orc.quant_per_channel(inps[0].w_f32)
    packed = ops.prepack_weight(torch.from_numpy(wq_ref).to(DEV))
    ws = torch.from_numpy(ws_ref).to(DEV)
    xs_dev = [bf16_dev(i.x_bf16) for i in inps]
    xq = torch.empty((M, K), dtype=torch.int8, device=DEV)
    xs = torch.empty((M,), dtype=torch.float32, device=DEV)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    refs = []
    for inp in inps:
        q_ref, s_ref = orc.quant_per_token(inp.x_bf16)
        refs.append(orc.epilogue_f32(orc.gemm_i32(q_ref, wq_ref), s_ref, ws_ref))
    for it in range(8):
        k = it % 2
        ops.quant_scaled_mm(xs_dev[k], packed, ws, N, out=out, xq=xq, xs=xs)
        torch.cuda.synchronize()
        assert np.array_equal(bits_np(out), refs[k]), f"call {it}"


def test_linear_keeps_leading_dims(ops, orc):
    from w8a8_int8_dynamic_amd import W8A8Linear
    inp = wl.random_case(2 * 37, 320, 48, 7001)
    layer = W8A8Linear.from_float(torch.from_numpy(inp.w_f32).to(DEV), bf16_dev(inp.bias_bf16))
    x = bf16_dev(inp.x_bf16)
    y2 = layer(x)
    y3 = layer(x.view(2, 37, 320))
    assert y3.shape == (2, 37, 48)
    assert torch.equal(y3.reshape(74, 48).view(torch.int16), y2.view(torch.int16))
    with pytest.raises(ValueError):
        layer(x[:, :300])


def test_binding_errors_on_device(ops):
    from w8a8_int8_dynamic_amd import W8A8Error
    xq = torch.zeros((4, 72), dtype=torch.int8, device=DEV)
    packed = ops.prepack_weight(torch.zeros((16, 72), dtype=torch.int8, device=DEV))
    with pytest.raises(W8A8Error) as e:
        ops.scaled_mm(xq, torch.ones(4, device=DEV), packed, torch.ones(16, device=DEV), 16)
    assert e.value.status == 2    # K = 72 is not a multiple of 16


def test_binding_argument_checks(ops):
    """The wrappers refuse what the C ABI cannot check: a packed weight too
    small for (N, K), and out / xq buffers of the wrong shape, for the int8
    calls and their e4m3 twins."""
    bf = torch.bfloat16
    x = torch.zeros((4, 64), dtype=bf, device=DEV)
    w = torch.zeros((16, 64), device=DEV)
    packed, ws = ops.quant_prepack_weight(w)
    packed8, ws8 = ops.fp8_quant_prepack_weight(w)
    xq, xs = ops.quant_per_token(x)
    xq8, xs8 = ops.fp8_quant_per_token(x)
    small = packed[:-16]
    bad_out = torch.empty((4, 8), dtype=bf, device=DEV)
    cases = [
        lambda: ops.scaled_mm(xq, xs, small, ws, 16),
        lambda: ops.scaled_mm(xq, xs, packed, ws, 16, out=bad_out),
        lambda: ops.quant_scaled_mm(x, small, ws, 16),
        lambda: ops.quant_scaled_mm(x, packed, ws, 16, out=bad_out),
        lambda: ops.quant_scaled_mm(x, packed, ws, 16, xq=torch.empty((4, 32), dtype=torch.int8,
                                                                      device=DEV)),
        lambda: ops.quant_per_token(x, xq=torch.empty((4, 32), dtype=torch.int8, device=DEV)),
        lambda: ops.fp8_scaled_mm(xq8, xs8, packed8[:-16], ws8, 16),
        lambda: ops.fp8_scaled_mm(xq8, xs8, packed8, ws8, 16, out=bad_out),
        lambda: ops.fp8_quant_scaled_mm(x, packed8[:-16], ws8, 16),
        lambda: ops.fp8_quant_scaled_mm(x, packed8, ws8, 16, out=bad_out),
        lambda: ops.fp8_quant_scaled_mm(x, packed8, ws8, 16,
                                        xq=torch.empty((4, 32), dtype=torch.uint8, device=DEV)),
        lambda: ops.fp8_quant_per_token(x, xq=torch.empty((4, 32), dtype=torch.uint8, device=DEV)),
    ]
    for i, case in enumerate(cases):
        with pytest.raises(ValueError):
            case()
            pytest.fail(f"case {i} was accepted")
    # and the well-formed calls still run, the fp8 one with caller buffers
    out8, q8, s8 = ops.fp8_quant_scaled_mm(x, packed8, ws8, 16, xq=xq8, xs=xs8)
    assert q8.data_ptr() == xq8.data_ptr() and s8.data_ptr() == xs8.data_ptr()
    assert out8.shape == (4, 16)


def test_quant_scaled_mm_own_rows_path(ops, orc):
    """The one-launch path's bounded wait run out at once (bound 0, set from
    the host): every workgroup quantizes its tile's rows itself instead of
    waiting for their producers. Codes, scales and outputs stay bit-exact to
    the oracle on every main tile, int8 and e4m3."""
    from w8a8_int8_dynamic_amd import _lib
    L = _lib.lib()
    main = [t for t in range(ops.tile_count()) if not ops.tile_name(t).startswith("s")]
    cases = []
    for i, (M, N, K) in enumerate([(512, 1536, 512), (257, 300, 1040), (130, 200, 336)]):
        inp = wl.random_case(M, K, N, 9500 + i, bias=True)
        wq_ref, ws_ref = orc.quant_per_channel(inp.w_f32)
        xq_ref, xs_ref = orc.quant_per_token(inp.x_bf16)
        ref32 = orc.epilogue_f32(orc.gemm_i32(xq_ref, wq_ref), xs_ref, ws_ref, inp.bias_bf16)
        packed = ops.prepack_weight(torch.from_numpy(wq_ref).to(DEV))
        cases.append((inp, N, packed, torch.from_numpy(ws_ref).to(DEV), xq_ref, xs_ref, ref32))
    inp8 = cases[0][0]
    packed8, ws8 = ops.fp8_quant_prepack_weight(torch.from_numpy(inp8.w_f32).to(DEV))
    x8, b8 = bf16_dev(inp8.x_bf16), bf16_dev(inp8.bias_bf16)
    waited = [ops.fp8_quant_scaled_mm(x8, packed8, ws8, cases[0][1], b8, tile=t)[0].clone()
              for t in main]
    prev = L.w8a8_fused_wait_limit(0)
    try:
        for inp, N, packed, ws, xq_ref, xs_ref, ref32 in cases:
            x, b = bf16_dev(inp.x_bf16), bf16_dev(inp.bias_bf16)
            for t in main:
                out, xq, xs = ops.quant_scaled_mm(x, packed, ws, N, b, tile=t)
                torch.cuda.synchronize()
                name = f"{ops.tile_name(t)} {inp.x_bf16.shape}"
                assert np.array_equal(xq.cpu().numpy(), xq_ref), name
                assert np.array_equal(xs.cpu().numpy(), xs_ref), name
                assert np.array_equal(bits_np(out), ref32), name
        for t, ref in zip(main, waited):
            out8, _, _ = ops.fp8_quant_scaled_mm(x8, packed8, ws8, cases[0][1], b8, tile=t)
            assert torch.equal(out8.view(torch.int16), ref.view(torch.int16)), ops.tile_name(t)
    finally:
        L.w8a8_fused_wait_limit(prev)


@pytest.mark.parametrize("q_off,s_off", [(16, 1), (0, 1), (16, 0), (256, 64), (48, 3)])
def test_quant_scaled_mm_offset_code_and_scale_views(ops, orc, q_off, s_off):
    """Codes and scales written into views that start inside a larger buffer
    (xq at q_off bytes, xs at s_off floats): rows of two row tiles can then
    share a cache line, which the one-launch path must not depend on (it is
    taken only for 256-byte aligned buffers). Every main tile, int8 and
    e4m3, against the oracle; the bytes around the views stay untouched."""
    M, N, K = 384, 1536, 1040
    inp = wl.random_case(M, K, N, 9650 + q_off + s_off, bias=True)
    wq_ref, ws_ref = orc.quant_per_channel(inp.w_f32)
    xq_ref, xs_ref = orc.quant_per_token(inp.x_bf16)
    ref32 = orc.epilogue_f32(orc.gemm_i32(xq_ref, wq_ref), xs_ref, ws_ref, inp.bias_bf16)
    packed = ops.prepack_weight(torch.from_numpy(wq_ref).to(DEV))
    ws, x, b = torch.from_numpy(ws_ref).to(DEV), bf16_dev(inp.x_bf16), bf16_dev(inp.bias_bf16)
    ldq = 1056                                      # a multiple of 16, not of 128
    qbuf = torch.full((M * ldq + q_off + 64,), 0x5A, dtype=torch.int8, device=DEV)
    sbuf = torch.full((M + s_off + 16,), -7.0, dtype=torch.float32, device=DEV)
    xq = qbuf[q_off:q_off + M * ldq].view(M, ldq)[:, :K]
    xs = sbuf[s_off:s_off + M]
    main = [t for t in range(ops.tile_count()) if not ops.tile_name(t).startswith("s")]
    for t in main:
        qbuf.fill_(0x5A)
        sbuf.fill_(-7.0)
        out, _, _ = ops.quant_scaled_mm(x, packed, ws, N, b, tile=t, xq=xq, xs=xs)
        torch.cuda.synchronize()
        name = f"{ops.tile_name(t)} q_off {q_off} s_off {s_off}"
        assert np.array_equal(xq.cpu().numpy(), xq_ref), name
        assert np.array_equal(xs.cpu().numpy(), xs_ref), name
        assert np.array_equal(bits_np(out), ref32), name
        qh = qbuf.cpu().numpy()
        assert np.all(qh[:q_off] == 0x5A) and np.all(qh[q_off + M * ldq:] == 0x5A), name
        assert np.all(qh[q_off:q_off + M * ldq].reshape(M, ldq)[:, K:] == 0x5A), name
        sh = sbuf.cpu().numpy()
        assert np.all(sh[:s_off] == -7.0) and np.all(sh[s_off + M:] == -7.0), name
    packed8, ws8 = ops.fp8_quant_prepack_weight(torch.from_numpy(inp.w_f32).to(DEV))
    q8buf = torch.zeros((M * ldq + q_off + 64,), dtype=torch.uint8, device=DEV)
    xq8 = q8buf[q_off:q_off + M * ldq].view(M, ldq)[:, :K]
    for t in main:
        ref8, rq8, rs8 = ops.fp8_quant_scaled_mm(x, packed8, ws8, N, b, tile=t)
        out8, q8, s8 = ops.fp8_quant_scaled_mm(x, packed8, ws8, N, b, tile=t, xq=xq8, xs=xs)
        torch.cuda.synchronize()
        assert torch.equal(q8, rq8) and torch.equal(s8, rs8), ops.tile_name(t)
        assert torch.equal(out8.view(torch.int16), ref8.view(torch.int16)), ops.tile_name(t)


def test_quant_scaled_mm_overlapping_streams(ops, orc):
    """Single-launch calls on two streams at once share the producer-flag
    words; each launch accepts only its own launch number, so a clobbered
    wait runs out and the workgroup quantizes its rows itself. Every call's
    codes, scales and outputs must match the oracle for its own input."""
    M, N, K = 512, 1536, 1024
    cases = []
    for i in range(2):
        inp = wl.random_case(M, K, N, 9600 + i, bias=True)
        wq_ref, ws_ref = orc.quant_per_channel(inp.w_f32)
        xq_ref, xs_ref = orc.quant_per_token(inp.x_bf16)
        ref32 = orc.epilogue_f32(orc.gemm_i32(xq_ref, wq_ref), xs_ref, ws_ref, inp.bias_bf16)
        packed = ops.prepack_weight(torch.from_numpy(wq_ref).to(DEV))
        cases.append((bf16_dev(inp.x_bf16), packed, torch.from_numpy(ws_ref).to(DEV),
                      bf16_dev(inp.bias_bf16), xq_ref, xs_ref, ref32))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    results = []
    for it in range(8):
        for k, s in enumerate(streams):
            x, packed, ws, b, *_ = cases[k]
            with torch.cuda.stream(s):
                results.append((k, ops.quant_scaled_mm(x, packed, ws, N, b)))
    torch.cuda.synchronize()
    for k, (out, xq, xs) in results:
        _, _, _, _, xq_ref, xs_ref, ref32 = cases[k]
        assert np.array_equal(xq.cpu().numpy(), xq_ref) and np.array_equal(xs.cpu().numpy(), xs_ref)
        assert np.array_equal(bits_np(out), ref32)


def test_bf16_output_range_edges(ops, orc):
    """bf16 outputs across fp32's range on every tile: caller scales from
    1e-40 to 1e30 (and channel scales of 1e-30) take the fixed-order fp32
    epilogue into subnormals, to signed zeros and up to about 1e33. Bit-exact to the oracle's fp32 epilogue, signed zeros and
    subnormal results included."""
    M, N, K = 80, 136, 320
    rng = np.random.default_rng(8900)
    xq = rng.integers(-127, 128, (M, K), dtype=np.int8)
    wq = rng.integers(-127, 128, (N, K), dtype=np.int8)
    xs = (10.0 ** np.linspace(-40, 30, M)).astype(np.float32)
    ws = (rng.uniform(0.5, 2.0, N) * 1e-2).astype(np.float32)
    ws[::17] = np.float32(1e-30)                  # products that underflow to signed zeros
    acc = orc.gemm_i32(xq, wq)
    ref = orc.epilogue_f32(acc, xs, ws)
    assert ((ref & 0x7F80) == 0).any() and ((ref & 0x007F) != 0).any()   # bf16 subnormals
    assert (ref == 0x8000).any()                                         # negative zeros
    xq_d = torch.from_numpy(xq).to(DEV)
    packed = ops.prepack_weight(torch.from_numpy(wq).to(DEV))
    xs_d, ws_d = torch.from_numpy(xs).to(DEV), torch.from_numpy(ws).to(DEV)
    for t in range(ops.tile_count()):
        out = ops.scaled_mm(xq_d, xs_d, packed, ws_d, N, tile=t)
        assert np.array_equal(bits_np(out), ref), ops.tile_name(t)
