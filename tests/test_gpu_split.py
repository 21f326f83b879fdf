"""The split of K over workgroups for decode-shaped products (a few token
rows against a weight with few 16-channel column blocks), through the
workspace entry points int8_scaled_mm_ws and int8_quant_scaled_mm_ws.

Bar: bit-exact against the oracle (int32 accumulators, bf16 outputs against
the fixed-order fp32 epilogue, codes and scales) and bit-identical to the
same call without a workspace; the per-tile counters are back at zero after
every call, including graph replays.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w8a8_int8_dynamic_amd import ops as _ops
    return _ops


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def bits_np(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


# (M, N, K): long K against few column blocks, where the split pays: 8 ways
# (N = 16 at the largest K, N = 64), 4 ways (N = 128, the 32-row tile with
# ragged K, 17 rows), 2 ways with ragged N and K.
SPLIT_SHAPES = [(1, 16, 131056), (1, 64, 65536), (2, 128, 32768), (4, 1024, 32768),
                (17, 2000, 40960), (3, 300, 24640), (32, 1024, 50000)]


def _case(orc, M, N, K, seed, bias=True):
    inp = wl.random_case(M, K, N, seed, bias=bias)
    wq, ws = orc.quant_per_channel(inp.w_f32)
    xq, xs = orc.quant_per_token(inp.x_bf16)
    acc = orc.gemm_i32(xq, wq)
    ref32 = orc.epilogue_f32(acc, xs, ws, inp.bias_bf16 if bias else None)
    return inp, wq, ws, xq, xs, acc, ref32


def _count_bytes(ops, M, N, K):
    """Bytes of per-tile counters at the start of the workspace."""
    from w8a8_int8_dynamic_amd import _lib
    t = ops.tile_auto(M, N, K)
    name = ops.tile_name(t)
    bm, bn = (int(v) for v in name[1:].split("/")[0].split("x"))
    tiles = -(-M // bm) * -(-N // bn)
    return -(-tiles * 8 // 256) * 256


@pytest.mark.parametrize("M,N,K", SPLIT_SHAPES)
def test_split_k_bit_exact(ops, orc, M, N, K):
    need = ops.workspace_bytes(M, N, K)
    assert need > 0, f"{M}x{N}x{K} should split K"
    inp, wq, ws, xq_ref, xs_ref, acc_ref, ref32 = _case(orc, M, N, K, 9800 + M + N + K)
    packed = ops.prepack_weight(torch.from_numpy(wq).to(DEV))
    ws_d, b_d, x = torch.from_numpy(ws).to(DEV), bf16_dev(inp.bias_bf16), bf16_dev(inp.x_bf16)
    work = torch.zeros((need,), dtype=torch.uint8, device=DEV)
    xq_d, xs_d = torch.from_numpy(xq_ref).to(DEV), torch.from_numpy(xs_ref).to(DEV)
    cb = _count_bytes(ops, M, N, K)
    for rep in range(3):                          # the counters must reset every call
        acc = ops.scaled_mm(xq_d, None, packed, None, N, out_dtype=torch.int32, workspace=work)
        out = ops.scaled_mm(xq_d, xs_d, packed, ws_d, N, b_d, workspace=work)
        outq, q, s = ops.quant_scaled_mm(x, packed, ws_d, N, b_d, workspace=work)
        torch.cuda.synchronize()
        assert np.array_equal(acc.cpu().numpy(), acc_ref), rep
        assert np.array_equal(bits_np(out), ref32), rep
        assert np.array_equal(bits_np(outq), ref32), rep
        assert np.array_equal(q.cpu().numpy(), xq_ref) and np.array_equal(s.cpu().numpy(), xs_ref)
        assert not work[:cb].any(), "per-tile counters not back at zero"
    # the same calls without a workspace: identical bits
    plain = ops.quant_scaled_mm(x, packed, ws_d, N, b_d)[0]
    assert torch.equal(plain.view(torch.int16), outq.view(torch.int16))
    # a workspace one byte short: no split, same result
    short = torch.zeros((need - 1,), dtype=torch.uint8, device=DEV)
    again = ops.quant_scaled_mm(x, packed, ws_d, N, b_d, workspace=short)[0]
    assert torch.equal(again.view(torch.int16), plain.view(torch.int16))


def test_split_k_no_split_shapes(ops):
    # enough column blocks to fill the device, K too short for a split to
    # pay (the decode shapes of the five workloads), M beyond the small-M
    # tiles, or no rows
    assert ops.workspace_bytes(1, 12288, 4096) == 0
    assert ops.workspace_bytes(8, 3072, 12288) == 0
    assert ops.workspace_bytes(512, 3072, 32768) == 0
    assert ops.workspace_bytes(0, 1024, 32768) == 0


def test_split_k_graph_replays(ops, orc):
    """The split decode step captured in a HIP graph and replayed with a new
    input copied in before each replay and eager work in between: every
    replay matches the oracle for its own input, and the counters return to
    zero."""
    M, N, K = 2, 1024, 32768
    cases = [_case(orc, M, N, K, 9900 + i, bias=False) for i in range(3)]
    wq, ws = cases[0][1], cases[0][2]
    # one weight for all: recompute the references against it
    refs = []
    for inp, *_ in cases:
        xq, xs = orc.quant_per_token(inp.x_bf16)
        refs.append(orc.epilogue_f32(orc.gemm_i32(xq, wq), xs, ws, None))
    packed = ops.prepack_weight(torch.from_numpy(wq).to(DEV))
    ws_d = torch.from_numpy(ws).to(DEV)
    need = ops.workspace_bytes(M, N, K)
    work = torch.zeros((need,), dtype=torch.uint8, device=DEV)
    x = bf16_dev(cases[0][0].x_bf16)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    xq = torch.empty((M, K), dtype=torch.int8, device=DEV)
    xs = torch.empty((M,), dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ops.quant_scaled_mm(x, packed, ws_d, N, out=out, xq=xq, xs=xs, workspace=work)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ops.quant_scaled_mm(x, packed, ws_d, N, out=out, xq=xq, xs=xs, workspace=work)
    cb = _count_bytes(ops, M, N, K)
    for it in range(6):
        k = it % 3
        x.copy_(bf16_dev(cases[k][0].x_bf16))
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_np(out), refs[k]), it
        assert not work[:cb].any()
        torch.mm(torch.ones(64, 64, device=DEV), torch.ones(64, 64, device=DEV))   # eager work
