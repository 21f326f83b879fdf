"""int8_quant_scaled_mm_noalloc, the entry point for callers that cannot
allocate: its workspace is the library's static device array. Called
through the C ABI twice in a row, the second with a smaller input, and
compared element by element with int8_quant_scaled_mm_ws (caller
workspace) and with the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def test_no_alloc_matches_workspace_entry(orc):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w8a8_int8_dynamic_amd import _lib, ops
    L = _lib.lib()
    stream = torch.cuda.current_stream().cuda_stream
    # the first call splits K 4 ways; the second, smaller, 2 ways with
    # ragged N and K and a bias
    for (M, N, K, bias, seed) in [(4, 1024, 32768, False, 9950), (3, 300, 24640, True, 9951)]:
        inp = wl.random_case(M, K, N, seed, bias=bias)
        wq, ws = orc.quant_per_channel(inp.w_f32)
        xq_r, xs_r = orc.quant_per_token(inp.x_bf16)
        ref32 = orc.epilogue_f32(orc.gemm_i32(xq_r, wq), xs_r, ws, inp.bias_bf16 if bias else None)
        packed = ops.prepack_weight(torch.from_numpy(wq).to(DEV))
        ws_d = torch.from_numpy(ws).to(DEV)
        b_d = _bf16(inp.bias_bf16) if bias else None
        x = _bf16(inp.x_bf16)
        need = ops.workspace_bytes(M, N, K)
        assert need > 0
        work = torch.zeros((need,), dtype=torch.uint8, device=DEV)
        outs = []
        for name in ("int8_quant_scaled_mm_noalloc", "int8_quant_scaled_mm_ws"):
            out = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=DEV)
            xq = torch.zeros((M, K), dtype=torch.int8, device=DEV)
            xs = torch.zeros((M,), dtype=torch.float32, device=DEV)
            args = [x.data_ptr(), K, xq.data_ptr(), K, xs.data_ptr(), packed.data_ptr(),
                    ws_d.data_ptr(), None if b_d is None else b_d.data_ptr(), M, N, K, 0,
                    out.data_ptr(), N]
            if name.endswith("_ws"):
                args += [work.data_ptr(), need]
            rc = getattr(L, name)(*args, stream)
            assert rc == 0, (name, _lib.last_error())
            torch.cuda.synchronize()
            outs.append(out.view(torch.int16).cpu().numpy().view(np.uint16))
            assert np.array_equal(xq.cpu().numpy(), xq_r), name
            assert np.array_equal(xs.cpu().numpy(), xs_r), name
        assert np.array_equal(outs[0], outs[1])
        assert np.array_equal(outs[0], ref32)
