"""Parity report of the GPU path against the oracle on the five workloads.

    python tests/parity_report.py > report.md      (needs a gfx950 GPU)

For each workload at full size, through the product path (W8A8Linear):
codes and scales compared with the oracle on every row; int32 accumulators
on sampled rows (all rows for the tiny workload) and through exact row and
column sums; bf16 outputs on the sampled rows against the oracle's fp32
epilogue (bit-exact count), its fp64 epilogue (max relative error, rel-L2),
an fp64 matmul of the dequantized operands (the pages' 0.17 % statistic)
and an fp64 matmul of the raw bf16 X and fp32 W (the quantization error).
Prints one markdown table. Not a test: the assertions live in
tests/test_gpu_parity.py.
"""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as wl  # noqa: E402
from w8a8_int8_dynamic_amd import W8A8Linear, ops  # noqa: E402


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _f64(bits):
    return wl.bf16_bits_to_f32(bits).astype(np.float64)


def _rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def report_row(orc, w) -> str:
    inp = wl.generate(w)
    bias = None if inp.bias_bf16 is None else _bf16_dev(inp.bias_bf16)
    layer = W8A8Linear.from_float(torch.from_numpy(inp.w_f32).cuda(), bias)
    x = _bf16_dev(inp.x_bf16)
    out = layer(x)
    xq, xs = ops.quant_per_token(x)
    acc = ops.scaled_mm(xq, None, layer.w_packed, None, w.N, out_dtype=torch.int32).cpu().numpy()
    torch.cuda.synchronize()

    wq_r, ws_r = orc.quant_per_channel(inp.w_f32)
    xq_r, xs_r = orc.quant_per_token(inp.x_bf16)
    codes_ok = int((xq.cpu().numpy() == xq_r).sum())
    scales_ok = int((xs.cpu().numpy() == xs_r).sum()) + int((layer.w_scale.cpu().numpy() == ws_r).sum())
    if w.M <= 64:
        rows = np.arange(w.M)
    else:
        rng = np.random.default_rng(w.seed)
        rows = np.array(sorted(set(rng.choice(w.M, 40, replace=False).tolist()) | {0, w.M - 1}))
    acc_r = orc.gemm_i32(xq_r, wq_r, rows)
    acc_ok = int((acc[rows] == acc_r).sum())
    x64, w64 = xq_r.astype(np.int64), wq_r.astype(np.int64)
    sums_ok = bool(np.array_equal(acc.sum(axis=1, dtype=np.int64), x64 @ w64.sum(axis=0)) and
                   np.array_equal(acc.sum(axis=0, dtype=np.int64), x64.sum(axis=0) @ w64.T))
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)[rows]
    ref32 = orc.epilogue_f32(acc_r, xs_r[rows], ws_r, inp.bias_bf16)
    ref64 = orc.epilogue_f64(acc_r, xs_r[rows], ws_r, inp.bias_bf16)
    g, r = _f64(got), _f64(ref64)
    nz = r != 0
    max_rel = float(np.max(np.abs(g - r)[nz] / np.abs(r)[nz]))
    b64 = 0.0 if inp.bias_bf16 is None else _f64(inp.bias_bf16)[None, :]
    deq = (xq_r[rows].astype(np.float64) * xs_r[rows, None]) @ \
          (wq_r.astype(np.float64) * ws_r[:, None]).T + b64
    raw = _f64(inp.x_bf16[rows]) @ inp.w_f32.astype(np.float64).T + b64
    n_codes = w.M * w.K
    return (f"| {w.name} | {w.M} x {w.K} x {w.N} | {codes_ok:,} / {n_codes:,} | "
            f"{scales_ok:,} / {w.M + w.N:,} | {acc_ok:,} / {len(rows) * w.N:,} ({len(rows)} rows) | "
            f"{'exact' if sums_ok else 'DIFFER'} | {int((got == ref32).sum()):,} / {got.size:,} | "
            f"{max_rel:.2e} | {100 * _rel_l2(g, r):.4f} % | {100 * _rel_l2(g, deq):.3f} % | "
            f"{100 * _rel_l2(g, raw):.2f} % |")


def main() -> int:
    if not torch.cuda.is_available():
        print("needs a GPU", file=sys.stderr)
        return 1
    orc = oracle.load()
    print("| workload | M x K x N | codes equal | scales equal (xs, ws) | int32 acc equal | "
          "acc row/col sums | bf16 out equal to fp32 epilogue | max rel err vs fp64 epilogue | "
          "rel-L2 vs fp64 epilogue | rel-L2 vs fp64 dequantized matmul | rel-L2 vs fp64 raw X W |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    for w in wl.WORKLOADS:
        print(report_row(orc, w), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
