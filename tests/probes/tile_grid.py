"""Every main tile of int8_scaled_mm timed on a grid of layer shapes, next to
the tile the library picks by itself. Measurement infrastructure, not a
test: it checks that the automatic choice (a cost model of MFMA time, L2
reads per CU and rounds of workgroups) lands on the fastest tile.

    python3 tests/probes/tile_grid.py

Shapes: M in 256..4096 tokens against (N, K) of 2048x4096, 4096x4096,
8192x4096 and 12288x3072; seeded uniform int8 codes, per-token scales in
[0.5, 1.5), a bf16-quantized Gaussian weight, bf16 output, no bias. For each
shape every tile's output is compared bit for bit with tile 0's, then the
tiles are timed interleaved, three rounds of back-to-back launches (HIP
events on the launch stream), and the median is printed. One JSON line per
shape.
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from w8a8_int8_dynamic_amd import _lib, ops  # noqa: E402


def main() -> int:
    import torch
    if not torch.cuda.is_available():
        print("no GPU", file=sys.stderr)
        return 2
    lib = _lib.lib()
    stream = torch.cuda.current_stream().cuda_stream
    main_tiles = [t for t in range(ops.tile_count()) if not ops.tile_name(t).startswith("s")]
    names = {t: ops.tile_name(t) for t in main_tiles}
    shapes = [(M, N, K) for M in (256, 512, 1024, 2048, 4096)
              for (N, K) in ((2048, 4096), (4096, 4096), (8192, 4096), (12288, 3072))]
    for (M, N, K) in shapes:
        g = torch.Generator().manual_seed(M * 7 + N)
        xq = torch.randint(-127, 128, (M, K), generator=g, dtype=torch.int8).cuda()
        xs = torch.rand(M, generator=g).cuda() + 0.5
        w = torch.randn(N, K, generator=g).cuda()
        packed, ws = ops.quant_prepack_weight(w)
        out = {t: torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for t in main_tiles}
        calls = {t: bench.Bound(lib.int8_scaled_mm_tile, xq.data_ptr(), K, xs.data_ptr(),
                                packed.data_ptr(), ws.data_ptr(), None, M, N, K, 0,
                                out[t].data_ptr(), N, stream, t) for t in main_tiles}
        for c in calls.values():
            c()
        torch.cuda.synchronize()
        first = main_tiles[0]
        same = all(torch.equal(out[t].view(torch.int16), out[first].view(torch.int16))
                   for t in main_tiles)
        iters = max(20, min(500, int(20000 / max(1.0, 2.0 * M * N * K / 2e9))))
        bench.settle(torch, calls[first], 0.1)
        times = {t: [] for t in main_tiles}
        for _ in range(3):
            for t, c in calls.items():
                times[t].append(bench.time_loop(torch, c, iters) * 1e3)
        med = {names[t]: round(float(np.median(v)), 2) for t, v in times.items()}
        auto = names[ops.tile_auto(M, N, K)]
        best = min(med, key=med.get)
        print(json.dumps({"M": M, "N": N, "K": K, "identical": same, "auto": auto, "best": best,
                          "auto_over_best": round(med[auto] / med[best], 3), "us": med}),
              flush=True)
        if not same:
            return 1
    return 0


if __name__ == "__main__":
    sys.exit(main())
