"""Per-workgroup phase timeline of the main matmul kernel on one workload:
the one-launch quant + matmul (int8_quant_scaled_mm) and the matmul alone
(int8_scaled_mm), from the measurement twin of the library
(libw8a8_timeline.so: the same kernels with clock stamps at their phase
boundaries, see csrc/timeline.hpp). Measurement infrastructure, not a test.

    python3 tests/probes/fused_timeline.py [workload] [--reps N]

Each form runs N times back to back (the records hold the last launch);
then both are timed with HIP events over 200 launches. Every output is
checked bit for bit against the library proper. Prints JSON lines: per
phase, the min / median / max over workgroups of the stamp (us after the
first workgroup's start) and of the phase's duration per workgroup, and the
shader clock per workgroup (s_memtime cycles over s_memrealtime time).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

SLOTS = 16            # words per workgroup record (timeline.hpp)
MAX_BLOCKS = 16384
STAMPS = ["start", "quantized", "published", "waited", "prologue_done", "loop_done", "end"]


def stats(v):
    return {"min": round(float(np.min(v)), 3), "med": round(float(np.median(v)), 3),
            "max": round(float(np.max(v)), 3)}


def summarize(rec: np.ndarray, fused: bool) -> dict:
    if fused and np.any(rec[:, 1] == 0):
        return {"error": "no stamps of the one-launch path: the launch took the two-step form"}
    rt = rec[:, :8].astype(np.int64)          # 100 MHz clock
    mt = rec[:, 8:15].astype(np.int64)        # shader cycles
    us = (rt - rt[:, 0].min()) * 0.01
    out = {}
    for i, name in enumerate(STAMPS):
        if fused or i in (0, 4, 5, 6):
            out[name] = stats(us[:, i])
    phases = ([("quant", 0, 1), ("publish", 1, 2), ("wait", 2, 3), ("prologue", 3, 4)] if fused
              else [("prologue", 0, 4)]) + [("loop", 4, 5), ("epilogue", 5, 6), ("total", 0, 6)]
    out["phase_us"] = {n: stats((rt[:, j] - rt[:, i]) * 0.01) for n, i, j in phases}
    out["sclk_ghz"] = stats((mt[:, 6] - mt[:, 0]) / ((rt[:, 6] - rt[:, 0]) * 10.0))
    if fused:
        out["first_seen_after_last_publish_us"] = round(float(us[:, 3].min() - us[:, 2].max()), 3)
    xcc = (rec[:, 15] >> np.uint64(32)).astype(np.int64) & 0xF
    out["xcc_is_block_mod_8"] = float(np.mean(xcc == (np.arange(len(rec)) % 8)))
    out["span_us"] = round(float(us[:, 6].max()), 3)
    return out


def main(argv=None) -> int:
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("workload", nargs="?", default="fused_qkv")
    p.add_argument("--reps", type=int, default=300)
    p.add_argument("--save", metavar="DIR", default=None,
                   help="also write each form's raw records (uint64 [workgroups, 16]) as .npy")
    args = p.parse_args(argv)

    import torch
    import workloads as wl
    from w8a8_int8_dynamic_amd import _lib, ops

    lib_path = os.path.join(ROOT, "w8a8_int8_dynamic_amd", "libw8a8_timeline.so")
    if not os.path.exists(lib_path):
        print("libw8a8_timeline.so is not built (w8a8_int8_dynamic_amd/build.py)", file=sys.stderr)
        return 1
    T = ctypes.CDLL(lib_path)
    for name, sig in (("int8_quant_scaled_mm_tile", _lib.SIGNATURES["int8_quant_scaled_mm_tile"]),
                      ("int8_scaled_mm_tile", _lib.SIGNATURES["int8_scaled_mm_tile"])):
        fn = getattr(T, name)
        fn.restype, fn.argtypes = sig
    T.w8a8_timeline_read.restype = ctypes.c_int
    T.w8a8_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]

    w = wl.by_name(args.workload)
    M, K, N = w.M, w.K, w.N
    inp = wl.generate(w)
    x = torch.from_numpy(inp.x_bf16.view(np.int16)).view(torch.bfloat16).cuda()
    bias = None if inp.bias_bf16 is None else \
        torch.from_numpy(inp.bias_bf16.view(np.int16)).view(torch.bfloat16).cuda()
    wq, ws = ops.quant_per_channel(torch.from_numpy(inp.w_f32).cuda())
    packed = ops.prepack_weight(wq)
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    xs = torch.empty((M,), dtype=torch.float32, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    tile = ops.tile_auto(M, N, K)
    bm, bn = (int(v) for v in ops.tile_name(tile).split("/")[0].split("x"))
    grid = -(-M // bm) * -(-N // bn)
    if grid > MAX_BLOCKS or not ops.tile_name(tile)[0].isdigit():
        print(f"{args.workload}: tile {ops.tile_name(tile)} with {grid} workgroups is not "
              f"recorded (main kernel, at most {MAX_BLOCKS} workgroups)", file=sys.stderr)
        return 1
    bptr = None if bias is None else bias.data_ptr()

    def fused():
        r = T.int8_quant_scaled_mm_tile(x.data_ptr(), K, xq.data_ptr(), K, xs.data_ptr(),
                                        packed.data_ptr(), ws.data_ptr(), bptr, M, N, K, 0,
                                        out.data_ptr(), N, stream, tile)
        assert r == 0, r

    def plain():
        r = T.int8_scaled_mm_tile(xq.data_ptr(), K, xs.data_ptr(), packed.data_ptr(),
                                  ws.data_ptr(), bptr, M, N, K, 0, out.data_ptr(), N, stream, tile)
        assert r == 0, r

    ref = ops.quant_scaled_mm(x, packed, ws, N, bias=bias)[0]
    torch.cuda.synchronize()
    print(json.dumps({"workload": w.description, "tile": ops.tile_name(tile), "grid": grid,
                      "reps": args.reps}), flush=True)
    for label, fn in (("int8_quant_scaled_mm", fused), ("int8_scaled_mm", plain)):
        out.zero_()
        for _ in range(args.reps):
            fn()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"{label}: output differs"
        buf = np.zeros(grid * SLOTS, dtype=np.uint64)
        err = T.w8a8_timeline_read(buf.ctypes.data, buf.nbytes)
        assert err == 0, err
        rec = {"form": label}
        rec.update(summarize(buf.reshape(grid, SLOTS), label == "int8_quant_scaled_mm"))
        if args.save:
            os.makedirs(args.save, exist_ok=True)
            np.save(os.path.join(args.save, f"timeline_{args.workload}_{label}.npy"),
                    buf.reshape(grid, SLOTS))
        print(json.dumps(rec), flush=True)
    for label, fn in (("int8_quant_scaled_mm", fused), ("int8_scaled_mm", plain)):
        for _ in range(50):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(200):
            fn()
        b.record()
        torch.cuda.synchronize()
        print(json.dumps({"form": label, "us_per_launch_events": round(a.elapsed_time(b) * 5.0, 3)}),
              flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
