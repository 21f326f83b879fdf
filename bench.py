#!/usr/bin/env python3
"""Benchmark of the W8A8 int8-dynamic linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload fused_qkv]

One step is the whole hot path on one batch: the per-token activation quant
and the int8 MFMA matmul with its fused scale/bias/bf16 epilogue, issued as
one library call (int8_quant_scaled_mm: a single launch when the matmul's
grid fits the device, else the two kernels back to back). The weight is
quantized per output channel and repacked once, before timing. Inputs are
seeded synthetic tensors (workloads/), already resident in HBM when the
timed region starts. After the --warmup steps the step keeps running,
untimed, for 0.3 s so that the timed loops start at steady clocks. The
default of 2000 timed steps (about 70 ms) averages over the part's power
management, which moves 200-step loops of the same step by up to 10 %.

Printed: one JSON line with the step throughput (int8 TOP/s of 2*M*N*K per
step), the same step as two separate calls, the roofline of the matmul
kernel (int8_scaled_mm alone: its average launch duration from HIP events on
the launch stream), the quant pass's GB/s, the same layer at one token
(decode: the small-M kernel, weights streamed from HBM), and the CPU oracle
timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, TOP/s
PEAK_HBM_GBPS = 8000.0       # MI355X HBM3E, GB/s


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000,
                   help="timed steps (2000: about 70 ms of back-to-back steps on the default workload; 200-step loops vary by up to 10 %% with the part's power state)")
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="fused_qkv")
    p.add_argument("--tile", type=int, default=-1, help="force a matmul tile id (-1 = automatic)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target wall time of the oracle's sampled GEMM")
    p.add_argument("--no-quant-large", action="store_true",
                   help="skip the quant bandwidth run on the FFN-down activations")
    p.add_argument("--hw-probes", action="store_true",
                   help="run the memory-path probes (tests/probes/hw_probes) and print their results")
    p.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV", default=None,
                   help="print the summary of a rocprofv3 kernel trace of a bench run (no GPU)")
    p.add_argument("--no-workloads", action="store_true",
                   help="skip the per-workload GPU and oracle records and the accuracy record")
    p.add_argument("--no-decode", action="store_true",
                   help="skip the one-token (decode) measurement of the fused-QKV layer")
    p.add_argument("--only", choices=["step", "step2", "mm", "mm8", "quant", "copy", "decode"],
                   default=None,
                   help="launch only this part in a loop (for profiler runs); 'copy' is a "
                        "plain 256 MiB device copy kernel, the calibration for HBM byte "
                        "counters; 'decode' is the one-token fused-QKV step; 'mm8' is the "
                        "e4m3 twin's scaled matmul on the same layer")
    return p.parse_args(argv)


def world_size() -> int:
    return int(os.environ.get("WORLD_SIZE", "1"))


def source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "w8a8_int8_dynamic_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


class Bound:
    """A libw8a8 entry point with its arguments marshalled once."""

    def __init__(self, fn, *args):
        self.fn, self.args = fn, args

    def __call__(self):
        rc = self.fn(*self.args)
        if rc != 0:
            from w8a8_int8_dynamic_amd import _lib
            raise RuntimeError(f"{self.fn.__name__} failed: {_lib.last_error()}")


def time_loop(torch, fn, iters: int) -> float:
    """Average milliseconds per call of fn over iters back-to-back calls, from
    HIP events recorded on torch's current stream (the launch stream)."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(iters):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / iters


def settle(torch, fn, seconds: float = 0.3) -> None:
    """Keep calling fn, untimed, in short synchronized batches for `seconds` of
    wall time, so that the first timed loop starts at the GPU's steady
    clocks (measured: after a few milliseconds of warmup the first loop of
    the FFN-down step ran 10 % slower than every later one)."""
    end = time.perf_counter() + seconds
    while time.perf_counter() < end:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def time_each(torch, fn, iters: int):
    """Median and minimum microseconds of single launches of fn, each
    bracketed by its own pair of HIP events on the launch stream. An isolated
    launch pays its own ramp and the events' cost, so these sit above the
    back-to-back mean that the throughput figures use."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    return round(float(np.median(us)), 3), round(us[0], 3)


def sclk_under_load(torch, fn, seconds: float = 1.0) -> dict:
    """The shader clock while fn runs back to back: amd-smi's per-XCD gfx
    clocks, sampled a few times from the host while another thread keeps
    the GPU busy. None fields when amd-smi is unavailable."""
    import subprocess
    import threading
    stop = threading.Event()

    def busy():
        while not stop.is_set():
            for _ in range(64):
                fn()
            torch.cuda.synchronize()

    t = threading.Thread(target=busy)
    t.start()
    samples, err = [], None
    try:
        time.sleep(0.2)
        end = time.perf_counter() + seconds
        while time.perf_counter() < end:
            r = subprocess.run(["amd-smi", "metric", "--clock", "--json"], capture_output=True,
                               text=True, timeout=10)
            if r.returncode != 0:
                err = r.stderr.strip()[:120]
                break
            data = json.loads(r.stdout)
            gpus = data["gpu_data"] if isinstance(data, dict) else data
            clk = gpus[0]["clock"]
            samples.append([v["clk"]["value"] for k, v in sorted(clk.items())
                            if k.startswith("gfx_") and isinstance(v.get("clk"), dict)
                            and isinstance(v["clk"].get("value"), (int, float))])
    except Exception as ex:                        # a tool missing or an unexpected format
        err = f"{type(ex).__name__}: {ex}"[:120]
    finally:
        stop.set()
        t.join()
    vals = [v for smp in samples for v in smp]
    return {"mhz_mean": round(float(np.mean(vals)), 1) if vals else None,
            "mhz_min": min(vals) if vals else None, "mhz_max": max(vals) if vals else None,
            "samples": len(samples), "xcds": len(samples[-1]) if samples else 0,
            "source": "amd-smi metric --clock (gfx clocks of every XCD) while the step runs "
                      "back to back", **({"error": err} if err else {})}


def sha16(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()[:16]


def dev_bf16(torch, bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def cpu_baseline(w, inp, target_s: float) -> dict:
    """The oracle (as it stands) on a bounded sample of the workload.

    A step of the oracle is the full per-token quant, the exact int32 GEMM and
    the fp32 epilogue. When one full step takes less than target_s seconds,
    whole steps are repeated until target_s has passed and the mean is taken;
    otherwise the GEMM and epilogue run on a sample of token rows sized to
    about target_s seconds and are scaled to all M rows. Returns int8 TOP/s of
    2*M*N*K per step.
    """
    import oracle
    o = oracle.load()
    wq, ws = o.quant_per_channel(inp.w_f32)        # offline weight prep, not timed
    rng = np.random.default_rng(w.seed)

    parts = {"quant": 0.0, "gemm": 0.0, "epilogue": 0.0}

    def step(rows):
        t0 = time.perf_counter()
        xq, xs = o.quant_per_token(inp.x_bf16)
        t1 = time.perf_counter()
        acc = o.gemm_i32(xq, wq, rows)
        t2 = time.perf_counter()
        o.epilogue_f32(acc, xs if rows is None else xs[rows], ws, inp.bias_bf16)
        t3 = time.perf_counter()
        parts["quant"] += t1 - t0
        parts["gemm"] += t2 - t1
        parts["epilogue"] += t3 - t2
        return t1 - t0, t3 - t1

    xq, _ = o.quant_per_token(inp.x_bf16)
    probe = np.sort(rng.choice(w.M, min(w.M, 4), replace=False))
    t0 = time.perf_counter()
    o.gemm_i32(xq, wq, probe)
    per_row = (time.perf_counter() - t0) / len(probe)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    if per_row * w.M < target_s / 2:
        reps, t_sum, start = 0, 0.0, time.perf_counter()
        while reps == 0 or time.perf_counter() - start < target_s:
            tq, tg = step(None)
            t_sum += tq + tg
            reps += 1
        t_total = t_sum / reps
        scale = 1.0
        sample = (f"{reps} full oracle steps (per-token quant of X [{w.M},{w.K}], exact int32 "
                  f"GEMM and fp32 epilogue on all rows), {t_sum:.1f} s measured, mean per step")
    else:
        n_rows = int(min(w.M, max(4, target_s / 2 / max(per_row, 1e-9))))
        rows = np.sort(rng.choice(w.M, n_rows, replace=False))
        reps, tq_sum, tg_sum, start = 0, 0.0, 0.0, time.perf_counter()
        while reps == 0 or time.perf_counter() - start < target_s:
            tq, tg = step(rows)
            tq_sum, tg_sum, reps = tq_sum + tq, tg_sum + tg, reps + 1
        scale = w.M / n_rows
        t_total = (tq_sum + tg_sum * scale) / reps
        sample = (f"{reps} x (full per-token quant of X [{w.M},{w.K}] plus exact int32 GEMM "
                  f"and fp32 epilogue on {n_rows} of {w.M} token rows, x{scale:.2f} to all "
                  f"rows); {tq_sum + tg_sum:.1f} s measured, mean per step")
    t_quant = parts["quant"] / reps
    t_gemm = parts["gemm"] * scale / reps
    t_epi = parts["epilogue"] * scale / reps
    return {
        "value": round(w.ops / t_total / 1e12, 6),
        "unit": "TOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": sample,
        "seconds_per_step": round(t_total, 4),
        "cpu_model": cpu_model(),
        "parts_per_full_step": {
            "quant_s": sig4(t_quant), "quant_gbps": sig4((3 * w.M * w.K + 4 * w.M) / t_quant / 1e9),
            "gemm_s": sig4(t_gemm), "gemm_gops": sig4(w.ops / t_gemm / 1e9),
            "epilogue_s": sig4(t_epi),
        },
    }


def sig4(v: float) -> float:
    return float(f"{v:.4g}")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_reference(torch, steps: int) -> dict:
    """A plain device copy kernel (torch neg) over 256 MiB in and 256 MiB out:
    the achievable-bandwidth reference for the HBM-bound quant pass."""
    src = torch.ones((64 << 20,), dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    ms = time_loop(torch, lambda: torch.neg(src, out=dst), max(10, min(steps, 50)))
    nbytes = 2 * src.numel() * 4
    del src, dst
    torch.cuda.empty_cache()
    return {"gbps": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes": nbytes,
            "frac_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}


def traffic_record(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, when they
    were taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    entry = rec.get(f"{kernel}:{workload}")
    if not entry or entry.get("source_digest") != source_digest():
        return None
    return entry.get("bytes_per_launch")


def omp_threads(n=None) -> int:
    """OpenMP threads of the oracle's parallel regions started from this
    thread: set to n when given; returns the current maximum."""
    gomp = ctypes.CDLL("libgomp.so.1")
    if n is not None:
        gomp.omp_set_num_threads(int(n))
    return int(gomp.omp_get_max_threads())


def workload_records(torch, L, ops, wl, steps: int) -> dict:
    """Every workload at full size on the GPU: the step (int8_quant_scaled_mm,
    one call), the two separate calls, int8_scaled_mm alone and the per-token
    quant alone, each as the mean of back-to-back launches from HIP events on
    the launch stream, with TOP/s and the fraction of the int8 MFMA peak
    (matmul) or of HBM (quant). Inputs are resident in HBM; for the two
    largest workloads the whole set fits the 256 MB last-level cache only in
    part, so these are the figures of an ordinary layer call."""
    recs = {}
    stream = torch.cuda.current_stream().cuda_stream
    for w in wl.WORKLOADS:
        M, K, N = w.M, w.K, w.N
        inp = wl.generate(w)
        x = dev_bf16(torch, inp.x_bf16)
        bias = None if inp.bias_bf16 is None else dev_bf16(torch, inp.bias_bf16)
        packed, ws = ops.quant_prepack_weight(torch.from_numpy(inp.w_f32).cuda())
        xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
        xs = torch.empty((M,), dtype=torch.float32, device="cuda")
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        bp = None if bias is None else bias.data_ptr()
        tile = ops.tile_auto(M, N, K)
        quant = Bound(L.int8_quant_per_token, x.data_ptr(), M, K, K, xq.data_ptr(), K,
                      xs.data_ptr(), stream)
        step = Bound(L.int8_quant_scaled_mm, x.data_ptr(), K, xq.data_ptr(), K, xs.data_ptr(),
                     packed.data_ptr(), ws.data_ptr(), bp, M, N, K, 0, out.data_ptr(), N, stream)
        mm = Bound(L.int8_scaled_mm, xq.data_ptr(), K, xs.data_ptr(), packed.data_ptr(),
                   ws.data_ptr(), bp, M, N, K, 0, out.data_ptr(), N, stream)

        def two():
            quant()
            mm()

        iters = max(10, min(steps, int(20000 / max(1.0, w.ops / 2.0e9))))
        settle(torch, step, 0.15)
        t_step = time_loop(torch, step, iters)
        t_two = time_loop(torch, two, iters)
        t_mm = time_loop(torch, mm, iters)
        t_q = time_loop(torch, quant, iters)
        qbytes = 3 * M * K + 4 * M
        tops = w.ops / (t_mm * 1e-3) / 1e12
        recs[w.name] = {
            "M": M, "K": K, "N": N, "tile": ops.tile_name(tile), "launches": iters,
            "step_us": round(t_step * 1e3, 3),
            "step_tops": round(w.ops / (t_step * 1e-3) / 1e12, 1),
            "two_calls_us": round(t_two * 1e3, 3),
            "scaled_mm_us": round(t_mm * 1e3, 3), "scaled_mm_tops": round(tops, 1),
            "scaled_mm_frac_mfma_peak": round(tops / PEAK_INT8_TOPS, 4),
            "quant_us": round(t_q * 1e3, 3),
            "quant_gbps": round(qbytes / (t_q * 1e-3) / 1e9, 1),
            "quant_frac_hbm_peak": round(qbytes / (t_q * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        }
        del x, bias, packed, ws, xq, xs, out
        torch.cuda.empty_cache()
    return recs


def oracle_records(wl, target_s: float = 2.5) -> dict:
    """The oracle on every workload, on all host cores and (for the three
    smaller workloads) on one core: per-token quant of all rows, then the
    exact int32 GEMM and fp32 epilogue on a sample of token rows sized to
    about target_s seconds, scaled to all rows (all rows when a full step is
    shorter). int8 TOP/s of 2*M*N*K per full step."""
    import oracle
    o = oracle.load()
    full = omp_threads()
    recs = {"build_flags": " ".join(oracle.CFLAGS), "cpu_model": cpu_model(),
            "threads_all": full}
    for w in wl.WORKLOADS:
        inp = wl.generate(w)
        wq, ws = o.quant_per_channel(inp.w_f32)
        rng = np.random.default_rng(w.seed + 77)
        rec = {}
        for label, threads in (("all_cores", full), ("one_core", 1)):
            if label == "one_core" and w.name not in ("tiny", "attn_out", "fused_qkv"):
                continue
            omp_threads(threads)
            t0 = time.perf_counter()
            xq, xs = o.quant_per_token(inp.x_bf16)
            tq = time.perf_counter() - t0
            probe = np.sort(rng.choice(w.M, min(w.M, 2), replace=False))
            t0 = time.perf_counter()
            o.gemm_i32(xq, wq, probe)
            per_row = (time.perf_counter() - t0) / len(probe)
            n_rows = int(min(w.M, max(2, target_s / max(per_row, 1e-9))))
            rows = None if n_rows >= w.M else np.sort(rng.choice(w.M, n_rows, replace=False))
            t0 = time.perf_counter()
            acc = o.gemm_i32(xq, wq, rows)
            o.epilogue_f32(acc, xs if rows is None else xs[rows], ws, inp.bias_bf16)
            tg = (time.perf_counter() - t0) * (w.M / (w.M if rows is None else n_rows))
            rec[label] = {"threads": threads, "seconds_per_step": sig4(tq + tg),
                          "tops": sig4(w.ops / (tq + tg) / 1e12),
                          "quant_gbps": sig4((3 * w.M * w.K + 4 * w.M) / tq / 1e9),
                          "rows_timed": w.M if rows is None else n_rows}
        omp_threads(full)
        recs[w.name] = rec
    return recs


def accuracy_record(torch, ops, wl) -> dict:
    """Rel-L2 of the fused-QKV layer's bf16 output (the product path, every
    element) against fp32 matmuls (NumPy float32 GEMM) of the dequantized
    operands (xq*xs)(wq*ws)^T and of the raw bf16 X and fp32 W, next to the
    0.17 % the pages report for their raw-op check against a float32
    reference. The first is the bf16 output rounding (plus the fp32
    reference's own rounding); the second adds the quantization error."""
    w = wl.by_name("fused_qkv")
    inp = wl.generate(w)
    from w8a8_int8_dynamic_amd import W8A8Linear
    layer = W8A8Linear.from_float(torch.from_numpy(inp.w_f32).cuda())
    x = dev_bf16(torch, inp.x_bf16)
    out = layer(x)
    xq, xs = ops.quant_per_token(x)
    wq = ops.unpack_weight(layer.w_packed, w.N, w.K)
    g = out.float().cpu().numpy().astype(np.float64)
    a = (xq.cpu().numpy().astype(np.float32) * xs.cpu().numpy()[:, None])
    b = (wq.cpu().numpy().astype(np.float32) * layer.w_scale.cpu().numpy()[:, None])
    deq = (a @ b.T).astype(np.float64)
    raw = (wl.bf16_bits_to_f32(inp.x_bf16) @ inp.w_f32.T).astype(np.float64)

    def rel(r):
        return float(np.linalg.norm(g - r) / np.linalg.norm(r))

    return {"workload": w.description,
            "rel_l2_vs_fp32_dequantized_matmul_pct": round(100 * rel(deq), 4),
            "rel_l2_vs_fp32_raw_matmul_pct": round(100 * rel(raw), 3),
            "pages_rel_l2_pct": 0.17,
            "reading": "the pages' figure is read as the bf16 rounding of the output against "
                       "a float32 matmul of the dequantized operands"}


def trace_summary(path: str) -> str:
    """Summary of a rocprofv3 kernel trace (its kernel_trace.csv) of a bench
    run: per kernel, the dispatch count and mean / min / max duration, over
    the whole run, over the timed step loop alone (the dispatches between
    the first two bitwise_not marker launches) and over the roofline's
    matmul loop (between the third and fourth), with each loop's
    start-to-start period. Markdown text."""
    import csv
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))
    marks = [i for i, r in enumerate(rows) if "bitwise_not" in r["Kernel_Name"]]

    def short(name: str) -> str:
        name = name.replace("(anonymous namespace)::", "").replace("w8a8::", "")
        return name.split("(")[0].replace("void ", "")

    def table(sel, title):
        by = {}
        for r in sel:
            by.setdefault(short(r["Kernel_Name"]), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        out = [f"{title}", "", "| kernel | dispatches | mean us | min us | max us |",
               "|---|---|---|---|---|"]
        for k, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
            out.append(f"| `{k}` | {len(v)} | {np.mean(v):.3f} | {min(v):.3f} | {max(v):.3f} |")
        return out

    lines = table(rows, "All dispatches of the run:")
    for a, b, what in ((0, 1, "timed step loop"), (2, 3, "roofline's matmul loop")):
        if len(marks) <= b:
            break
        loop = rows[marks[a] + 1:marks[b]]
        starts = [int(r["Start_Timestamp"]) for r in loop]
        ends = [int(r["End_Timestamp"]) for r in loop]
        lines += [""] + table(loop, f"The {what} (between markers {a + 1} and {b + 1}):")
        if len(loop) > 1:
            lines += ["", f"{what[0].upper() + what[1:]}: {len(loop)} dispatches, first start to last end "
                          f"{(ends[-1] - starts[0]) / 1e3:.3f} us, "
                          f"{(ends[-1] - starts[0]) / 1e3 / len(loop):.3f} us per dispatch; mean "
                          f"start-to-start period {(starts[-1] - starts[0]) / 1e3 / (len(loop) - 1):.3f} us."]
    return "\n".join(lines)


def main(argv=None) -> int:
    args = parse_args(argv)
    if args.hw_probes:
        import subprocess
        exe = os.path.join(ROOT, "tests", "probes", "hw_probes")
        if not os.path.exists(exe):
            print("tests/probes/hw_probes is not built (__graft_entry__.build())", file=sys.stderr)
            return 1
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
        if r.returncode != 0:
            print(r.stderr, file=sys.stderr)
            return r.returncode
        print(json.dumps({"hw_probes": [json.loads(l) for l in r.stdout.splitlines() if l.strip()]}))
        return 0
    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return 0
    if args.gpus != 1 or world_size() != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world_size()}); the library has no multi-GPU path.", file=sys.stderr)
        return 2

    import torch
    import workloads as wl
    from w8a8_int8_dynamic_amd import _lib, ops

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    L = _lib.lib()
    dev = torch.cuda.current_device()
    if not ops.device_supported(dev):
        print("the current device is not gfx950", file=sys.stderr)
        return 1

    w = wl.by_name(args.workload)
    M, K, N = w.M, w.K, w.N
    inp = wl.generate(w)
    x = dev_bf16(torch, inp.x_bf16)
    bias = None if inp.bias_bf16 is None else dev_bf16(torch, inp.bias_bf16)
    wq, ws = ops.quant_per_channel(torch.from_numpy(inp.w_f32).cuda())   # load time
    packed = ops.prepack_weight(wq)
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    xs = torch.empty((M,), dtype=torch.float32, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    tile = args.tile if args.tile >= 0 else ops.tile_auto(M, N, K)

    quant = Bound(L.int8_quant_per_token, x.data_ptr(), M, K, K, xq.data_ptr(), K, xs.data_ptr(),
                  stream)
    fused = Bound(L.int8_quant_scaled_mm_tile, x.data_ptr(), K, xq.data_ptr(), K, xs.data_ptr(),
                  packed.data_ptr(), ws.data_ptr(), None if bias is None else bias.data_ptr(),
                  M, N, K, 0, out.data_ptr(), N, stream, tile)
    mm = Bound(L.int8_scaled_mm_tile, xq.data_ptr(), K, xs.data_ptr(), packed.data_ptr(),
               ws.data_ptr(), None if bias is None else bias.data_ptr(), M, N, K, 0,
               out.data_ptr(), N, stream, tile)

    def step():                    # the layer's forward: one library call
        fused()

    def step_two_calls():
        quant()
        mm()

    if args.only == "decode":
        n = args.warmup + args.steps
        decode_record(torch, ops, launches=n)
        print(json.dumps({"only": "decode", "launches": n, "workload": "fused_qkv, M=1"}),
              flush=True)
        return 0
    if args.only:
        copy_src = copy_dst = None
        if args.only == "copy":
            copy_src = torch.ones((64 << 20,), dtype=torch.float32, device="cuda")
            copy_dst = torch.empty_like(copy_src)
        mm8 = None
        if args.only == "mm8":
            packed8, ws8 = ops.fp8_quant_prepack_weight(torch.from_numpy(inp.w_f32).cuda())
            xq8, xs8 = ops.fp8_quant_per_token(x)
            mm8 = Bound(L.fp8_scaled_mm_tile, xq8.data_ptr(), xq8.stride(0), xs8.data_ptr(),
                        packed8.data_ptr(), ws8.data_ptr(),
                        None if bias is None else bias.data_ptr(), M, N, K, 0, out.data_ptr(), N,
                        stream, tile)
        fn = {"step": step, "step2": step_two_calls, "mm": mm, "mm8": mm8, "quant": quant,
              "copy": lambda: torch.neg(copy_src, out=copy_dst)}[args.only]
        for _ in range(args.warmup + args.steps):
            fn()
        torch.cuda.synchronize()
        print(json.dumps({"only": args.only, "launches": args.warmup + args.steps,
                          "workload": w.name, "tile": ops.tile_name(tile),
                          "copy_bytes_each_way": None if copy_src is None else
                          copy_src.numel() * 4}), flush=True)
        return 0

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    settle(torch, step)
    # Two launches of a kernel used nowhere else bracket the timed step loop,
    # so a kernel trace of this run can pick out exactly its dispatches.
    marker = torch.zeros((7,), dtype=torch.int16, device="cuda")
    torch.bitwise_not(marker, out=marker)
    ms_step = time_loop(torch, step, args.steps)
    torch.bitwise_not(marker, out=marker)
    ms_step2 = time_loop(torch, step_two_calls, args.steps)
    torch.bitwise_not(marker, out=marker)      # the matmul loop of the roofline: markers 3 and 4
    ms_mm = time_loop(torch, mm, args.steps)
    torch.bitwise_not(marker, out=marker)
    ms_quant = time_loop(torch, quant, args.steps)
    each = {name: time_each(torch, fn, min(args.steps, 100))
            for name, fn in (("step", step), ("mm", mm), ("quant", quant))}

    # Cold variant of the matmul: rotate over weight copies larger than the
    # 256 MB last-level cache so each launch streams its weight from HBM.
    copies = max(2, int(np.ceil(512e6 / packed.numel())))
    cold_packs = [packed.clone() for _ in range(min(copies, 16))]
    cold_calls = [Bound(L.int8_scaled_mm_tile, xq.data_ptr(), K, xs.data_ptr(), p.data_ptr(),
                        ws.data_ptr(), None if bias is None else bias.data_ptr(), M, N, K, 0,
                        out.data_ptr(), N, stream, tile) for p in cold_packs]
    it = iter(range(1 << 30))
    ms_mm_cold = time_loop(torch, lambda: cold_calls[next(it) % len(cold_calls)](), args.steps)
    del cold_packs, cold_calls

    # Context only: the vendor library's int8 GEMM (torch._int_mm, int32
    # output, no scale epilogue) on the same operands.
    vendor = None
    try:
        wt = wq.t()
        torch._int_mm(xq, wt)
        vendor_ms = time_loop(torch, lambda: torch._int_mm(xq, wt), args.steps)
        vendor = {"op": "torch._int_mm(xq [M,K], wq[N,K].T) -> int32, no epilogue",
                  "us": round(vendor_ms * 1e3, 3),
                  "tops": round(2 * M * N * K / (vendor_ms * 1e-3) / 1e12, 2)}
    except Exception as ex:                        # not every shape is supported
        vendor = {"op": "torch._int_mm", "error": str(ex)[:160]}
    inputs_sha = {"x_bf16": sha16(inp.x_bf16), "wq": sha16(wq.cpu().numpy()),
                  "ws": sha16(ws.cpu().numpy()),
                  "bias_bf16": None if inp.bias_bf16 is None else sha16(inp.bias_bf16),
                  "digest": "first 16 hex of sha256 over the bytes"}
    del wq

    quant_bytes = 3 * M * K + 4 * M
    mm_ops = 2 * M * N * K
    mm_min_bytes = M * K + packed.numel() + 4 * M + 4 * N + 2 * M * N + (0 if bias is None else 2 * N)
    achieved = mm_ops / (ms_mm * 1e-3) / 1e12
    rec = {
        "metric": "int8 TOPS + % MFMA peak of quant+scaled_mm at M512 K4096 N12288; quant GB/s",
        "value": round(mm_ops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded; workloads/ recipe), weights quantized per channel on the GPU",
        "config": {"workload": w.description, "M": M, "K": K, "N": N,
                   "bias": bias is not None, "tile": ops.tile_name(tile),
                   "step": "int8_quant_scaled_mm: per-token quant + scaled matmul (bf16 out), "
                           "one call"},
        "pct_mfma_peak_step": round(100 * mm_ops / (ms_step * 1e-3) / 1e12 / PEAK_INT8_TOPS, 2),
        "step_us_isolated_median": each["step"][0], "step_us_isolated_min": each["step"][1],
        "step_two_calls": {"us": round(ms_step2 * 1e3, 3),
                           "tops": round(mm_ops / (ms_step2 * 1e-3) / 1e12, 2),
                           "calls": "int8_quant_per_token then int8_scaled_mm"},
        "scaled_mm": {"us": round(ms_mm * 1e3, 3), "tops": round(achieved, 2),
                      "us_isolated_median": each["mm"][0], "us_isolated_min": each["mm"][1],
                      "us_cold": round(ms_mm_cold * 1e3, 3),
                      "tops_cold": round(mm_ops / (ms_mm_cold * 1e-3) / 1e12, 2),
                      "min_hbm_bytes": mm_min_bytes},
        "quant": {"us": round(ms_quant * 1e3, 3), "us_isolated_median": each["quant"][0],
                  "us_isolated_min": each["quant"][1],
                  "gbps": round(quant_bytes / (ms_quant * 1e-3) / 1e9, 1),
                  "bytes": quant_bytes},
        "roofline": {
            "kernel": "int8_scaled_mm",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_INT8_TOPS,
            "unit": "TOP/s",
            "frac": round(achieved / PEAK_INT8_TOPS, 4),
            "traffic": traffic_record("int8_scaled_mm", w.name),
        },
        "vendor_int8_gemm": vendor,
        "source_digest": source_digest(),
        "inputs_sha256": inputs_sha,
        "sclk_under_load": sclk_under_load(torch, step),
    }

    if not args.no_decode:
        rec["decode"] = decode_record(torch, ops)
        rec["decode_ffn_down"] = decode_record(torch, ops, M=8, N=3072, K=12288,
                                               label="FFN down-projection")
    if not args.no_quant_large:
        rec["quant_large"] = quant_bandwidth(torch, L, wl, stream, args.steps)
        rec["hbm_copy_reference"] = copy_reference(torch, args.steps)
    del x, xq, xs, out, packed
    torch.cuda.empty_cache()
    if not args.no_workloads:
        rec["workloads"] = workload_records(torch, L, ops, wl, args.steps)
        rec["accuracy"] = accuracy_record(torch, ops, wl)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
        rec["cpu_baseline"]["build_flags"] = " ".join(__import__("oracle").CFLAGS)
        if not args.no_workloads:
            rec["oracle_workloads"] = oracle_records(wl)
    print(json.dumps(rec), flush=True)
    return 0


def decode_record(torch, ops, M: int = 1, N: int = 12288, K: int = 4096, launches: int = 0,
                  label: str = "fused-QKV layer") -> dict:
    """A layer at a few tokens (decode): int8_quant_scaled_mm through the
    small-M kernel, with the layer's workspace (K split over workgroups when
    the weight has too few column blocks to keep every CU streaming),
    rotating over weight copies larger than the 256 MB last-level cache
    (each call streams its weight from HBM, as a model's layers would),
    replayed from a HIP graph so that host launch costs stay out of the
    timing. Every replay's output is checked against the eager result.
    Weights and activations are seeded random data of the layer's shape."""
    g = torch.Generator(device="cpu").manual_seed(20251)
    w = torch.randint(-127, 128, (N, K), dtype=torch.int8, generator=g).cuda()
    x = (torch.randn((M, K), generator=g) * 2.0).to(torch.bfloat16).cuda()
    ws = (torch.rand((N,), generator=g) * 1e-3).cuda()
    packed = ops.prepack_weight(w)
    copies = max(2, int(np.ceil(600e6 / packed.numel())))
    packs = [packed] + [packed.clone() for _ in range(copies - 1)]
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    xs = torch.empty((M,), dtype=torch.float32, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    work = ops.new_workspace(N, K, max_rows=M)
    ref = ops.quant_scaled_mm(x, packed, ws, N)[0]
    reps = 2 * copies
    if launches:                   # profiler runs: plain eager launches, nothing timed
        for i in range(launches):
            ops.quant_scaled_mm(x, packs[i % copies], ws, N, out=out, xq=xq, xs=xs, workspace=work)
        torch.cuda.synchronize()
        return {}

    def capture(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(copies):
                fn(packs[i])
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(reps):
                fn(packs[i % copies])
        return graph

    def replay_us(graph, rounds=7):
        ts = []
        for _ in range(rounds):
            out.fill_(0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            if not torch.equal(out.view(torch.int16), ref.view(torch.int16)):
                raise RuntimeError("graph replay of the decode step differs from the eager result")
            ts.append(e0.elapsed_time(e1) * 1e3 / reps)
        return float(np.median(ts))

    step = replay_us(capture(lambda p: ops.quant_scaled_mm(x, p, ws, N, out=out, xq=xq, xs=xs,
                                                           workspace=work)))
    ops.quant_per_token(x, xq, xs)
    mm = replay_us(capture(lambda p: ops.scaled_mm(xq, xs, p, ws, N, out=out, workspace=work)))
    wbytes = packed.numel()
    rec = {"workload": f"{label} at {M} token(s): M={M} K={K} N={N}, bf16 out, no bias",
           "tile": ops.tile_name(ops.tile_auto(M, N, K)),
           "workspace_bytes": ops.workspace_bytes(M, N, K),
           "weight_copies": copies, "timing": "HIP graph replay, median per call",
           "step_us": round(step, 3), "scaled_mm_us": round(mm, 3),
           "weight_bytes": wbytes,
           "step_weight_gbps": round(wbytes / (step * 1e-6) / 1e9, 1),
           "scaled_mm_weight_gbps": round(wbytes / (mm * 1e-6) / 1e9, 1),
           "scaled_mm_frac_hbm_peak": round(wbytes / (mm * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
           "step_traffic": traffic_record("int8_quant_scaled_mm",
                                          ("fused_qkv" if N == 12288 else "ffn_down") + f"_m{M}")}
    del packs, packed, w
    torch.cuda.empty_cache()
    return rec


def quant_bandwidth(torch, L, wl, stream, steps: int) -> dict:
    """int8_quant_per_token on the FFN-down activations [8192, 12288], rotating
    over input/output sets larger than the last-level cache (302 MB moved per
    launch: bf16 read, int8 codes and fp32 scales written)."""
    w = wl.by_name("ffn_down")
    inp = wl.generate(w)
    M, K = w.M, w.K
    x0 = dev_bf16(torch, inp.x_bf16)
    sets = []
    for i in range(3):
        x = x0 if i == 0 else x0.clone()
        sets.append((x, torch.empty((M, K), dtype=torch.int8, device="cuda"),
                     torch.empty((M,), dtype=torch.float32, device="cuda")))
    calls = [Bound(L.int8_quant_per_token, x.data_ptr(), M, K, K, q.data_ptr(), K, s.data_ptr(),
                   stream) for x, q, s in sets]
    for c in calls:
        c()
    it = iter(range(1 << 30))
    iters = max(10, min(steps, 100))
    ms = time_loop(torch, lambda: calls[next(it) % len(calls)](), iters)
    nbytes = 3 * M * K + 4 * M
    gbps = nbytes / (ms * 1e-3) / 1e9
    del sets, calls, x0
    torch.cuda.empty_cache()
    return {"workload": w.description, "us": round(ms * 1e3, 3), "gbps": round(gbps, 1),
            "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4), "bytes": nbytes,
            "buffers": "3 rotating sets (906 MB)",
            "traffic": traffic_record("int8_quant_per_token", w.name)}


if __name__ == "__main__":
    sys.exit(main())
