"""libw8a8 C ABI on the CPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call.

No call here launches a kernel: argument errors return before the device is
touched, and on a machine without a GPU a well-formed call must fail with
W8A8_ERR_DEVICE (never a silent fallback).
"""
import ast
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w8a8.h")
PKG = os.path.join(ROOT, "w8a8_int8_dynamic_amd")

from w8a8_int8_dynamic_amd import _lib  # noqa: E402

L = _lib.lib()
OK, NULL, SHAPE, ALIGN, DEVICE, MODE = 0, 1, 2, 3, 4, 5
A = 0x10000          # a 16-byte-aligned fake device address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(\w+)\s*\(", text, flags=re.M)) -
                  {"defined"})


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ("int8_prepack_weight", "int8_quant_per_token", "int8_scaled_mm",
                 "int8_quant_per_channel", "int8_unpack_weight", "int8_prepack_weight_bytes",
                 "int8_quant_prepack_weight"):
        assert must in names


def test_library_exports_every_declared_symbol():
    exported = subprocess.run(["nm", "-D", "--defined-only", _lib.LIBRARY], capture_output=True,
                              text=True, check=True).stdout
    syms = {line.split()[-1] for line in exported.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in syms, f"{name} declared in w8a8.h but not exported"
        assert hasattr(L, name)
    # the binding's signature table covers exactly the header
    assert sorted(_lib.SIGNATURES) == declared_functions()


def test_only_the_abi_is_exported():
    exported = subprocess.run(["nm", "-D", "--defined-only", _lib.LIBRARY], capture_output=True,
                              text=True, check=True).stdout
    text_syms = {line.split()[-1] for line in exported.splitlines()
                 if len(line.split()) == 3 and line.split()[1] == "T"}
    assert text_syms <= set(declared_functions()), text_syms - set(declared_functions())


def test_timeline_twin_exports_the_abi_and_its_reader():
    """The measurement twin (libw8a8_timeline.so, built beside the library)
    exports the same entry points plus w8a8_timeline_read; the library proper
    has no trace of the timeline."""
    twin = os.path.join(os.path.dirname(_lib.LIBRARY), "libw8a8_timeline.so")
    if not os.path.exists(twin):
        pytest.skip("libw8a8_timeline.so not built")

    def text_syms(path):
        out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                             check=True).stdout
        return {line.split()[-1] for line in out.splitlines()
                if len(line.split()) == 3 and line.split()[1] == "T"}

    lib, tw = text_syms(_lib.LIBRARY), text_syms(twin)
    assert tw == lib | {"w8a8_timeline_read"}
    assert "w8a8_timeline_read" not in lib


def test_constants_match_header():
    text = open(HEADER).read()
    assert f"#define W8A8_MAX_K {_lib.W8A8_MAX_K}" in text
    assert 128 * 128 * _lib.W8A8_MAX_K < 2 ** 31 and _lib.W8A8_MAX_K % 16 == 0
    assert 128 * 128 * (_lib.W8A8_MAX_K + 16) >= 2 ** 31
    # the main kernel's 32-bit offsets: 256 token rows of pitch ldq from a
    # tile's first row
    assert f"#define W8A8_MAX_LDQ {_lib.W8A8_MAX_LDQ}" in text
    assert 256 * _lib.W8A8_MAX_LDQ + _lib.W8A8_MAX_K < 2 ** 31


def test_status_strings():
    for s in range(7):
        assert _lib.status_string(s) and _lib.status_string(s) != "unknown status"
    assert _lib.status_string(99) == "unknown status"


def test_prepack_bytes():
    f = L.int8_prepack_weight_bytes
    assert f(1, 1) == 16 * 64
    assert f(16, 64) == 1024
    assert f(17, 65) == 32 * 128
    assert f(12288, 4096) == 12288 * 4096
    assert f(0, 64) == 0 and f(16, 0) == 0 and f(-1, 64) == 0
    assert f(2 ** 31, 64) == 0


def quant(x=A, M=4, K=64, ldx=64, q=A, ldq=64, s=A):
    return L.int8_quant_per_token(x, M, K, ldx, q, ldq, s, None)


def qchan(w=A, N=4, K=64, ldw=64, q=A, ldq=64, s=A):
    return L.int8_quant_per_channel(w, N, K, ldw, q, ldq, s, None)


def test_quant_validation():
    assert quant(M=-1) == SHAPE
    assert quant(K=0) == SHAPE
    assert quant(ldx=63) == SHAPE
    assert quant(ldq=63) == SHAPE
    assert quant(M=0, x=None, q=None, s=None) == OK          # empty is a no-op
    assert quant(x=None) == NULL and quant(q=None) == NULL and quant(s=None) == NULL
    assert quant(x=A + 8) == ALIGN                           # bf16 rows need 16 bytes
    assert quant(ldx=68, K=64) == ALIGN                      # ldx % 8
    assert quant(q=A + 4) == ALIGN and quant(ldq=68) == ALIGN
    assert quant(s=A + 2) == ALIGN
    assert qchan(ldw=66) == ALIGN                            # fp32 rows: ldw % 4
    assert qchan(ldw=68) in (OK, DEVICE)
    assert "int8_quant_per_token" in (quant(x=None) and _lib.last_error())


def test_prepack_validation():
    p = L.int8_prepack_weight
    assert p(A, 0, 64, 64, A, None) == SHAPE
    assert p(A, 16, 0, 64, A, None) == SHAPE
    assert p(A, 16, 64, 63, A, None) == SHAPE
    assert p(None, 16, 64, 64, A, None) == NULL
    assert p(A, 16, 64, 64, None, None) == NULL
    assert p(A, 16, 64, 64, A + 8, None) == ALIGN
    u = L.int8_unpack_weight
    assert u(A + 8, 16, 64, A, 64, None) == ALIGN
    assert u(A, 16, 64, None, 64, None) == NULL


def test_f16_entry_points_validation():
    def q16(x=A, M=4, K=64, ldx=64, q=A, ldq=64, s=A):
        return L.int8_quant_per_token_f16(x, M, K, ldx, q, ldq, s, None)
    assert q16(M=-1) == SHAPE and q16(K=0) == SHAPE and q16(ldx=63) == SHAPE
    assert q16(M=0, x=None, q=None, s=None) == OK
    assert q16(x=None) == NULL and q16(x=A + 8) == ALIGN and q16(ldx=68) == ALIGN
    assert q16() == DEVICE

    def qm16(x=A, ldx=64, mode=2, tile=-1, **kw):
        a = dict(xq=A, ldq=64, xs=A, wp=A, ws=A, bias=None, M=4, N=16, K=64, out=A, ldo=16)
        a.update(kw)
        return L.int8_quant_scaled_mm_f16_tile(x, ldx, a["xq"], a["ldq"], a["xs"], a["wp"],
                                               a["ws"], a["bias"], a["M"], a["N"], a["K"], mode,
                                               a["out"], a["ldo"], None, tile)
    assert qm16(mode=3) == MODE and qm16(tile=-2) == MODE
    assert qm16(ldx=48) == SHAPE and qm16(x=None) == NULL and qm16(x=A + 8) == ALIGN
    assert qm16() == DEVICE and qm16(mode=0) == DEVICE and qm16(mode=1) == DEVICE
    assert L.int8_quant_scaled_mm_f16(A, 64, A, 64, A, A, A, None, 4, 16, 64, 2, A, 16,
                                      None) == DEVICE


def test_quant_prepack_validation():
    def qp(w=A, dt=0, N=16, K=64, ldw=64, wp=A, ws=A):
        return L.int8_quant_prepack_weight(w, dt, N, K, ldw, wp, ws, None)
    assert qp(dt=2) == MODE and qp(dt=-1) == MODE
    assert qp(N=0) == SHAPE and qp(K=0) == SHAPE and qp(ldw=63) == SHAPE
    assert qp(w=None) == NULL and qp(wp=None) == NULL and qp(ws=None) == NULL
    assert qp(w=A + 8) == ALIGN and qp(wp=A + 8) == ALIGN and qp(ws=A + 2) == ALIGN
    assert qp(ldw=66) == ALIGN                              # fp32 rows: ldw % 4
    assert qp(dt=1, ldw=68) == ALIGN                        # bf16 rows: ldw % 8
    assert qp() == DEVICE and qp(dt=1, ldw=72) == DEVICE    # valid; no GPU here


def mm(xq=A, ldq=64, xs=A, wp=A, ws=A, bias=None, M=4, N=16, K=64, mode=0, out=A, ldo=16, tile=-1):
    return L.int8_scaled_mm_tile(xq, ldq, xs, wp, ws, bias, M, N, K, mode, out, ldo, None, tile)


def test_scaled_mm_validation():
    assert mm(mode=3) == MODE and mm(mode=-1) == MODE
    assert mm(mode=2) == DEVICE and mm(mode=2, out=A + 1) == ALIGN     # fp16 out is valid
    assert mm(tile=L.w8a8_mm_tile_count()) == MODE and mm(tile=-2) == MODE
    assert mm(M=-1) == SHAPE and mm(N=0) == SHAPE
    assert mm(K=0) == SHAPE and mm(K=8) == SHAPE and mm(K=72) == SHAPE
    assert mm(K=_lib.W8A8_MAX_K + 16, ldq=_lib.W8A8_MAX_K + 16) == SHAPE
    assert mm(ldq=48) == SHAPE and mm(ldo=15) == SHAPE
    assert mm(ldq=_lib.W8A8_MAX_LDQ + 16) == SHAPE and mm(ldq=_lib.W8A8_MAX_LDQ) == DEVICE
    assert mm(M=0, xq=None, xs=None, wp=None, ws=None, out=None) == OK
    assert mm(xq=None) == NULL and mm(wp=None) == NULL and mm(out=None) == NULL
    assert mm(xs=None) == NULL and mm(ws=None) == NULL
    assert mm(xq=A + 8) == ALIGN and mm(ldq=72, K=64) == ALIGN and mm(wp=A + 4) == ALIGN
    assert mm(out=A + 1) == ALIGN and mm(out=A + 2, mode=1) == ALIGN
    assert mm(xs=A + 2) == ALIGN and mm(bias=A + 1) == ALIGN
    # int32 debug mode ignores scales and bias
    assert mm(mode=1, xs=None, ws=None, bias=A + 1) in (OK, DEVICE)
    # a grid whose workgroups times threads cannot fit one launch is refused
    # on the host, for the forced smallest tile and for the automatic one
    big = 2 ** 31 - 1
    assert mm(M=big, N=big, ldo=big, tile=0) == SHAPE
    assert mm(M=big, N=big, ldo=big) == SHAPE
    assert mm(M=2 ** 24, N=16, tile=0) in (OK, DEVICE)     # 2^18 workgroups fit


def qmm(x=A, ldx=64, xq=A, ldq=64, xs=A, wp=A, ws=A, bias=None, M=4, N=16, K=64, mode=0, out=A,
        ldo=16, tile=-1):
    return L.int8_quant_scaled_mm_tile(x, ldx, xq, ldq, xs, wp, ws, bias, M, N, K, mode, out, ldo,
                                       None, tile)


def test_quant_scaled_mm_validation():
    # the matmul's own rules
    assert qmm(mode=3) == MODE and qmm(tile=-2) == MODE
    assert qmm(K=72) == SHAPE and qmm(ldq=48) == SHAPE and qmm(ldo=15) == SHAPE
    assert qmm(ldq=_lib.W8A8_MAX_LDQ + 16) == SHAPE
    assert qmm(xq=None) == NULL and qmm(wp=None) == NULL and qmm(out=None) == NULL
    assert qmm(xq=A + 8) == ALIGN
    # the input rows
    assert qmm(ldx=48) == SHAPE
    assert qmm(x=None) == NULL
    assert qmm(x=A + 8) == ALIGN and qmm(ldx=68) == ALIGN
    # the token scales are written, so they are needed in the int32 mode too
    assert qmm(mode=1, xs=None, ws=None) == NULL
    assert qmm(M=0, x=None, xq=None, xs=None, wp=None, ws=None, out=None) == OK


def fp8_mm(xq=A, ldq=64, xs=A, wp=A, ws=A, bias=None, M=4, N=16, K=64, mode=0, out=A, ldo=16,
           tile=-1):
    return L.fp8_scaled_mm_tile(xq, ldq, xs, wp, ws, bias, M, N, K, mode, out, ldo, None, tile)


def fp8_qmm(x=A, ldx=64, xq=A, ldq=64, xs=A, wp=A, ws=A, bias=None, M=4, N=16, K=64, mode=0,
            out=A, ldo=16, tile=-1):
    return L.fp8_quant_scaled_mm_tile(x, ldx, xq, ldq, xs, wp, ws, bias, M, N, K, mode, out, ldo,
                                      None, tile)


def test_fp8_entry_points_validation():
    """The e4m3 twin's entry points apply the int8 rules on the host."""
    assert L.w8a8_fp8_tile_count() == L.w8a8_mm_tile_count()
    for shape in [(512, 12288, 4096), (1, 12288, 4096), (8, 3072, 12288)]:
        assert L.w8a8_fp8_tile_auto(*shape) == L.w8a8_mm_tile_auto(*shape)
    # quant
    fq = lambda **k: L.fp8_quant_per_token(k.get("x", A), k.get("M", 4), k.get("K", 64),
                                           k.get("ldx", 64), k.get("q", A), k.get("ldq", 64),
                                           k.get("s", A), None)
    assert fq(M=-1) == SHAPE and fq(K=0) == SHAPE and fq(ldx=32) == SHAPE and fq(ldq=32) == SHAPE
    assert fq(x=None) == NULL and fq(q=None) == NULL and fq(s=None) == NULL
    assert fq(x=A + 8) == ALIGN and fq(ldx=68) == ALIGN and fq(q=A + 4) == ALIGN
    assert fq(M=0, x=None, q=None, s=None) == OK
    fc = lambda **k: L.fp8_quant_per_channel(k.get("w", A), k.get("N", 4), k.get("K", 64),
                                             k.get("ldw", 64), k.get("q", A), k.get("ldq", 64),
                                             k.get("s", A), None)
    assert fc(ldw=32) == SHAPE and fc(w=None) == NULL and fc(w=A + 8) == ALIGN and fc(ldw=66) == ALIGN
    # online weight quant
    fp = lambda **k: L.fp8_quant_prepack_weight(k.get("w", A), k.get("dt", 1), k.get("N", 16),
                                                k.get("K", 64), k.get("ldw", 64), k.get("p", A),
                                                k.get("s", A), None)
    assert fp(dt=7) == MODE and fp(N=0) == SHAPE and fp(ldw=32) == SHAPE
    assert fp(w=None) == NULL and fp(s=None) == NULL and fp(p=A + 8) == ALIGN
    # matmul
    assert fp8_mm(mode=3) == MODE and fp8_mm(tile=L.w8a8_fp8_tile_count()) == MODE
    assert fp8_mm(K=72) == SHAPE and fp8_mm(ldq=48) == SHAPE and fp8_mm(ldo=15) == SHAPE
    assert fp8_mm(ldq=_lib.W8A8_MAX_LDQ + 16) == SHAPE and fp8_qmm(ldq=_lib.W8A8_MAX_LDQ + 16) == SHAPE
    assert fp8_mm(xq=None) == NULL and fp8_mm(ws=None) == NULL and fp8_mm(xs=None) == NULL
    assert fp8_mm(xq=A + 8) == ALIGN and fp8_mm(out=A + 1) == ALIGN
    assert fp8_mm(M=0, xq=None, xs=None, wp=None, ws=None, out=None) == OK
    big = 2 ** 31 - 1
    assert fp8_mm(M=big, N=big, ldo=big, tile=0) == SHAPE
    # fused
    assert fp8_qmm(ldx=48) == SHAPE and fp8_qmm(x=None) == NULL and fp8_qmm(x=A + 8) == ALIGN
    assert fp8_qmm(mode=1, xs=None, ws=None) == NULL
    assert fp8_qmm(M=0, x=None, xq=None, xs=None, wp=None, ws=None, out=None) == OK


def test_no_fallback_without_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert quant() == DEVICE
    assert mm() == DEVICE
    assert qmm() == DEVICE
    assert L.int8_prepack_weight(A, 16, 64, 64, A, None) == DEVICE
    assert fp8_mm() == DEVICE and fp8_qmm() == DEVICE
    assert L.fp8_quant_per_token(A, 4, 64, 64, A, 64, A, None) == DEVICE
    assert L.w8a8_device_supported(0) == 0
    assert "device" in _lib.last_error()


def test_fused_wait_limit_setter():
    """The bound on the fused path's polls: query, set, restore (host only)."""
    cur = L.w8a8_fused_wait_limit(-1)
    assert cur == 4096
    try:
        assert L.w8a8_fused_wait_limit(0) == cur
        assert L.w8a8_fused_wait_limit(-1) == 0
        assert L.w8a8_fused_wait_limit(7) == 0
        assert L.w8a8_fused_wait_limit(-5) == 7
    finally:
        L.w8a8_fused_wait_limit(cur)
    assert L.w8a8_fused_wait_limit(-1) == cur


def test_tile_table():
    n = L.w8a8_mm_tile_count()
    assert n >= 4
    names = [L.w8a8_mm_tile_name(i).decode() for i in range(n)]
    assert len(set(names)) == n and all(names)
    assert L.w8a8_mm_tile_name(n) == b""
    for shape in [(512, 12288, 4096), (512, 4096, 4096), (4096, 12288, 3072),
                  (8192, 3072, 12288), (64, 128, 256), (1, 1, 16)]:
        t = L.w8a8_mm_tile_auto(*shape)
        assert 0 <= t < n
        assert t == L.w8a8_mm_tile_auto(*shape)             # deterministic


def test_tile_auto_small_m():
    """Decode-shaped inputs (a few token rows) go to the small-M kernel, whose
    tiles are named s<rows>x<channels>/...; from 33 rows on, and for the five
    workloads, the main kernel's tiles are chosen."""
    name = lambda *s: L.w8a8_mm_tile_name(L.w8a8_mm_tile_auto(*s)).decode()
    for shape in [(1, 4096, 4096), (1, 12288, 4096), (4, 4096, 4096), (8, 3072, 12288),
                  (32, 3072, 12288)]:
        assert name(*shape).startswith("s"), (shape, name(*shape))
    for shape in [(33, 3072, 12288), (64, 128, 256), (512, 4096, 4096), (512, 12288, 4096),
                  (4096, 12288, 3072), (8192, 3072, 12288)]:
        assert not name(*shape).startswith("s"), (shape, name(*shape))


def test_binding_rejects_host_tensors():
    import torch
    from w8a8_int8_dynamic_amd import ops
    with pytest.raises(ValueError):
        ops.quant_per_token(torch.zeros(4, 64, dtype=torch.bfloat16))


def test_product_never_touches_the_oracle():
    """No module of the package imports or loads the oracle."""
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            path = os.path.join(dirpath, f)
            if f.endswith(".py"):
                tree = ast.parse(open(path).read())
                for node in ast.walk(tree):
                    if isinstance(node, ast.Import):
                        assert not any(a.name.split(".")[0] == "oracle" for a in node.names), path
                    if isinstance(node, ast.ImportFrom):
                        assert (node.module or "").split(".")[0] != "oracle", path
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                assert "liboracle" not in open(path).read(), path
