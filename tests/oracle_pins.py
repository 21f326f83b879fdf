"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin takes an ``oracle.Oracle`` and raises ``AssertionError`` when the
oracle disagrees with what the pages or the mathematics fix:

* closed forms built by hand from the rounding rule (ties to even, the
  argmax maps to +-127, the zero-row rule);
* invariants (|x - q*s| <= s/2, odd symmetry, power-of-two scaling,
  idempotence, stacking of fused QKV blocks);
* brute force with Python integers and exact rationals on tiny inputs;
* library routines on special cases (NumPy int64/float64 matmul, NumPy
  float32 division, torch's bf16 cast, NumPy's half-precision conversions);
* the statistics the pages print (0.17 % rel-L2 at three shapes; the
  missing-act_scale signature: 97 % error and norm ratio E[act_scale]).

``tests/test_oracle_pins.py`` runs every pin on the real oracle;
``tests/test_oracle_mutants.py`` plants plausible mistakes in copies of
``oracle.c`` and checks that some pin fails for each.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bits(vals) -> np.ndarray:
    """Exact bf16 bit patterns of bf16-representable values."""
    f = np.asarray(vals, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value is not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def _f32(bits: np.ndarray) -> np.ndarray:
    return wl.bf16_bits_to_f32(bits)


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return _f32(bits).astype(np.float64)


def _rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


# ---------------------------------------------------------------------------
# Quantization: closed forms
# ---------------------------------------------------------------------------
# (row, expected codes, expected scale). Built by hand from the rule
# q = rint_even(x * fl32(127/absmax)), s = fl32(absmax/127).
TIE_CASES = [
    # absmax 127 -> inv = 1, s = 1; halves round to even, not away from zero
    ([127.0, 62.5, -62.5, 0.5, 1.5, 2.5], [127, 62, -62, 0, 2, 2], 1.0),
    # absmax 254 -> inv = 0.5, s = 2
    ([254.0, 5.0, -3.0, 1.0], [127, 2, -2, 0], 2.0),
    # absmax 2 -> inv = 63.5 exactly; 1*63.5 = 63.5 ties to 64
    ([1.0, -2.0, 0.5], [64, -127, 32], float(np.float32(2.0) / np.float32(127.0))),
    # odd/even neighbours of ties
    ([127.0, 3.5, -3.5, 4.5, -4.5, 5.5], [127, 4, -4, 4, -4, 6], 1.0),
    # negative absmax element maps to -127
    ([-127.0, 10.0, 0.25], [-127, 10, 0], 1.0),
]


def pin_quant_ties(o):
    for row, q_exp, s_exp in TIE_CASES:
        x = _bits(row)[None, :]
        q, s = o.quant_per_token(x)
        assert q[0].tolist() == q_exp, (row, q[0].tolist(), q_exp)
        assert s[0] == np.float32(s_exp), (row, s[0], s_exp)
        qw, sw = o.quant_per_channel(np.asarray([row], np.float32))
        assert qw[0].tolist() == q_exp and sw[0] == np.float32(s_exp)


def pin_quant_zero_rows(o):
    # all-zero row, and rows whose absmax is below / at the 2^-100 threshold
    rows = np.zeros((4, 8), np.float32)
    rows[1, 3] = 2.0 ** -101
    rows[2, 5] = -(2.0 ** -100)      # at the threshold: quantized normally
    rows[3, :] = 2.0 ** -99
    q, s = o.quant_per_token(_bits(rows))
    assert s[0] == 0 and s[1] == 0 and not q[0].any() and not q[1].any()
    assert s[2] == np.float32(np.float32(2.0 ** -100) / np.float32(127))
    assert q[2].tolist() == [0, 0, 0, 0, 0, -127, 0, 0]
    assert q[3].tolist() == [127] * 8
    qw, sw = o.quant_per_channel(rows)
    assert np.array_equal(qw, q) and np.array_equal(sw, s)


# ---------------------------------------------------------------------------
# Quantization: invariants on the workloads' value distributions
# ---------------------------------------------------------------------------
def _quant_rows_under_test(seed=7):
    rng = np.random.default_rng(seed)
    parts = [
        rng.standard_normal((16, 300)).astype(np.float32),
        (rng.standard_normal((8, 1000)) * 30).astype(np.float32),
        rng.standard_cauchy((8, 257)).astype(np.float32),
        rng.uniform(-1e-3, 1e-3, (8, 64)).astype(np.float32),
    ]
    gelu = wl.random_case(16, 512, 8, seed + 1, x_kind="gelu", outlier_frac=0,
                          row_loguniform=True, bias=False)
    return [_f32(wl.f32_to_bf16_bits(p)) for p in parts] + [_f32(gelu.x_bf16)]


def pin_quant_invariants(o):
    for x in _quant_rows_under_test():
        bits = wl.f32_to_bf16_bits(x)
        q, s = o.quant_per_token(bits)
        x64 = x.astype(np.float64)
        s64 = s.astype(np.float64)[:, None]
        a = np.abs(x).max(axis=1)
        # scale is the correctly rounded fp32 quotient absmax / 127
        assert np.array_equal(s, (a / np.float32(127)).astype(np.float32))
        # every element lies within half a step of its code (plus fp32 slack)
        err = np.abs(x64 - q.astype(np.float64) * s64)
        assert np.all(err <= s64 * (0.5 + 2.0 ** -14)), float((err / s64).max())
        # codes are the nearest integers to x * fl32(127/absmax) (NumPy rint)
        inv = (np.float32(127) / a).astype(np.float32)[:, None]
        assert np.array_equal(q, np.clip(np.rint(x * inv), -127, 127).astype(np.int8))
        # the absmax element maps to +-127 with its sign
        idx = np.abs(x).argmax(axis=1)
        top = q[np.arange(len(q)), idx].astype(int)
        assert np.all(np.abs(top) == 127)
        assert np.all(np.sign(top) == np.sign(x[np.arange(len(x)), idx]))
        assert q.min() >= -127
        # odd symmetry
        qn, sn = o.quant_per_token(bits ^ np.uint16(0x8000))
        assert np.array_equal(qn, -q) and np.array_equal(sn, s)
        # power-of-two scaling leaves codes unchanged and scales s exactly
        for j in (-3, 5):
            qj, sj = o.quant_per_token(wl.f32_to_bf16_bits(x * np.float32(2.0 ** j)))
            assert np.array_equal(qj, q)
            assert np.array_equal(sj, (s * np.float32(2.0 ** j)).astype(np.float32))
        # idempotence: re-quantizing the dequantized row returns the codes
        deq = (q.astype(np.float32) * s[:, None]).astype(np.float32)
        q2, _ = o.quant_per_channel(deq)
        assert np.array_equal(q2, q)
        # the bf16 entry point equals the fp32 entry point on widened values
        qf, sf = o.quant_per_channel(x)
        assert np.array_equal(qf, q) and np.array_equal(sf, s)


# ---------------------------------------------------------------------------
# int32 accumulators
# ---------------------------------------------------------------------------
def pin_gemm_bruteforce(o):
    rng = np.random.default_rng(11)
    for (M, N, K) in [(1, 1, 1), (3, 5, 7), (8, 6, 96), (5, 9, 130)]:
        a = rng.integers(-128, 128, (M, K), dtype=np.int8)
        b = rng.integers(-128, 128, (N, K), dtype=np.int8)
        acc = o.gemm_i32(a, b)
        al, bl = a.tolist(), b.tolist()
        for m in range(M):
            for n in range(N):
                assert acc[m, n] == sum(x * y for x, y in zip(al[m], bl[n])), (M, N, K, m, n)


def pin_gemm_numpy(o):
    rng = np.random.default_rng(12)
    M, N, K = 130, 70, 777
    a = rng.integers(-127, 128, (M, K), dtype=np.int8)
    b = rng.integers(-127, 128, (N, K), dtype=np.int8)
    ref = a.astype(np.int64) @ b.astype(np.int64).T
    acc = o.gemm_i32(a, b)
    assert np.array_equal(acc.astype(np.int64), ref)
    rows = np.array([129, 0, 64, 64, 3])
    assert np.array_equal(o.gemm_i32(a, b, rows).astype(np.int64), ref[rows])
    # the largest sums that fit, and one that does not
    K = 133144
    ones = np.full((1, K), 127, np.int8)
    assert int(o.gemm_i32(ones, ones)[0, 0]) == 127 * 127 * K
    ones = np.full((1, K + 1), 127, np.int8)
    try:
        o.gemm_i32(ones, ones)
    except OverflowError:
        pass
    else:
        raise AssertionError("int32 overflow not reported")


# ---------------------------------------------------------------------------
# Epilogue and bf16 rounding
# ---------------------------------------------------------------------------
def _exact_bf16(v: Fraction) -> int:
    """bf16 bits of the exact rational v, rounded to nearest-even (normal range)."""
    if v == 0:
        return 0
    neg = v < 0
    v = -v if neg else v
    e = v.numerator.bit_length() - v.denominator.bit_length()
    if Fraction(2) ** e > v:
        e -= 1
    # v in [2^e, 2^(e+1)); bf16 keeps 8 significant bits
    ulp = Fraction(2) ** (e - 7)
    t = v / ulp
    r = int(t)
    frac = t - r
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and r % 2 == 1):
        r += 1
    f = np.float32(float(r * ulp))
    assert Fraction(float(f)) == r * ulp
    bits = int(np.asarray(f).view(np.uint32)) >> 16
    return bits | (0x8000 if neg else 0)


def pin_bf16_rounding(o):
    import torch
    rng = np.random.default_rng(13)
    f = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * np.float32(1e3),
        # exact ties: low 16 bits 0x8000, both parities of bit 16
        (rng.integers(0x3000, 0x4F00, 500).astype(np.uint32) << 16 | 0x8000).view(np.float32),
        # values that carry into the next binade
        np.array([0x3F7FFFFF, 0x3F7F8000, 0x477F8000, 0xBF7FFFFF], np.uint32).view(np.float32),
    ])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([o.float_to_bf16(float(v)) for v in f], np.uint16)
    assert np.array_equal(got, ref)
    # double -> bf16 rounds once: exact rational check on random doubles
    d = rng.standard_normal(2000) * 10.0 ** rng.uniform(-6, 6, 2000)
    # doubles a hair above / below a bf16 tie: rounding through float first
    # would land exactly on the tie and round to even instead
    base = 1.0 + 2.0 ** -8
    near = [base + 2.0 ** -30, base - 2.0 ** -30, -(base + 2.0 ** -31),
            3.0 * (1.0 + 3 * 2.0 ** -8) - 2.0 ** -28]
    assert o.double_to_bf16(base + 2.0 ** -30) == 0x3F81
    assert o.double_to_bf16(base - 2.0 ** -30) == 0x3F80
    for v in list(d) + near:
        assert o.double_to_bf16(float(v)) == _exact_bf16(Fraction(float(v))), v


def pin_epilogue_exact(o):
    rng = np.random.default_rng(14)
    M, N = 6, 7
    acc = rng.integers(-2 ** 24, 2 ** 24, (M, N)).astype(np.int32)
    acc[0, 0] = 2 ** 31 - 1
    acc[1, 1] = -2 ** 31
    xs = (rng.uniform(0.01, 1, M)).astype(np.float32)
    ws = (rng.uniform(1e-4, 1e-2, N)).astype(np.float32)
    bias = wl.f32_to_bf16_bits(rng.standard_normal(N).astype(np.float32) * np.float32(0.01))
    for b in (None, bias):
        got = o.epilogue_f64(acc, xs, ws, b)
        for m in range(M):
            for n in range(N):
                v = Fraction(int(acc[m, n])) * Fraction(float(xs[m])) * Fraction(float(ws[n]))
                if b is not None:
                    v += Fraction(float(_f32(b[n:n + 1])[0]))
                assert got[m, n] == _exact_bf16(v), (m, n)
    # the fixed-order fp32 epilogue stays within one bf16 ulp of the exact value
    f32 = o.epilogue_f32(acc, xs, ws, bias).astype(np.int32)
    f64 = o.epilogue_f64(acc, xs, ws, bias).astype(np.int32)
    assert np.all(np.abs(f32 - f64) <= 1)


# ---------------------------------------------------------------------------
# The fp16 twin: conversions, quant on fp16 rows, fp16 epilogue
# ---------------------------------------------------------------------------
def _exact_f16(v: Fraction) -> int:
    """IEEE binary16 bits of the exact rational v, nearest-even, with gradual
    underflow (step 2^-24 below 2^-14) and overflow to infinity."""
    neg = v < 0
    v = -v if neg else v
    sign = 0x8000 if neg else 0
    if v == 0:
        return sign
    e = v.numerator.bit_length() - v.denominator.bit_length()
    if Fraction(2) ** e > v:
        e -= 1
    ulp = Fraction(2) ** (max(e, -14) - 10)        # 11 significant bits, or subnormal step
    t = v / ulp
    r = int(t)
    frac = t - r
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and r % 2 == 1):
        r += 1
    val = r * ulp
    if val > 65504:
        return sign | 0x7C00
    h = np.float16(float(val))
    assert Fraction(float(h)) == val
    return sign | int(np.asarray(h).view(np.uint16))


def pin_f16_conversions(o):
    # every binary16 pattern widens like NumPy's half type
    for h in range(0x10000):
        ref = float(np.array([h], np.uint16).view(np.float16)[0])
        got = o.f16_to_float(h)
        assert got == ref or (np.isnan(got) and np.isnan(ref)), hex(h)
    # hand-built ties and edges
    for d, bits in [(1.0 + 2.0 ** -11, 0x3C00), (1.0 + 3 * 2.0 ** -11, 0x3C02),
                    (1.0 + 2.0 ** -11 + 2.0 ** -40, 0x3C01), (2.0 ** -25, 0x0000),
                    (3 * 2.0 ** -25, 0x0002), (2.0 ** -25 + 2.0 ** -60, 0x0001),
                    (2.0 ** -14 - 2.0 ** -25, 0x0400), (65504.0, 0x7BFF), (65519.99, 0x7BFF),
                    (65520.0, 0x7C00), (-65520.0, 0xFC00), (-0.0, 0x8000), (1e30, 0x7C00)]:
        assert o.double_to_f16(d) == bits, (d, hex(o.double_to_f16(d)))
    # random doubles over the whole range: exact rational rounding and
    # NumPy's own double -> half conversion
    rng = np.random.default_rng(21)
    d = rng.standard_normal(3000) * 10.0 ** rng.uniform(-9, 5.5, 3000)
    ref = d.astype(np.float16).view(np.uint16)
    for v, r in zip(d, ref):
        got = o.double_to_f16(float(v))
        assert got == int(r) == _exact_f16(Fraction(float(v))), v


def pin_quant_f16(o):
    # values exact in both bf16 and fp16 (8 significant bits, fp16's normal
    # range): the fp16 quant must equal the bf16 one, codes and scales
    rng = np.random.default_rng(22)
    v = (rng.integers(-255, 256, (24, 96)) * 2.0 ** rng.integers(-12, 6, (24, 1))).astype(np.float32)
    v[3] = 0.0
    v[5, 7] = -255.0 * 2.0 ** -12                      # argmax negative
    h = v.astype(np.float16).view(np.uint16)
    q16, s16 = o.quant_per_token_f16(h)
    qb, sb = o.quant_per_token(_bits(v))
    assert np.array_equal(q16, qb) and np.array_equal(s16, sb)
    assert s16[3] == 0 and not q16[3].any()
    # random fp16 rows incl. subnormals: |x - q*s| <= s/2 (+fp32 slack), argmax -> +-127
    x = (rng.standard_normal((32, 200)) * 10.0 ** rng.uniform(-6, 4, (32, 1))).astype(np.float16)
    x[0, :] = np.float16(6e-8)                         # subnormal-only row
    q, s = o.quant_per_token_f16(x.view(np.uint16))
    xf = x.astype(np.float64)
    err = np.abs(xf - q.astype(np.float64) * s.astype(np.float64)[:, None])
    assert np.all(err <= s.astype(np.float64)[:, None] * (0.5 + 1e-5))
    am = np.argmax(np.abs(xf), axis=1)
    assert np.all(np.abs(q[np.arange(32), am]) == 127)


def pin_epilogue_f16_exact(o):
    rng = np.random.default_rng(23)
    M, N = 6, 7
    acc = rng.integers(-2 ** 20, 2 ** 20, (M, N)).astype(np.int32)
    acc[0, 0] = 2 ** 31 - 1                            # overflows fp16 -> inf
    acc[1, 1] = -2 ** 31
    acc[2, 2] = 3                                      # lands in the subnormal range
    xs = (rng.uniform(0.01, 1, M)).astype(np.float32)
    ws = (rng.uniform(1e-4, 1e-2, N)).astype(np.float32)
    xs[0] = xs[1] = 1.0
    ws[0] = ws[1] = 1.0
    xs[2], ws[2] = np.float32(2.0 ** -12), np.float32(2.0 ** -12)
    bias = (rng.standard_normal(N) * 0.01).astype(np.float16).view(np.uint16)
    bias[2] = 0
    for b in (None, bias):
        got = o.epilogue_f64_f16(acc, xs, ws, b)
        for m in range(M):
            for n in range(N):
                v = Fraction(int(acc[m, n])) * Fraction(float(xs[m])) * Fraction(float(ws[n]))
                if b is not None:
                    v += Fraction(float(np.array([b[n]], np.uint16).view(np.float16)[0]))
                assert got[m, n] == _exact_f16(v), (m, n)
    assert got[0, 0] == 0x7C00 and got[1, 1] == 0xFC00
    # the fixed-order fp32 epilogue rounds the fp32 value once to fp16: it
    # stays within one fp16 step of the exact value (same sign, so the bit
    # patterns differ by at most one)
    f32 = o.epilogue_f32_f16(acc, xs, ws, bias).astype(np.int32)
    f64 = o.epilogue_f64_f16(acc, xs, ws, bias).astype(np.int32)
    assert np.all(np.abs(f32 - f64) <= 1)


# ---------------------------------------------------------------------------
# The FP8 (e4m3) twin
# ---------------------------------------------------------------------------
def _exact_e4m3(v: Fraction) -> int:
    """OCP e4m3 bits of the exact rational v (|v| <= 448), nearest-even."""
    neg = v < 0
    v = -v if neg else v
    sign = 0x80 if neg else 0
    if v == 0:
        return sign
    e = v.numerator.bit_length() - v.denominator.bit_length()
    if Fraction(2) ** e > v:
        e -= 1
    ulp = Fraction(2) ** (max(e, -6) - 3)          # 4 significant bits, or subnormal step 2^-9
    t = v / ulp
    r = int(t)
    frac = t - r
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and r % 2 == 1):
        r += 1
    val = r * ulp
    assert val <= 448
    if val < Fraction(2) ** -6:
        return sign | int(val / Fraction(2) ** -9)
    E = val.numerator.bit_length() - val.denominator.bit_length()
    if Fraction(2) ** E > val:
        E -= 1
    mant = int(val / Fraction(2) ** E * 8) - 8
    return sign | ((E + 7) << 3) | mant


def pin_e4m3_conversions(o):
    import torch
    for c in range(256):
        ref = torch.tensor([c], dtype=torch.uint8).view(torch.float8_e4m3fn).double().item()
        got = o.e4m3_to_double(c)
        assert got == ref or (np.isnan(got) and np.isnan(ref)), c
    for d, bits in [(448.0, 0x7E), (-448.0, 0xFE), (2.0 ** -9, 0x01), (2.0 ** -10, 0x00),
                    (3 * 2.0 ** -10, 0x02), (1.0 + 2.0 ** -4, 0x38), (1.0 + 3 * 2.0 ** -4, 0x3A),
                    (1.0 + 2.0 ** -4 + 2.0 ** -30, 0x39), (2.0 ** -6 - 2.0 ** -10, 0x08),
                    (-0.0, 0x80), (240.0, 0x77)]:
        assert o.double_to_e4m3(d) == bits, (d, hex(o.double_to_e4m3(d)))
    rng = np.random.default_rng(31)
    v = np.clip(rng.standard_normal(3000) * 10.0 ** rng.uniform(-4, 2.7, 3000), -448, 448)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for x, r in zip(v.astype(np.float32), ref):
        got = o.double_to_e4m3(float(x))
        assert got == int(r) == _exact_e4m3(Fraction(float(x))), x


def pin_fp8_quant(o):
    rng = np.random.default_rng(32)
    x = (rng.standard_normal((24, 300)) * 10.0 ** rng.uniform(-3, 3, (24, 1))).astype(np.float32)
    x[2] = 0.0
    x[4, 9] = -np.abs(x[4]).max() * 2                  # negative argmax
    xb = wl.f32_to_bf16_bits(x)
    q, s = o.fp8_quant_per_token(xb)
    xf = _bf16_to_f64(xb)
    dec = np.vectorize(o.e4m3_to_double)(q)
    assert s[2] == 0 and not q[2].any()
    assert not np.any((q & 0x7F) == 0x7F)               # never NaN
    am = np.argmax(np.abs(xf), axis=1)
    live = s > 0
    assert np.all(np.abs(dec[np.arange(24), am])[live] == 448.0)
    # each code is the nearest e4m3 value of x / s: within half a step
    # (relative 2^-4, absolute 2^-10 in the subnormal range), plus fp32 slack
    y = xf / np.where(live, s, 1).astype(np.float64)[:, None]
    err = np.abs(dec - y)
    assert np.all(err[live] <= (np.abs(y) * 2.0 ** -4 + 2.0 ** -10 + np.abs(y) * 2.0 ** -20)[live])
    # odd symmetry (signed zeros included: negating x flips every code's
    # sign bit) and the weight path on the same rows
    qn, sn = o.fp8_quant_per_token(wl.f32_to_bf16_bits(-x))
    assert np.array_equal(sn, s) and np.array_equal(qn[live], q[live] ^ 0x80)
    qw, sw = o.fp8_quant_per_channel(_f32(xb))
    assert np.array_equal(qw, q) and np.array_equal(sw, s)


def _torch_e4m3(v32: np.ndarray) -> np.ndarray:
    """torch's float8_e4m3fn cast of fp32 values (round to nearest even), as codes."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(v32, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def _fp8_rule(x32: np.ndarray):
    """The FP8 quant rule written out with NumPy fp32 arithmetic and torch's
    e4m3 cast: s = fl32(a/448), codes = e4m3_rne(clamp(fl32(x * fl32(448/a)), +-448))."""
    a = np.abs(x32).max(axis=1)
    live = a >= np.float32(2.0 ** -100)
    s = np.where(live, a / np.float32(448), np.float32(0)).astype(np.float32)
    inv = np.where(live, np.float32(448) / np.where(live, a, 1), 0).astype(np.float32)
    t = np.clip((x32 * inv[:, None]).astype(np.float32), -448, 448).astype(np.float32)
    q = _torch_e4m3(t)
    q[~live] = 0
    return q, s


def _fp8_tie_rows(seed=35, rows=192):
    """fp32 rows whose products x * fl32(448/a) land exactly on e4m3 rounding
    ties. Element 0 is the absmax a (uniform in [1, 2), sign alternating);
    the rest are the fp32 values nearest T / fl32(448/a), kept where the
    product rounds back to exactly T, for ties T between neighbouring e4m3
    values (normal and subnormal)."""
    rng = np.random.default_rng(seed)
    ties = np.array([1.0625, 1.1875, 0.53125, 3.375, 13.0, 0.02734375, 2.0 ** -10, 3 * 2.0 ** -10,
                     -1.0625, -1.1875, -2.0 ** -10], np.float32)
    out = []
    while len(out) < rows:
        a = np.float32(rng.uniform(1, 2))
        inv = np.float32(448) / a
        row = [a if len(out) % 2 == 0 else -a]
        for T in ties:
            x = np.float32(T / inv)
            for cand in (x, np.nextafter(x, np.float32(np.inf)), np.nextafter(x, np.float32(-np.inf))):
                if np.float32(cand * inv) == T and abs(cand) < a:
                    row.append(cand)
                    break
        if len(row) > 6:
            out.append(np.array(row + [np.float32(0)] * (len(ties) + 1 - len(row)), np.float32))
    return np.stack(out)


def pin_fp8_quant_exact(o):
    """The FP8 quant rule exactly (page "Online Quantization", Parameters: FP8
    with the dynamic activation scheme, read like the int8 rule with 448 in
    place of 127): the scale is the correctly rounded fp32 quotient a/448 and
    each code is torch's e4m3 (nearest-even) cast of fl32(x * fl32(448/a))
    clamped to +-448; on hand-built rows whose products fall exactly on
    ties, and on hand-checked codes."""
    # hand-checked: a = 448 gives inv = 1 and s = 1, so the codes are the
    # e4m3 roundings of x itself; 1.0625 is the tie between 1 (0x38) and
    # 1.125 (0x39) -> even 0x38; 1.1875 between 1.125 and 1.25 -> 0x3A;
    # 2^-10 between 0 and 2^-9 -> +0; 3*2^-10 between 2^-9 (0x01) and
    # 2^-8 (0x02) -> 0x02; a = 224 gives inv = 2, s = 0.5.
    x = np.array([[448, 1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -10, -2.0 ** -10, 240],
                  [224, 0.53125, 0.59375, -0.53125, 2.0 ** -11, 3 * 2.0 ** -11, 0, -224]], np.float32)
    want = np.array([[0x7E, 0x38, 0x3A, 0xB8, 0x00, 0x02, 0x80, 0x77],
                     [0x7E, 0x38, 0x3A, 0xB8, 0x00, 0x02, 0x00, 0xFE]], np.uint8)
    for q, s in (o.fp8_quant_per_channel(x), o.fp8_quant_per_token(wl.f32_to_bf16_bits(x))):
        assert np.array_equal(s, np.array([1.0, 0.5], np.float32)), s
        assert np.array_equal(q, want), q
    # the rule on random rows (scale quotient, reciprocal product, cast)
    rng = np.random.default_rng(36)
    xr = (rng.standard_normal((64, 333)) * 10.0 ** rng.uniform(-6, 6, (64, 1))).astype(np.float32)
    xr[5] = 0
    xr[6] *= np.float32(2.0 ** -110)
    for src, (q, s) in ((xr, o.fp8_quant_per_channel(xr)),
                        (_f32(wl.f32_to_bf16_bits(xr)), o.fp8_quant_per_token(wl.f32_to_bf16_bits(xr)))):
        qr, sr = _fp8_rule(src)
        assert np.array_equal(s, sr)
        assert np.array_equal(q, qr)
    # products exactly on ties
    xt = _fp8_tie_rows()
    q, s = o.fp8_quant_per_channel(xt)
    qr, sr = _fp8_rule(xt)
    assert np.array_equal(s, sr)
    assert np.array_equal(q, qr)


def pin_fp8_gemm(o):
    rng = np.random.default_rng(33)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    a = rng.choice(codes, (5, 37))
    b = rng.choice(codes, (6, 37))
    acc = o.fp8_gemm(a, b)
    frac = {int(c): Fraction(o.e4m3_to_double(int(c))) for c in codes}
    for i in range(5):
        for n in range(6):
            assert Fraction(acc[i, n]) == sum(frac[int(a[i, k])] * frac[int(b[n, k])] for k in range(37))
    a = rng.choice(codes, (64, 4096))
    b = rng.choice(codes, (48, 4096))
    dec = np.vectorize(o.e4m3_to_double)
    assert np.array_equal(o.fp8_gemm(a, b), dec(a) @ dec(b).T)     # exact sums either way
    rows = np.array([5, 0, 63])
    assert np.array_equal(o.fp8_gemm(a, b, rows), (dec(a) @ dec(b).T)[rows])


def pin_fp8_epilogue(o):
    rng = np.random.default_rng(34)
    M, N = 5, 6
    acc = (rng.standard_normal((M, N)) * 1e4).round(3)
    xs = rng.uniform(0.01, 1, M).astype(np.float32)
    ws = rng.uniform(1e-4, 1e-2, N).astype(np.float32)
    bias = wl.f32_to_bf16_bits(rng.standard_normal(N).astype(np.float32) * np.float32(0.01))
    for b in (None, bias):
        o32, o64 = o.fp8_epilogue(acc, xs, ws, b)
        for m in range(M):
            for n in range(N):
                v = Fraction(float(acc[m, n])) * Fraction(float(xs[m])) * Fraction(float(ws[n]))
                if b is not None:
                    v += Fraction(float(_f32(b[n:n + 1])[0]))
                assert o64[m, n] == _exact_bf16(v), (m, n)
                t = np.float32(acc[m, n]) * xs[m] * ws[n]
                assert abs(int(o32[m, n]) - int(o64[m, n])) <= 1 or np.sign(t) == 0
    # fp16 bias and outputs
    b16 = (rng.standard_normal(N) * 0.01).astype(np.float16).view(np.uint16)
    o32, o64 = o.fp8_epilogue(acc, xs, ws, b16, f16=True)
    for m in range(M):
        for n in range(N):
            v = Fraction(float(acc[m, n])) * Fraction(float(xs[m])) * Fraction(float(ws[n]))
            v += Fraction(float(np.array([b16[n]], np.uint16).view(np.float16)[0]))
            assert o64[m, n] == _exact_f16(v), (m, n)
            assert abs(int(o32[m, n]) - int(o64[m, n])) <= 1


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------
def _dequant_reference(xq, xs, wq, ws, bias=None):
    """fp64 (xq*xs) @ (wq*ws)^T (+bias) with NumPy's matmul."""
    ref = (xq.astype(np.float64) * xs.astype(np.float64)[:, None]) @ \
          (wq.astype(np.float64) * ws.astype(np.float64)[:, None]).T
    if bias is not None:
        ref = ref + _bf16_to_f64(bias)[None, :]
    return ref


def pin_layer_vs_numpy(o):
    for seed, (M, K, N), bias in [(21, (37, 320, 45), True), (22, (64, 256, 128), False)]:
        inp = wl.random_case(M, K, N, seed, bias=bias)
        wq, ws = o.quant_per_channel(inp.w_f32)
        xq, xs, acc, out = o.linear(inp.x_bf16, wq, ws, inp.bias_bf16)
        ref = _dequant_reference(xq, xs, wq, ws, inp.bias_bf16)
        got = _bf16_to_f64(out)
        # one bf16 rounding (2^-9 relative) plus fp32 rounding slack
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30), \
            float(np.abs(got - ref).max())
        # permuting X rows / W rows permutes output rows / columns
        pm, pn = np.random.default_rng(seed).permutation(M), np.random.default_rng(seed + 1).permutation(N)
        b = None if inp.bias_bf16 is None else inp.bias_bf16[pn]
        _, _, _, out_p = o.linear(inp.x_bf16[pm], wq[pn], ws[pn], b)
        assert np.array_equal(out_p, out[pm][:, pn])
    # negating X negates the output exactly when there is no bias
    inp = wl.random_case(16, 192, 24, 23, bias=False)
    wq, ws = o.quant_per_channel(inp.w_f32)
    _, _, _, out = o.linear(inp.x_bf16, wq, ws)
    _, _, _, outn = o.linear(inp.x_bf16 ^ np.uint16(0x8000), wq, ws)
    assert np.array_equal(_f32(outn), -_f32(out))   # values: +0 stays +0
    # an all-zero token row yields exactly the bias (or +0 without bias)
    inp = wl.random_case(8, 128, 16, 24, bias=True)
    x = inp.x_bf16.copy()
    x[3] = 0
    wq, ws = o.quant_per_channel(inp.w_f32)
    _, xs, _, out = o.linear(x, wq, ws, inp.bias_bf16)
    assert xs[3] == 0 and np.array_equal(out[3], inp.bias_bf16)
    _, _, _, out = o.linear(x, wq, ws)
    assert not out[3].any()


def pin_fused_qkv_stack(o):
    rng = np.random.default_rng(25)
    blocks = [rng.standard_normal((40, 192)).astype(np.float32) * np.float32(0.02)
              for _ in range(3)]
    wq, ws = o.quant_per_channel(np.concatenate(blocks))
    parts = [o.quant_per_channel(b) for b in blocks]
    assert np.array_equal(wq, np.concatenate([p[0] for p in parts]))
    assert np.array_equal(ws, np.concatenate([p[1] for p in parts]))
    x = wl.random_case(24, 192, 8, 26).x_bf16
    xq, xs = o.quant_per_token(x)
    acc = o.gemm_i32(xq, wq)
    assert np.array_equal(acc, np.concatenate([o.gemm_i32(xq, p[0]) for p in parts], axis=1))


# ---------------------------------------------------------------------------
# The pages' printed statistics
# ---------------------------------------------------------------------------
def _golden():
    with open(os.path.join(GOLDEN, "pages_statistics.json")) as f:
        return json.load(f)


def pin_pages_rel_l2(o, rows: int = 96):
    """0.17 % rel-L2 against a float32 reference at the three printed shapes.

    Reading: the float32 reference is evaluated on the dequantized operands
    (xq*xs)(wq*ws)^T, so what remains is the bf16 rounding of the output.
    Inputs: the tiny, attention out-projection and fused-QKV workloads;
    the two large shapes are checked on a sample of token rows.
    """
    g = _golden()["raw_op_rel_l2"]
    shapes = [tuple(s) for s in g["shapes_MKN"]]
    for w in (wl.by_name("tiny"), wl.by_name("attn_out"), wl.by_name("fused_qkv")):
        assert (w.M, w.K, w.N) in shapes
        inp = wl.generate(w)
        wq, ws = o.quant_per_channel(inp.w_f32)
        sel = None if w.M <= rows else np.random.default_rng(w.seed).choice(w.M, rows, replace=False)
        xq, xs, acc, out = o.linear(inp.x_bf16, wq, ws, inp.bias_bf16, rows=sel)
        if sel is not None:
            xq, xs = xq[sel], xs[sel]
        ref = _dequant_reference(xq, xs, wq, ws, inp.bias_bf16)
        r = _rel_l2(_bf16_to_f64(out), ref)
        assert round(r * 100, 2) == round(g["value"] * 100, 2), (w.name, r)


def pin_pages_missing_act_scale(o, rows: int = 64):
    """The missing-act_scale signature: 97 % error; norm ratio = E[act_scale].

    Reading: the probe's rows were plain N(0,1) tokens at the (512,4096,4096)
    shape (no outlier columns), giving act_scale near 0.03.
    """
    g = _golden()["missing_act_scale"]
    inp = wl.random_case(rows, 4096, 4096, 27, outlier_frac=0, bias=False)
    wq, ws = o.quant_per_channel(inp.w_f32)
    xq, xs, acc, out = o.linear(inp.x_bf16, wq, ws)
    R = acc.astype(np.float64) * ws.astype(np.float64)[None, :]   # reference without xs
    got = _bf16_to_f64(out)
    assert round(_rel_l2(got, R), 2) == g["error"]
    ratio = np.linalg.norm(got, axis=1) / np.linalg.norm(R, axis=1)
    assert np.all(np.abs(ratio / xs - 1) < 5e-3)
    assert abs(ratio.mean() / xs.mean() - 1) < 1e-3
    # rows sharing one absmax share one act_scale: the Frobenius ratio is it
    x = _f32(inp.x_bf16).copy()
    x[:, 0] = np.float32(4.0)
    xb = wl.f32_to_bf16_bits(np.clip(x, -4.0, 4.0))
    xq, xs, acc, out = o.linear(xb, wq, ws)
    assert np.all(xs == xs[0])
    R = acc.astype(np.float64) * ws.astype(np.float64)[None, :]
    fro = np.linalg.norm(_bf16_to_f64(out)) / np.linalg.norm(R)
    assert abs(fro / float(xs.mean()) - 1) < 1e-3


def _round_binary(v: Fraction, sig: int, emin: int) -> Fraction:
    """v rounded to nearest-even in a binary format with `sig` significant
    bits and gradual underflow below 2^emin (the IEEE rule, on exact
    rationals; no overflow handling: the callers stay in range)."""
    if v == 0:
        return v
    neg = v < 0
    a = -v if neg else v
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp = Fraction(2) ** (max(e, emin) - (sig - 1))
    t = a / ulp
    r = int(t)
    frac = t - r
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and r % 2 == 1):
        r += 1
    return -(r * ulp) if neg else r * ulp


def _fl32(v: Fraction) -> Fraction:
    return _round_binary(v, 24, -126)


def _order_sensitive_inputs(n: int, seed: int, out_bits: int, limit: float):
    """Seeded (acc, xs, ws) triples whose result, rounded to `out_bits`
    significant bits, depends on the order of the two scale products:
    (acc*xs)*ws, (acc*ws)*xs and acc*(xs*ws) in fp32 do not all round to the
    same output. NumPy's float32 arithmetic (IEEE, round to nearest) finds
    them; the pin then checks the oracle against the exact model. Results of
    magnitude `limit` or more are left out (fp16 overflows at 65520)."""
    rng = np.random.default_rng(seed)
    acc = rng.integers(-2 ** 26, 2 ** 26, n).astype(np.int64)
    xs = rng.uniform(1e-3, 1.0, n).astype(np.float32)
    ws = rng.uniform(1e-5, 1e-2, n).astype(np.float32)
    a = acc.astype(np.float32)
    r1 = (a * xs) * ws
    r2 = (a * ws) * xs
    r3 = a * (xs * ws)

    def out(r):   # round the fp32 values to out_bits significant bits, nearest-even
        m, e = np.frexp(r.astype(np.float64))
        return np.ldexp(np.round(np.ldexp(m, out_bits)), e - out_bits)
    o1 = out(r1)
    pick = np.nonzero(((o1 != out(r2)) | (o1 != out(r3))) & (np.abs(r1) < limit))[0]
    return acc[pick], xs[pick], ws[pick]


def pin_epilogue_order(o):
    """The fp32 epilogue takes its steps in the stated order, each rounded
    once to fp32: fl(fl(fl(acc)*xs)*ws) (+bias), then one rounding to bf16 or
    fp16. Checked on inputs where another order gives another output, against
    an exact rational model of IEEE fp32 rounding; the fp8 epilogue (the same
    steps on fl32 of its exact sums) too."""
    for out_bits, fn, exact, limit in ((8, "epilogue_f32", _exact_bf16, np.inf),
                                       (11, "epilogue_f32_f16", _exact_f16, 6.0e4)):
        acc, xs, ws = _order_sensitive_inputs(1 << 22, 1500 + out_bits, out_bits, limit)
        assert len(acc) >= 8, len(acc)          # the inputs do tell the orders apart
        acc, xs, ws = acc[:64], xs[:64], ws[:64]
        k = len(acc)
        # a k x k accumulator matrix whose diagonal holds the cases: output
        # (i, i) takes acc[i], xs[i] and ws[i]
        got = getattr(o, fn)(np.diag(acc).astype(np.int32), xs, ws)
        for i in range(k):
            t = _fl32(Fraction(int(acc[i])))
            t = _fl32(t * Fraction(float(xs[i])))
            t = _fl32(t * Fraction(float(ws[i])))
            assert got[i, i] == exact(t), (fn, i)
        if out_bits == 8:
            own, _ = o.fp8_epilogue(np.diag(acc).astype(np.float64), xs, ws)
            assert np.array_equal(np.diag(own), np.diag(got)), "fp8 epilogue order"


FAST_PINS = [pin_quant_ties, pin_quant_zero_rows, pin_quant_invariants, pin_gemm_bruteforce,
             pin_gemm_numpy, pin_bf16_rounding, pin_epilogue_exact, pin_epilogue_order,
             pin_f16_conversions,
             pin_quant_f16, pin_epilogue_f16_exact, pin_e4m3_conversions, pin_fp8_quant,
             pin_fp8_quant_exact, pin_fp8_gemm, pin_fp8_epilogue, pin_layer_vs_numpy, pin_fused_qkv_stack]
PAGE_PINS = [pin_pages_rel_l2, pin_pages_missing_act_scale]
ALL_PINS = FAST_PINS + PAGE_PINS
