"""Planted mistakes in the oracle must fail a pin.

Each mutant is a copy of oracle.c with one plausible error (a dropped term,
a wrong rounding rule, a wrong constant, a wrong index, a flipped sign),
compiled on the CPU into a temporary library. The pins are run against it;
at least one must fail, otherwise the pins would not catch that mistake.
"""
import os

import pytest

import oracle
from tests import oracle_pins as P

MUTANTS = {
    "drop_act_scale": ("t = t * xs[m];", ""),
    "drop_w_scale_f64": ("* (double)ws[n];", ";"),
    "round_half_away": ("t = rintf(t);", "t = roundf(t);"),
    "scale_128": ("float s = a / 127.0f;", "float s = a / 128.0f;"),
    "inv_128": ("float inv = 127.0f / a;", "float inv = 128.0f / a;"),
    "absmax_no_abs": ("float m = fabsf(v[k]);", "float m = v[k];"),
    "truncate_not_round": ("t = rintf(t);", "t = truncf(t);"),
    "no_zero_row_rule": ("if (a < 0x1p-100f) {\n        *scale = 0.0f;",
                         "if (a < 0.0f) {\n        *scale = 0.0f;"),
    "gemm_wrong_b_row": ("const int8_t *br = b + n * ldb;", "const int8_t *br = b + (N - 1 - n) * ldb;"),
    "gemm_short_k": ("for (int64_t k = 0; k < K; ++k)\n                s +=",
                     "for (int64_t k = 0; k + 1 < K; ++k)\n                s +="),
    "gemm_rows_ignored": ("a + (rows ? rows[i] : i) * lda", "a + i * lda"),
    "bias_subtracted": ("t = t + bf16_bits_to_float(bias[n]);", "t = t - bf16_bits_to_float(bias[n]);"),
    "bf16_truncate": ("u += 0x7fffu + lsb;", "u += 0u * lsb;"),
    "bf16_round_half_up": ("u += 0x7fffu + lsb;", "u += 0x8000u + 0u * lsb;"),
    "xs_indexed_by_column": ("t = t * xs[m];", "t = t * xs[n % M];"),
    "f64_double_rounding": ("double r = nearbyint(ldexp(m, 8));", "double r = nearbyint(ldexp((float)m, 8));"),
    "f16_truncate": ("double r = nearbyint(ldexp(a, -q));             /* a / 2^q, ties to even */",
                     "double r = floor(ldexp(a, -q));"),
    "f16_coarse_subnormals": ("q = -24;                                    /* subnormal step 2^-24 */",
                              "q = -23;"),
    "f16_overflow_early": ("if (a >= 65520.0)", "if (a > 65504.0)"),
    "f16_decode_exponent": ("v = ldexpf((float)(m | 0x400), e - 25);", "v = ldexpf((float)(m | 0x400), e - 24);"),
    "f16_bias_dropped": ("t = t + f16_bits_to_float(bias[n]);", "t = t;"),
    "f16_out_through_bf16": ("out[m * ldo + n] = double_to_f16_rne((double)t);",
                             "out[m * ldo + n] = double_to_f16_rne((double)bf16_bits_to_float(float_to_bf16_rne(t)));"),
    "fp8_max_240": ("float s = a / 448.0f;", "float s = a / 240.0f;"),
    "fp8_inv_240": ("float inv = 448.0f / a;", "float inv = 240.0f / a;"),
    "fp8_truncate": ("double r = nearbyint(ldexp(a, -q));             /* ties to even */",
                     "double r = floor(ldexp(a, -q));"),
    "fp8_coarse_subnormals": ("q = -9;                                     /* subnormal step 2^-9 */",
                              "q = -8;"),
    "fp8_decode_exponent": ("v = ldexp((double)(8 + m), e - 10);", "v = ldexp((double)(8 + m), e - 9);"),
    "fp8_gemm_raw_weight": ("s += e4m3_to_double(ar[k]) * e4m3_to_double(br[k]);",
                            "s += e4m3_to_double(ar[k]) * (double)br[k];"),
    "fp8_epilogue_drops_xs": ("double d = acc[m * ldc + n] * (double)xs[m] * (double)ws[n];",
                              "double d = acc[m * ldc + n] * (double)ws[n];"),
    "epilogue_scales_swapped": ("t = t * xs[m];\n            t = t * ws[n];",
                                "t = t * ws[n];\n            t = t * xs[m];"),
    "epilogue_scales_fused": ("t = t * xs[m];\n            t = t * ws[n];",
                              "t = t * (xs[m] * ws[n]);"),
    "fp8_sign_dropped": ("uint8_t sign = signbit(d) ? 0x80u : 0x00u;", "uint8_t sign = 0x00u;"),
    "fp8_zero_loses_sign": ("if (a == 0.0)\n        return sign;", "if (a == 0.0)\n        return 0;"),
    "fp8_underflow_loses_sign": ("if (r == 0.0)\n        return sign;", "if (r == 0.0)\n        return 0;"),
    "fp8_exponent_bias_8": ("((exp_unbiased + 7) << 3)", "((exp_unbiased + 8) << 3)"),
    "fp8_subnormal_boundary": ("if (exp_unbiased < -6)", "if (exp_unbiased < -7)"),
    "fp8_scale_by_reciprocal": ("float s = a / 448.0f;", "float s = a * (1.0f / 448.0f);"),
    "fp8_codes_by_divide": ("float t = v[k] * inv;\n        if (t > 448.0f)", "float t = v[k] / s;\n        if (t > 448.0f)"),
    "int8_scale_by_reciprocal": ("float s = a / 127.0f;", "float s = a * (1.0f / 127.0f);"),
    "int8_codes_by_divide": ("float t = v[k] * inv;\n        t = rintf(t);",
                             "float t = v[k] / s;\n        t = rintf(t);"),
    "int8_inv_from_scale": ("float inv = 127.0f / a;", "float inv = 1.0f / s;"),
    "absmax_skips_first": ("for (int64_t k = 0; k < K; ++k) {\n        float m = fabsf(v[k]);",
                           "for (int64_t k = 1; k < K; ++k) {\n        float m = fabsf(v[k]);"),
    "gemm_skips_first_k": ("for (int64_t k = 0; k < K; ++k)\n                s += (int64_t)ar[k]",
                           "for (int64_t k = 1; k < K; ++k)\n                s += (int64_t)ar[k]"),
    "bias_before_w_scale": ("t = t * ws[n];\n            if (bias)\n                t = t + bf16_bits_to_float(bias[n]);\n"
                            "            out[m * ldo + n] = float_to_bf16_rne(t);",
                            "if (bias)\n                t = t + bf16_bits_to_float(bias[n]);\n            t = t * ws[n];\n"
                            "            out[m * ldo + n] = float_to_bf16_rne(t);"),
    "acc_transposed_index": ("float t = (float)acc[m * ldc + n];\n            t = t * xs[m];\n            t = t * ws[n];\n"
                             "            if (bias)\n                t = t + bf16_bits_to_float(bias[n]);",
                             "float t = (float)acc[(n % M) * ldc + (m % N)];\n            t = t * xs[m];\n"
                             "            t = t * ws[n];\n            if (bias)\n                t = t + bf16_bits_to_float(bias[n]);"),
    "fp8_no_zero_row_rule": ("if (a < 0x1p-100f) {\n        *scale = 0.0f;\n        for (int64_t k = 0; k < K; ++k)\n            q[k] = 0;\n        return;\n    }\n    float s = a / 448.0f;",
                             "if (a < 0.0f) {\n        *scale = 0.0f;\n        for (int64_t k = 0; k < K; ++k)\n            q[k] = 0;\n        return;\n    }\n    float s = a / 448.0f;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new, 1)
    path = os.path.join(tmp_path, "mutant.c")
    with open(path, "w") as f:
        f.write(mutated)
    lib = oracle.build(path, os.path.join(tmp_path, "libmutant.so"))
    o = oracle.Oracle(lib)
    failures = []
    for pin in P.ALL_PINS:
        try:
            pin(o)
        except (AssertionError, OverflowError, ValueError, IndexError) as e:
            failures.append(pin.__name__)
            break
    assert failures, f"no pin detects mutant {name}"
