/*
 * CPU oracle for W8A8 int8-dynamic linear layers.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call this code:
 * only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * load it. It shares no source, header, table or helper with the HIP library.
 *
 * It is the plain definition of what the layer computes, written as simple
 * loops in the order the method states, with OpenMP across rows only:
 *
 *   1. Per-token dynamic symmetric int8 activation quantization
 *      (page "Issue 5 probe: int8 quantized DiT serve paths on the RTX 3090
 *      (24 GB)", section "Round two": int8 weights with dynamic per-token
 *      symmetric int8 activations; page "Online Quantization", Parameters
 *      table: activation_scheme "dynamic" scales activations at run time).
 *   2. Per-output-channel symmetric int8 weight quantization with fp32
 *      scales (same page, "Round one" setup paragraph and the "Round two"
 *      artifacts paragraph: int8 weights unpacked plus fp32 per-channel
 *      scales). Both use the same rule on a row of floats.
 *   3. Exact int8 x int8 dot products (page "INT8 Quant for Dual-Max Recipe",
 *      the reply on the soak numbers: W8A8 multiplies int8 by int8 with no
 *      dequantization). Accumulated in int64, then checked to fit int32.
 *   4. The scale epilogue acc * a_scale[m] * w_scale[n] (+ bias) -> bf16
 *      (the "Round two" kernel-path paragraph: the probe that left out the
 *      act_scale factor saw the output norm shrink by E[act_scale]).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - symmetric int8 range is [-127, 127]; scale = absmax / 127;
 *   - q = clamp(rint_even(x * fl32(127 / absmax)), -127, 127);
 *   - a row whose absmax is below 2^-100 (including all-zero rows) gets
 *     scale 0 and all-zero codes;
 *   - epilogue in fp32, each step rounded once, no fused multiply-add:
 *     t = fl(fl(fl(acc) * xs) * ws); t = fl(t + bias); out = bf16_rne(t);
 *   - a second epilogue evaluates the same value in fp64 and rounds once
 *     to bf16, for tolerance checks independent of the fp32 order;
 *   - the fp16 twin (the pages run the layer with bf16 and with fp16
 *     activations: "Issue 5 probe ...", the Marlin isolation paragraph)
 *     widens fp16 activations exactly, takes its bias in fp16 and rounds
 *     the same fp32 value (or the fp64 one) to fp16, nearest-even, with
 *     gradual underflow and overflow to infinity.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC.
 * fp32 arithmetic here is IEEE single precision (SSE), round-to-nearest-even.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARGS 1
#define ORACLE_ERR_OVERFLOW 2

static float bf16_bits_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a float to bfloat16, nearest-even. Finite inputs; NaN maps to a
 * quiet NaN. Carry into the exponent handles the round-up to the next
 * binade (and to infinity) naturally. */
static uint16_t float_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu))
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

/* Round a double to bfloat16 once (no intermediate float rounding).
 * Normal bf16 range only; the magnitudes in this layer never leave it. */
static uint16_t double_to_bf16_rne(double d)
{
    if (d == 0.0)
        return signbit(d) ? 0x8000u : 0x0000u;
    int e;
    double m = frexp(fabs(d), &e);          /* |d| = m * 2^e, m in [0.5, 1) */
    double r = nearbyint(ldexp(m, 8));      /* 8 significant bits, ties to even */
    double v = ldexp(r, e - 8);             /* exactly representable in bf16 */
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u >>= 16;
    if (d < 0)
        u |= 0x8000u;
    return (uint16_t)u;
}

/* IEEE binary16 bits -> float (exact: every half is a float). */
static float f16_bits_to_float(uint16_t h)
{
    int sign = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    float v;
    if (e == 0)
        v = ldexpf((float)m, -24);                  /* zero and subnormals: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexpf((float)(m | 0x400), e - 25);     /* (1024 + m) * 2^(e-25) */
    return sign ? -v : v;
}

/* Round a double to binary16 once, nearest-even, with gradual underflow
 * (step 2^-24 below 2^-14) and overflow to infinity: a magnitude rounds to
 * infinity when it is at least 65520 (half way between 65504, the largest
 * half, and 65536, the next step). NaN maps to a quiet NaN. A float input
 * is widened to double exactly, so the same routine rounds floats once. */
static uint16_t double_to_f16_rne(double d)
{
    if (isnan(d))
        return 0x7e00u;
    uint16_t sign = signbit(d) ? 0x8000u : 0x0000u;
    double a = fabs(d);
    if (a >= 65520.0)
        return sign | 0x7c00u;
    int e;
    frexp(a, &e);                                   /* a = m * 2^e, m in [0.5, 1) */
    int q = e - 11;                                 /* step of an 11-bit significand */
    if (q < -24)
        q = -24;                                    /* subnormal step 2^-24 */
    double r = nearbyint(ldexp(a, -q));             /* a / 2^q, ties to even */
    /* r * 2^q is the rounded magnitude; r may have carried into 2^11. */
    if (r == 0.0)
        return sign;
    int k;
    frexp(r, &k);                                   /* r < 2^k */
    int exp_unbiased = q + k - 1;                   /* value in [2^exp, 2^(exp+1)) */
    if (exp_unbiased < -14)                         /* subnormal: bits are r itself */
        return sign | (uint16_t)r;
    uint32_t sig = (uint32_t)ldexp(r, 11 - k);      /* 11 bits, leading one at bit 10 */
    return sign | (uint16_t)((exp_unbiased + 15) << 10) | (uint16_t)(sig & 0x3ffu);
}

/* One row of floats -> int8 codes + fp32 scale (steps 1 and 2 above). */
static void quantize_row(const float *v, int64_t K, int8_t *q, float *scale)
{
    float a = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        float m = fabsf(v[k]);
        if (m > a)
            a = m;
    }
    if (a < 0x1p-100f) {
        *scale = 0.0f;
        for (int64_t k = 0; k < K; ++k)
            q[k] = 0;
        return;
    }
    float s = a / 127.0f;
    float inv = 127.0f / a;
    for (int64_t k = 0; k < K; ++k) {
        float t = v[k] * inv;
        t = rintf(t);                        /* default mode: nearest-even */
        if (t > 127.0f)
            t = 127.0f;
        if (t < -127.0f)
            t = -127.0f;
        q[k] = (int8_t)t;
    }
    *scale = s;
}

/* Per-token quantization of bf16 activations X[M, ldx] (first K columns).
 * Each row is widened to fp32 (exact) and passed through quantize_row. */
int oracle_quant_rows_bf16(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                           int8_t *q, int64_t ldq, float *scale)
{
    if (M < 0 || K < 1 || ldx < K || ldq < K || (M > 0 && (!x || !q || !scale)))
        return ORACLE_ERR_ARGS;
    int failed = 0;
#pragma omp parallel reduction(| : failed)
    {
        float *row = (float *)malloc((size_t)K * sizeof(float));
        if (!row) {
            failed = 1;
        } else {
            int64_t m;
#pragma omp for schedule(static)
            for (m = 0; m < M; ++m) {
                const uint16_t *xr = x + m * ldx;
                for (int64_t k = 0; k < K; ++k)
                    row[k] = bf16_bits_to_float(xr[k]);
                quantize_row(row, K, q + m * ldq, &scale[m]);
            }
            free(row);
        }
    }
    return failed ? ORACLE_ERR_ARGS : ORACLE_OK;
}

/* Per-token quantization of fp16 activations X[M, ldx] (first K columns):
 * the same as oracle_quant_rows_bf16 with fp16 widening. */
int oracle_quant_rows_f16(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                          int8_t *q, int64_t ldq, float *scale)
{
    if (M < 0 || K < 1 || ldx < K || ldq < K || (M > 0 && (!x || !q || !scale)))
        return ORACLE_ERR_ARGS;
    int failed = 0;
#pragma omp parallel reduction(| : failed)
    {
        float *row = (float *)malloc((size_t)K * sizeof(float));
        if (!row) {
            failed = 1;
        } else {
            int64_t m;
#pragma omp for schedule(static)
            for (m = 0; m < M; ++m) {
                const uint16_t *xr = x + m * ldx;
                for (int64_t k = 0; k < K; ++k)
                    row[k] = f16_bits_to_float(xr[k]);
                quantize_row(row, K, q + m * ldq, &scale[m]);
            }
            free(row);
        }
    }
    return failed ? ORACLE_ERR_ARGS : ORACLE_OK;
}

/* Per-output-channel quantization of fp32 weights W[N, ldw] (first K cols). */
int oracle_quant_rows_f32(const float *w, int64_t N, int64_t K, int64_t ldw,
                          int8_t *q, int64_t ldq, float *scale)
{
    if (N < 0 || K < 1 || ldw < K || ldq < K || (N > 0 && (!w || !q || !scale)))
        return ORACLE_ERR_ARGS;
    int64_t n;
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; ++n)
        quantize_row(w + n * ldw, K, q + n * ldq, &scale[n]);
    return ORACLE_OK;
}

/* acc[i, n] = sum_k A[rows[i], k] * B[n, k] for the listed rows of A
 * (rows == NULL means rows 0..M-1). Exact: int64 sums, then a range check. */
int oracle_gemm_i32_rows(const int8_t *a, int64_t lda, const int64_t *rows, int64_t M,
                         const int8_t *b, int64_t ldb, int64_t N, int64_t K,
                         int32_t *acc, int64_t ldc)
{
    if (M < 0 || N < 1 || K < 1 || lda < K || ldb < K || ldc < N ||
        (M > 0 && (!a || !b || !acc)))
        return ORACLE_ERR_ARGS;
    int overflow = 0;
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : overflow)
    for (i = 0; i < M; ++i) {
        const int8_t *ar = a + (rows ? rows[i] : i) * lda;
        for (int64_t n = 0; n < N; ++n) {
            const int8_t *br = b + n * ldb;
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int64_t)ar[k] * (int64_t)br[k];
            if (s > INT32_MAX || s < INT32_MIN)
                overflow = 1;
            acc[i * ldc + n] = (int32_t)s;
        }
    }
    return overflow ? ORACLE_ERR_OVERFLOW : ORACLE_OK;
}

/* fp32 epilogue, fixed order, one rounding per step; out is bf16 bits.
 * xs is indexed by the row of acc; bias may be NULL. */
int oracle_epilogue_f32(const int32_t *acc, int64_t ldc, int64_t M, int64_t N,
                        const float *xs, const float *ws, const uint16_t *bias,
                        uint16_t *out, int64_t ldo)
{
    if (M < 0 || N < 1 || ldc < N || ldo < N || (M > 0 && (!acc || !xs || !ws || !out)))
        return ORACLE_ERR_ARGS;
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            float t = (float)acc[m * ldc + n];
            t = t * xs[m];
            t = t * ws[n];
            if (bias)
                t = t + bf16_bits_to_float(bias[n]);
            out[m * ldo + n] = float_to_bf16_rne(t);
        }
    }
    return ORACLE_OK;
}

/* The same value in fp64 (acc * xs * ws + bias), rounded once to bf16. */
int oracle_epilogue_f64(const int32_t *acc, int64_t ldc, int64_t M, int64_t N,
                        const float *xs, const float *ws, const uint16_t *bias,
                        uint16_t *out, int64_t ldo)
{
    if (M < 0 || N < 1 || ldc < N || ldo < N || (M > 0 && (!acc || !xs || !ws || !out)))
        return ORACLE_ERR_ARGS;
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double t = (double)acc[m * ldc + n] * (double)xs[m] * (double)ws[n];
            if (bias)
                t += (double)bf16_bits_to_float(bias[n]);
            out[m * ldo + n] = double_to_bf16_rne(t);
        }
    }
    return ORACLE_OK;
}

/* The fp16 twin of the epilogue: bias and output are fp16 bits; the fp32
 * steps are the same, the last rounding goes to fp16 (nearest-even). */
int oracle_epilogue_f32_f16(const int32_t *acc, int64_t ldc, int64_t M, int64_t N,
                            const float *xs, const float *ws, const uint16_t *bias,
                            uint16_t *out, int64_t ldo)
{
    if (M < 0 || N < 1 || ldc < N || ldo < N || (M > 0 && (!acc || !xs || !ws || !out)))
        return ORACLE_ERR_ARGS;
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            float t = (float)acc[m * ldc + n];
            t = t * xs[m];
            t = t * ws[n];
            if (bias)
                t = t + f16_bits_to_float(bias[n]);
            out[m * ldo + n] = double_to_f16_rne((double)t);
        }
    }
    return ORACLE_OK;
}

/* The same value in fp64, rounded once to fp16. */
int oracle_epilogue_f64_f16(const int32_t *acc, int64_t ldc, int64_t M, int64_t N,
                            const float *xs, const float *ws, const uint16_t *bias,
                            uint16_t *out, int64_t ldo)
{
    if (M < 0 || N < 1 || ldc < N || ldo < N || (M > 0 && (!acc || !xs || !ws || !out)))
        return ORACLE_ERR_ARGS;
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double t = (double)acc[m * ldc + n] * (double)xs[m] * (double)ws[n];
            if (bias)
                t += (double)f16_bits_to_float(bias[n]);
            out[m * ldo + n] = double_to_f16_rne(t);
        }
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------
 * The FP8 (e4m3) W8A8 twin (page "Online Quantization": FP8 W8A8 with the
 * "dynamic" activation scheme in its Parameters table). The pages give no
 * formula; the reading mirrors the int8 path: per-token activation scales
 * and per-output-channel weight scales, scale = absmax / 448 (448 is the
 * largest finite OCP e4m3 value), code = e4m3_rne(clamp(x * fl32(448 /
 * absmax), -448, 448)), a row below 2^-100 gets scale 0 and zero codes.
 * Products of two e4m3 values and their sums over K are exact in double
 * (every product is a multiple of 2^-18 below 2^18), so the accumulators
 * here are exact; the epilogue takes them rounded once to fp32.
 * OCP e4m3: sign, 4 exponent bits (bias 7), 3 mantissa bits; no infinity;
 * S.1111.111 is NaN; subnormals m * 2^-9.
 * --------------------------------------------------------------------- */
static double e4m3_to_double(uint8_t c)
{
    int sign = c >> 7, e = (c >> 3) & 0xf, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 10);
    return sign ? -v : v;
}

/* Round to e4m3 once, nearest-even; |d| must not exceed 448 (callers
 * clamp first), so no result leaves the finite range. */
static uint8_t double_to_e4m3_rne(double d)
{
    uint8_t sign = signbit(d) ? 0x80u : 0x00u;
    double a = fabs(d);
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);                                   /* a in [2^(e-1), 2^e) */
    int q = e - 4;                                  /* step of a 4-bit significand */
    if (q < -9)
        q = -9;                                     /* subnormal step 2^-9 */
    double r = nearbyint(ldexp(a, -q));             /* ties to even */
    if (r == 0.0)
        return sign;
    int k;
    frexp(r, &k);
    int exp_unbiased = q + k - 1;
    if (exp_unbiased < -6)                          /* subnormal: bits are r */
        return sign | (uint8_t)r;
    uint32_t sig = (uint32_t)ldexp(r, 4 - k);       /* 4 bits, leading one at bit 3 */
    return sign | (uint8_t)((exp_unbiased + 7) << 3) | (uint8_t)(sig & 7u);
}

static void quantize_row_fp8(const float *v, int64_t K, uint8_t *q, float *scale)
{
    float a = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        float m = fabsf(v[k]);
        if (m > a)
            a = m;
    }
    if (a < 0x1p-100f) {
        *scale = 0.0f;
        for (int64_t k = 0; k < K; ++k)
            q[k] = 0;
        return;
    }
    float s = a / 448.0f;
    float inv = 448.0f / a;
    for (int64_t k = 0; k < K; ++k) {
        float t = v[k] * inv;
        if (t > 448.0f)
            t = 448.0f;
        if (t < -448.0f)
            t = -448.0f;
        q[k] = double_to_e4m3_rne((double)t);
    }
    *scale = s;
}

/* FP8 codes of bf16 rows (activations, per token) or fp32 rows (weights,
 * per output channel). */
int oracle_fp8_quant_rows_bf16(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                               uint8_t *q, int64_t ldq, float *scale)
{
    if (M < 0 || K < 1 || ldx < K || ldq < K || (M > 0 && (!x || !q || !scale)))
        return ORACLE_ERR_ARGS;
    int failed = 0;
#pragma omp parallel reduction(| : failed)
    {
        float *row = (float *)malloc((size_t)K * sizeof(float));
        if (!row) {
            failed = 1;
        } else {
            int64_t m;
#pragma omp for schedule(static)
            for (m = 0; m < M; ++m) {
                for (int64_t k = 0; k < K; ++k)
                    row[k] = bf16_bits_to_float(x[m * ldx + k]);
                quantize_row_fp8(row, K, q + m * ldq, &scale[m]);
            }
            free(row);
        }
    }
    return failed ? ORACLE_ERR_ARGS : ORACLE_OK;
}

int oracle_fp8_quant_rows_f32(const float *w, int64_t N, int64_t K, int64_t ldw, uint8_t *q,
                              int64_t ldq, float *scale)
{
    if (N < 0 || K < 1 || ldw < K || ldq < K || (N > 0 && (!w || !q || !scale)))
        return ORACLE_ERR_ARGS;
    int64_t n;
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; ++n)
        quantize_row_fp8(w + n * ldw, K, q + n * ldq, &scale[n]);
    return ORACLE_OK;
}

/* acc[i, n] = sum_k dec(A[rows[i], k]) * dec(B[n, k]), exact (double). */
int oracle_fp8_gemm_rows(const uint8_t *a, int64_t lda, const int64_t *rows, int64_t M,
                         const uint8_t *b, int64_t ldb, int64_t N, int64_t K, double *acc,
                         int64_t ldc)
{
    if (M < 0 || N < 1 || K < 1 || lda < K || ldb < K || ldc < N ||
        (M > 0 && (!a || !b || !acc)))
        return ORACLE_ERR_ARGS;
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < M; ++i) {
        const uint8_t *ar = a + (rows ? rows[i] : i) * lda;
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t *br = b + n * ldb;
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s += e4m3_to_double(ar[k]) * e4m3_to_double(br[k]);
            acc[i * ldc + n] = s;
        }
    }
    return ORACLE_OK;
}

/* The epilogue on exact accumulators: fl32(acc), then the fp32 order of
 * oracle_epilogue_f32; and the fp64 value rounded once, the tolerance
 * reference. Bias and outputs are bf16 bits, or fp16 bits when f16. */
int oracle_fp8_epilogue(const double *acc, int64_t ldc, int64_t M, int64_t N, const float *xs,
                        const float *ws, const uint16_t *bias, uint16_t *out32, uint16_t *out64,
                        int64_t ldo, int f16)
{
    if (M < 0 || N < 1 || ldc < N || ldo < N ||
        (M > 0 && (!acc || !xs || !ws || !out32 || !out64)))
        return ORACLE_ERR_ARGS;
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            const float b = !bias ? 0.0f : f16 ? f16_bits_to_float(bias[n])
                                                : bf16_bits_to_float(bias[n]);
            float t = (float)acc[m * ldc + n];
            t = t * xs[m];
            t = t * ws[n];
            if (bias)
                t = t + b;
            out32[m * ldo + n] = f16 ? double_to_f16_rne((double)t) : float_to_bf16_rne(t);
            double d = acc[m * ldc + n] * (double)xs[m] * (double)ws[n];
            if (bias)
                d += (double)b;
            out64[m * ldo + n] = f16 ? double_to_f16_rne(d) : double_to_bf16_rne(d);
        }
    }
    return ORACLE_OK;
}

uint8_t oracle_double_to_e4m3(double d) { return double_to_e4m3_rne(d); }
double oracle_e4m3_to_double(uint8_t c) { return e4m3_to_double(c); }

/* Exposed for the pins: the scalar conversions used above. */
uint16_t oracle_float_to_bf16(float f) { return float_to_bf16_rne(f); }
uint16_t oracle_double_to_bf16(double d) { return double_to_bf16_rne(d); }
uint16_t oracle_double_to_f16(double d) { return double_to_f16_rne(d); }
float oracle_f16_to_float(uint16_t h) { return f16_bits_to_float(h); }
