// Per-row symmetric int8 quantization on gfx950.
//
// One kernel family serves two steps of the layer: the dynamic per-token
// activation quant (bf16 or fp16 rows; page "Issue 5 probe: int8 quantized
// DiT serve paths on the RTX 3090 (24 GB)", section "Round two", and the
// isolation table's bf16 and fp16 activation columns) and the
// per-output-channel weight quant (fp32 rows; same page, "Round one" setup
// and "Round two" artifacts paragraphs). The rule per row:
//   a = max |x|;  a < 2^-100 -> scale 0, codes 0;
//   else scale = fl32(a/127), inv = fl32(127/a),
//        q = clamp(rint_even(fl32(x*inv)), -127, 127).
//
// Design (HBM-bound; 3 bytes move per bf16 element):
//   - A row is split over WPR wavefronts (1, 2 or 4); each lane holds CH
//     16-byte chunks of the row in VGPRs, so HBM is read exactly once.
//     Chunk c of lane l in wave w of the row starts at element
//     ((c*WPR + w)*64 + l) * VEC: each load instruction moves 1 KiB of
//     consecutive bytes (fully coalesced dwordx4).
//   - |x| max is taken on the raw bit patterns (sign bit cleared), which
//     order like the values; a wavefront reduces with DPP (quad_perm,
//     row_half_mirror, row_mirror) and four readlanes; the WPR partials of
//     a row meet in LDS.
//   - Codes are written 8 (bf16, fp16) or 4 (fp32) per lane per chunk.
//   - The FP8 instantiations write e4m3 codes with scale absmax / 448 (the
//     e4m3 twin of the layer; bf16 activations and fp32 weights).
//   - The row loads of the single-pass kernel are nontemporal, and so are
//     the code stores of a quant on its own (each byte is touched once, and
//     keeping it out of the caches lifts HBM throughput). When the matmul
//     reads the codes in the very next launch (the two-launch form of
//     int8_quant_scaled_mm) they are stored plainly and stay in the caches:
//     measured on MI355X, the FFN-down layer's two launches 314 to 298 us,
//     while the quant alone of the FFN-up shape slows from 7.1 to 8.0 us.
//   - Rows longer than the register-resident limit take a two-pass kernel
//     that re-reads the row (from L2) for the quantize pass.
// Every tail (K not a multiple of the chunk width, rows beyond the last)
// is masked element by element.
#include <algorithm>

#include "internal.hpp"
#include "quant_rule.hpp"

namespace w8a8 {
namespace {

using namespace quant_rule;

// Register-resident kernel: CH chunks per lane, WPR waves per row, 4 waves per block.
template <int E, int CH, int WPR, bool FP8, bool STREAM>
__global__ __launch_bounds__(256) void quant_rows_kernel(const void *__restrict__ x, int64_t rows,
                                                         int K, int64_t ldx,
                                                         int8_t *__restrict__ q, int64_t ldq,
                                                         float *__restrict__ scale)
{
    constexpr int VEC = Elem<E>::VEC;
    constexpr int RPB = 4 / WPR;
    __shared__ u32 part[4];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave % WPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + wave / WPR;
    const bool valid = row < rows;
    const char *xrow = reinterpret_cast<const char *>(x) + row * ldx * Elem<E>::BYTES;

    uint4 v[CH];
    u32 m = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int64_t e = ((int64_t)(c * WPR + wr) * 64 + lane) * VEC;
        v[c] = (valid && e < K) ? load_chunk<E, true>(xrow, e, K) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c)
        m = max(m, chunk_absmax<E>(v[c]));
    m = wave_max(m);
    if (WPR > 1) {
        if (lane == 0)
            part[wave] = m;
        __syncthreads();
        const int first = (wave / WPR) * WPR;
        m = part[first];
#pragma unroll
        for (int i = 1; i < WPR; ++i)
            m = max(m, part[first + i]);
    }
    if (!valid)
        return;
    float s, inv;
    scale_of(m, E, s, inv, FP8);
    if (wr == 0 && lane == 0)
        scale[row] = s;
    int8_t *qrow = q + row * ldq;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int64_t e = ((int64_t)(c * WPR + wr) * 64 + lane) * VEC;
        if (e < K) {
            u32 lo, hi;
            chunk_codes<E, FP8>(v[c], inv, lo, hi);
            store_codes<E, STREAM>(qrow, e, K, lo, hi);
        }
    }
}

// Two-pass kernel for rows longer than the register-resident limit:
// one row per block of 4 waves; pass 1 finds the absmax, pass 2 re-reads.
template <int E, bool FP8, bool STREAM>
__global__ __launch_bounds__(256) void quant_rows_looped_kernel(const void *__restrict__ x,
                                                                int64_t rows, int K, int64_t ldx,
                                                                int8_t *__restrict__ q, int64_t ldq,
                                                                float *__restrict__ scale)
{
    constexpr int VEC = Elem<E>::VEC;
    __shared__ u32 part[4];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row = blockIdx.x;
    const char *xrow = reinterpret_cast<const char *>(x) + row * ldx * Elem<E>::BYTES;
    const int64_t step = 256 * VEC;
    u32 m = 0;
    for (int64_t e = (int64_t)threadIdx.x * VEC; e < K; e += step)
        m = max(m, chunk_absmax<E>(load_chunk<E>(xrow, e, K)));
    m = wave_max(m);
    if (lane == 0)
        part[wave] = m;
    __syncthreads();
    m = max(max(part[0], part[1]), max(part[2], part[3]));
    float s, inv;
    scale_of(m, E, s, inv, FP8);
    if (threadIdx.x == 0)
        scale[row] = s;
    int8_t *qrow = q + row * ldq;
    for (int64_t e = (int64_t)threadIdx.x * VEC; e < K; e += step) {
        u32 lo, hi;
        chunk_codes<E, FP8>(load_chunk<E>(xrow, e, K), inv, lo, hi);
        store_codes<E, STREAM>(qrow, e, K, lo, hi);
    }
}

typedef void (*QuantFn)(const void *, int64_t, int, int64_t, int8_t *, int64_t, float *);

constexpr int kChOptions[] = {1, 2, 3, 4, 6, 8, 12, 16};
constexpr int kNumCh = sizeof(kChOptions) / sizeof(kChOptions[0]);
constexpr int kWprOptions[] = {1, 2, 4};

template <int E, int WPR, bool FP8, bool STREAM>
QuantFn pick_ch(int idx)
{
    switch (idx) {
    case 0: return quant_rows_kernel<E, 1, WPR, FP8, STREAM>;
    case 1: return quant_rows_kernel<E, 2, WPR, FP8, STREAM>;
    case 2: return quant_rows_kernel<E, 3, WPR, FP8, STREAM>;
    case 3: return quant_rows_kernel<E, 4, WPR, FP8, STREAM>;
    case 4: return quant_rows_kernel<E, 6, WPR, FP8, STREAM>;
    case 5: return quant_rows_kernel<E, 8, WPR, FP8, STREAM>;
    case 6: return quant_rows_kernel<E, 12, WPR, FP8, STREAM>;
    default: return quant_rows_kernel<E, 16, WPR, FP8, STREAM>;
    }
}

template <int E, bool FP8, bool STREAM>
QuantFn pick(int wpr, int ch_idx)
{
    switch (wpr) {
    case 1: return pick_ch<E, 1, FP8, STREAM>(ch_idx);
    case 2: return pick_ch<E, 2, FP8, STREAM>(ch_idx);
    default: return pick_ch<E, 4, FP8, STREAM>(ch_idx);
    }
}

// The kernel for an element kind and code type; weights (fp32 rows) always
// stream their codes.
template <bool STREAM>
QuantFn pick_kind(int kind, bool fp8, int wpr, int ch_idx)
{
    if (kind == kF32)
        return fp8 ? pick<kF32, true, true>(wpr, ch_idx) : pick<kF32, false, true>(wpr, ch_idx);
    if (fp8)
        return pick<kBF16, true, STREAM>(wpr, ch_idx);
    return kind == kF16 ? pick<kF16, false, STREAM>(wpr, ch_idx) : pick<kBF16, false, STREAM>(wpr, ch_idx);
}

template <bool STREAM>
QuantFn pick_looped(int kind, bool fp8)
{
    if (kind == kF32)
        return fp8 ? quant_rows_looped_kernel<kF32, true, true> : quant_rows_looped_kernel<kF32, false, true>;
    if (fp8)
        return quant_rows_looped_kernel<kBF16, true, STREAM>;
    return kind == kF16 ? quant_rows_looped_kernel<kF16, false, STREAM>
                        : quant_rows_looped_kernel<kBF16, false, STREAM>;
}

}  // namespace

namespace {

// Launches fn over rows [0, rows) in slices of at most kMaxBlocksPerLaunch
// workgroups of rpb rows each.
hipError_t launch_row_slices(QuantFn fn, int rpb, const void *x, int esize, int64_t rows, int K,
                             int64_t ldx, int8_t *q, int64_t ldq, float *scale,
                             hipStream_t stream)
{
    const int64_t step = kMaxBlocksPerLaunch * rpb;
    for (int64_t r0 = 0; r0 < rows; r0 += step) {
        const int64_t n = std::min(rows - r0, step);
        hipLaunchKernelGGL(fn, dim3((unsigned)ceil_div(n, rpb)), dim3(256), 0, stream,
                           static_cast<const char *>(x) + r0 * ldx * esize, n, K, ldx,
                           q + r0 * ldq, ldq, scale + r0);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_quant_rows(const void *x, int kind, int64_t rows, int64_t K, int64_t ldx,
                             int8_t *q, int64_t ldq, float *scale, hipStream_t stream, bool fp8,
                             bool keep_codes)
{
    if (rows == 0)
        return hipSuccess;
    const int vec = kind == kF32 ? 4 : 8;
    const int esize = kind == kF32 ? 4 : 2;
    const int64_t chunks = ceil_div(K, vec);
    // Fewest waves per row that keep the row in registers, unless the grid
    // would then have too few waves to cover the machine's latency.
    const int64_t kEnoughWaves = 4096;
    for (int wi = 0; wi < 3; ++wi) {
        const int wpr = kWprOptions[wi];
        const int64_t need = ceil_div(chunks, 64 * wpr);
        int ch_idx = -1;
        for (int i = 0; i < kNumCh; ++i)
            if (kChOptions[i] >= need) {
                ch_idx = i;
                break;
            }
        if (ch_idx < 0)
            continue;
        if (wpr < 4 && need > 1 && rows * wpr < kEnoughWaves)
            continue;
        const int rpb = 4 / wpr;
        QuantFn fn = keep_codes ? pick_kind<false>(kind, fp8, wpr, ch_idx)
                                : pick_kind<true>(kind, fp8, wpr, ch_idx);
        return launch_row_slices(fn, rpb, x, esize, rows, (int)K, ldx, q, ldq, scale, stream);
    }
    QuantFn fn = keep_codes ? pick_looped<false>(kind, fp8) : pick_looped<true>(kind, fp8);
    return launch_row_slices(fn, 1, x, esize, rows, (int)K, ldx, q, ldq, scale, stream);
}

}  // namespace w8a8
