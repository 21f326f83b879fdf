// Per-row symmetric int8 quantization on gfx950.
//
// One kernel family serves two steps of the layer: the dynamic per-token
// activation quant (bf16 rows; page "Issue 5 probe: int8 quantized DiT serve
// paths on the RTX 3090 (24 GB)", section "Round two") and the
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
//   - Codes are written 8 (bf16) or 4 (fp32) per lane per chunk.
//   - The row loads of the single-pass kernel and all code stores are
//     nontemporal: each byte is touched once, and keeping it out of the
//     caches lifts HBM throughput.
//   - Rows longer than the register-resident limit take a two-pass kernel
//     that re-reads the row (from L2) for the quantize pass.
// Every tail (K not a multiple of the chunk width, rows beyond the last)
// is masked element by element.
#include "internal.hpp"

namespace w8a8 {
namespace {

typedef unsigned int u32;
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

// Wavefront max of non-negative values carried as unsigned bit patterns.
__device__ __forceinline__ u32 wave_max(u32 v)
{
    // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror:
    // afterwards every lane of a 16-lane row holds the row's max.
    v = max(v, (u32)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));
    v = max(v, (u32)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));
    v = max(v, (u32)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false));
    v = max(v, (u32)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false));
    u32 r0 = (u32)__builtin_amdgcn_readlane((int)v, 0);
    u32 r1 = (u32)__builtin_amdgcn_readlane((int)v, 16);
    u32 r2 = (u32)__builtin_amdgcn_readlane((int)v, 32);
    u32 r3 = (u32)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(r0, r1), max(r2, r3));
}

template <bool F32>
struct Elem {
    static constexpr int VEC = F32 ? 4 : 8;       // elements per 16-byte chunk
    static constexpr int BYTES = F32 ? 4 : 2;
};

// Largest |x| bit pattern in one chunk.
template <bool F32>
__device__ __forceinline__ u32 chunk_absmax(const uint4 &v)
{
    const u32 d[4] = {v.x, v.y, v.z, v.w};
    u32 m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (F32) {
            m = max(m, d[i] & 0x7fffffffu);
        } else {
            m = max(m, d[i] & 0x7fffu);
            m = max(m, (d[i] >> 16) & 0x7fffu);
        }
    }
    return m;
}

__device__ __forceinline__ u32 code(float f, float inv)
{
    float t = __builtin_rintf(f * inv);
    t = fminf(fmaxf(t, -127.0f), 127.0f);
    return (u32)((int)t) & 0xffu;
}

// Codes of one chunk: bf16 -> 8 codes in (lo, hi); fp32 -> 4 codes in lo.
template <bool F32>
__device__ __forceinline__ void chunk_codes(const uint4 &v, float inv, u32 &lo, u32 &hi)
{
    const u32 d[4] = {v.x, v.y, v.z, v.w};
    if (F32) {
        lo = code(__uint_as_float(d[0]), inv) | code(__uint_as_float(d[1]), inv) << 8 |
             code(__uint_as_float(d[2]), inv) << 16 | code(__uint_as_float(d[3]), inv) << 24;
        hi = 0;
    } else {
        u32 c[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            c[2 * i] = code(__uint_as_float(d[i] << 16), inv);
            c[2 * i + 1] = code(__uint_as_float(d[i] & 0xffff0000u), inv);
        }
        lo = c[0] | c[1] << 8 | c[2] << 16 | c[3] << 24;
        hi = c[4] | c[5] << 8 | c[6] << 16 | c[7] << 24;
    }
}

// Load chunk starting at element e of a row (row pointer as bytes). STREAM
// marks the data as read once (nontemporal: it is not kept in the caches),
// which the single-pass kernel uses; measured on MI355X this raises the
// quant's HBM throughput by about 14 % on 300 MB passes.
template <bool F32, bool STREAM = false>
__device__ __forceinline__ uint4 load_chunk(const char *row, int64_t e, int K)
{
    constexpr int VEC = Elem<F32>::VEC;
    constexpr int B = Elem<F32>::BYTES;
    if (e + VEC <= K) {
        if (STREAM) {
            const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(row + e * B));
            return make_uint4(t[0], t[1], t[2], t[3]);
        }
        return *reinterpret_cast<const uint4 *>(row + e * B);
    }
    u32 w[4] = {0, 0, 0, 0};
    for (int j = 0; j < VEC; ++j) {
        if (e + j < K) {
            if (F32)
                w[j] = reinterpret_cast<const u32 *>(row)[e + j];
            else
                w[j >> 1] |= (u32)reinterpret_cast<const uint16_t *>(row)[e + j] << (16 * (j & 1));
        }
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

template <bool F32>
__device__ __forceinline__ void store_codes(int8_t *qrow, int64_t e, int K, u32 lo, u32 hi)
{
    constexpr int VEC = Elem<F32>::VEC;
    if (e + VEC <= K) {
        // The codes are not read again by this pass: stream them out.
        if (F32)
            __builtin_nontemporal_store(lo, reinterpret_cast<u32 *>(qrow + e));
        else
            __builtin_nontemporal_store(v2u{lo, hi}, reinterpret_cast<v2u *>(qrow + e));
        return;
    }
    for (int j = 0; j < VEC; ++j)
        if (e + j < K)
            qrow[e + j] = (int8_t)((j < 4 ? lo >> (8 * j) : hi >> (8 * (j - 4))) & 0xffu);
}

__device__ __forceinline__ void scale_of(u32 m, bool f32, float &s, float &inv)
{
    const float a = __uint_as_float(f32 ? m : m << 16);
    if (a < 0x1p-100f) {
        s = 0.0f;
        inv = 0.0f;                      // x * 0 -> code 0 for every element
    } else {
        s = a / 127.0f;                  // correctly rounded fp32 divide
        inv = 127.0f / a;
    }
}

// Register-resident kernel: CH chunks per lane, WPR waves per row, 4 waves per block.
template <bool F32, int CH, int WPR>
__global__ __launch_bounds__(256) void quant_rows_kernel(const void *__restrict__ x, int64_t rows,
                                                         int K, int64_t ldx,
                                                         int8_t *__restrict__ q, int64_t ldq,
                                                         float *__restrict__ scale)
{
    constexpr int VEC = Elem<F32>::VEC;
    constexpr int RPB = 4 / WPR;
    __shared__ u32 part[4];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave % WPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + wave / WPR;
    const bool valid = row < rows;
    const char *xrow = reinterpret_cast<const char *>(x) + row * ldx * Elem<F32>::BYTES;

    uint4 v[CH];
    u32 m = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int64_t e = ((int64_t)(c * WPR + wr) * 64 + lane) * VEC;
        v[c] = (valid && e < K) ? load_chunk<F32, true>(xrow, e, K) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c)
        m = max(m, chunk_absmax<F32>(v[c]));
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
    scale_of(m, F32, s, inv);
    if (wr == 0 && lane == 0)
        scale[row] = s;
    int8_t *qrow = q + row * ldq;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int64_t e = ((int64_t)(c * WPR + wr) * 64 + lane) * VEC;
        if (e < K) {
            u32 lo, hi;
            chunk_codes<F32>(v[c], inv, lo, hi);
            store_codes<F32>(qrow, e, K, lo, hi);
        }
    }
}

// Two-pass kernel for rows longer than the register-resident limit:
// one row per block of 4 waves; pass 1 finds the absmax, pass 2 re-reads.
template <bool F32>
__global__ __launch_bounds__(256) void quant_rows_looped_kernel(const void *__restrict__ x,
                                                                int64_t rows, int K, int64_t ldx,
                                                                int8_t *__restrict__ q, int64_t ldq,
                                                                float *__restrict__ scale)
{
    constexpr int VEC = Elem<F32>::VEC;
    __shared__ u32 part[4];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row = blockIdx.x;
    const char *xrow = reinterpret_cast<const char *>(x) + row * ldx * Elem<F32>::BYTES;
    const int64_t step = 256 * VEC;
    u32 m = 0;
    for (int64_t e = (int64_t)threadIdx.x * VEC; e < K; e += step)
        m = max(m, chunk_absmax<F32>(load_chunk<F32>(xrow, e, K)));
    m = wave_max(m);
    if (lane == 0)
        part[wave] = m;
    __syncthreads();
    m = max(max(part[0], part[1]), max(part[2], part[3]));
    float s, inv;
    scale_of(m, F32, s, inv);
    if (threadIdx.x == 0)
        scale[row] = s;
    int8_t *qrow = q + row * ldq;
    for (int64_t e = (int64_t)threadIdx.x * VEC; e < K; e += step) {
        u32 lo, hi;
        chunk_codes<F32>(load_chunk<F32>(xrow, e, K), inv, lo, hi);
        store_codes<F32>(qrow, e, K, lo, hi);
    }
}

typedef void (*QuantFn)(const void *, int64_t, int, int64_t, int8_t *, int64_t, float *);

constexpr int kChOptions[] = {1, 2, 3, 4, 6, 8, 12, 16};
constexpr int kNumCh = sizeof(kChOptions) / sizeof(kChOptions[0]);
constexpr int kWprOptions[] = {1, 2, 4};

template <bool F32, int WPR>
QuantFn pick_ch(int idx)
{
    switch (idx) {
    case 0: return quant_rows_kernel<F32, 1, WPR>;
    case 1: return quant_rows_kernel<F32, 2, WPR>;
    case 2: return quant_rows_kernel<F32, 3, WPR>;
    case 3: return quant_rows_kernel<F32, 4, WPR>;
    case 4: return quant_rows_kernel<F32, 6, WPR>;
    case 5: return quant_rows_kernel<F32, 8, WPR>;
    case 6: return quant_rows_kernel<F32, 12, WPR>;
    default: return quant_rows_kernel<F32, 16, WPR>;
    }
}

template <bool F32>
QuantFn pick(int wpr, int ch_idx)
{
    switch (wpr) {
    case 1: return pick_ch<F32, 1>(ch_idx);
    case 2: return pick_ch<F32, 2>(ch_idx);
    default: return pick_ch<F32, 4>(ch_idx);
    }
}

}  // namespace

hipError_t launch_quant_rows(const void *x, bool in_f32, int64_t rows, int64_t K, int64_t ldx,
                             int8_t *q, int64_t ldq, float *scale, hipStream_t stream)
{
    if (rows == 0)
        return hipSuccess;
    const int vec = in_f32 ? 4 : 8;
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
        QuantFn fn = in_f32 ? pick<true>(wpr, ch_idx) : pick<false>(wpr, ch_idx);
        hipLaunchKernelGGL(fn, dim3((unsigned)ceil_div(rows, rpb)), dim3(256), 0, stream, x, rows,
                           (int)K, ldx, q, ldq, scale);
        return hipGetLastError();
    }
    if (in_f32)
        hipLaunchKernelGGL(quant_rows_looped_kernel<true>, dim3((unsigned)rows), dim3(256), 0,
                           stream, x, rows, (int)K, ldx, q, ldq, scale);
    else
        hipLaunchKernelGGL(quant_rows_looped_kernel<false>, dim3((unsigned)rows), dim3(256), 0,
                           stream, x, rows, (int)K, ldx, q, ldq, scale);
    return hipGetLastError();
}

}  // namespace w8a8
