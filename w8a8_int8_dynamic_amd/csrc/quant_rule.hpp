// The per-row symmetric int8 quantization rule, shared by the quant kernels
// and the fused quant + matmul path so that both produce the same codes bit
// for bit (page "Issue 5 probe: int8 quantized DiT serve paths on the RTX
// 3090 (24 GB)", section "Round two": dynamic per-token symmetric int8).
// Rows are bf16, fp32 or fp16 (element kinds kBF16, kF32, kF16; a bool
// template argument false / true still means bf16 / fp32); every element is
// widened to fp32 exactly first:
//   a = max |x|;  a < 2^-100 -> scale 0, codes 0;
//   else scale = fl32(a/127), inv = fl32(127/a),
//        q = clamp(rint_even(fl32(x*inv)), -127, 127).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {
namespace quant_rule {

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

constexpr int kBF16 = 0, kF32 = 1, kF16 = 2;

template <int E>
struct Elem {
    static constexpr bool F32 = E == kF32;
    static constexpr int VEC = F32 ? 4 : 8;       // elements per 16-byte chunk
    static constexpr int BYTES = F32 ? 4 : 2;
};

// fp16 bits (low 16 bits of h) -> fp32, exact.
__device__ __forceinline__ float f16_to_float(u32 h)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xffffu));
}

// Largest |x| bit pattern in one chunk (for bf16 and fp16 alike the 15 low
// bits of a 16-bit value order magnitudes).
template <int E>
__device__ __forceinline__ u32 chunk_absmax(const uint4 &v)
{
    constexpr bool F32 = E == kF32;
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

// The e4m3 twin's codes of four values (OCP e4m3: 4 exponent bits, bias 7,
// 3 mantissa bits, largest finite 448): t = clamp(fl32(f*inv), -448, 448)
// rounded to the nearest e4m3 value, ties to even, the sign kept (zeros
// included). gfx950's packed fp32 -> e4m3 conversion does the rounding, two
// values per instruction (bytes 0-1, then 2-3); the clamp keeps every input
// inside the finite range, away from its overflow handling.
__device__ __forceinline__ u32 codes4_fp8(float f0, float f1, float f2, float f3, float inv)
{
    auto t = [inv](float f) __attribute__((always_inline)) {
        return fminf(fmaxf(f * inv, -448.0f), 448.0f);
    };
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(t(f0), t(f1), 0, false);
    return (u32)__builtin_amdgcn_cvt_pk_fp8_f32(t(f2), t(f3), lo, true);
}

__device__ __forceinline__ u32 codes4_i8(float f0, float f1, float f2, float f3, float inv)
{
    return code(f0, inv) | code(f1, inv) << 8 | code(f2, inv) << 16 | code(f3, inv) << 24;
}

template <bool FP8>
__device__ __forceinline__ u32 codes4(float f0, float f1, float f2, float f3, float inv)
{
    return FP8 ? codes4_fp8(f0, f1, f2, f3, inv) : codes4_i8(f0, f1, f2, f3, inv);
}

// Codes of one chunk: bf16 or fp16 -> 8 codes in (lo, hi); fp32 -> 4 codes
// in lo. FP8: e4m3 codes instead of int8.
template <int E, bool FP8 = false>
__device__ __forceinline__ void chunk_codes(const uint4 &v, float inv, u32 &lo, u32 &hi)
{
    const u32 d[4] = {v.x, v.y, v.z, v.w};
    if (E == kF32) {
        lo = codes4<FP8>(__uint_as_float(d[0]), __uint_as_float(d[1]), __uint_as_float(d[2]),
                         __uint_as_float(d[3]), inv);
        hi = 0;
    } else {
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (E == kF16) {
                f[2 * i] = f16_to_float(d[i]);
                f[2 * i + 1] = f16_to_float(d[i] >> 16);
            } else {
                f[2 * i] = __uint_as_float(d[i] << 16);
                f[2 * i + 1] = __uint_as_float(d[i] & 0xffff0000u);
            }
        }
        lo = codes4<FP8>(f[0], f[1], f[2], f[3], inv);
        hi = codes4<FP8>(f[4], f[5], f[6], f[7], inv);
    }
}

// Load chunk starting at element e of a row (row pointer as bytes). STREAM
// marks the data as read once (nontemporal: it is not kept in the caches),
// which the single-pass kernel uses; measured on MI355X this raises the
// quant's HBM throughput by about 14 % on 300 MB passes.
template <int E, bool STREAM = false>
__device__ __forceinline__ uint4 load_chunk(const char *row, int64_t e, int K)
{
    constexpr bool F32 = E == kF32;
    constexpr int VEC = Elem<E>::VEC;
    constexpr int B = Elem<E>::BYTES;
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

// STREAM: the codes are written with nontemporal stores (nothing reads them
// soon); otherwise with plain stores, so that they stay in the caches for
// the launch that reads them next.
template <int E, bool STREAM = true>
__device__ __forceinline__ void store_codes(int8_t *qrow, int64_t e, int K, u32 lo, u32 hi)
{
    constexpr bool F32 = E == kF32;
    constexpr int VEC = Elem<E>::VEC;
    if (e + VEC <= K) {
        if constexpr (STREAM) {
            if (F32)
                __builtin_nontemporal_store(lo, reinterpret_cast<u32 *>(qrow + e));
            else
                __builtin_nontemporal_store(v2u{lo, hi}, reinterpret_cast<v2u *>(qrow + e));
        } else {
            if (F32)
                *reinterpret_cast<u32 *>(qrow + e) = lo;
            else
                *reinterpret_cast<v2u *>(qrow + e) = v2u{lo, hi};
        }
        return;
    }
    for (int j = 0; j < VEC; ++j)
        if (e + j < K)
            qrow[e + j] = (int8_t)((j < 4 ? lo >> (8 * j) : hi >> (8 * (j - 4))) & 0xffu);
}

// Scale and reciprocal of a row from its absmax bit pattern m (kind e):
// absmax / 127 for int8 codes, absmax / 448 for the e4m3 twin.
__device__ __forceinline__ void scale_of(u32 m, int e, float &s, float &inv, bool fp8 = false)
{
    const float a = e == kF32   ? __uint_as_float(m)
                    : e == kF16 ? f16_to_float(m)
                                : __uint_as_float(m << 16);
    const float qmax = fp8 ? 448.0f : 127.0f;
    if (a < 0x1p-100f) {
        s = 0.0f;
        inv = 0.0f;                      // x * 0 -> code 0 for every element
    } else {
        s = a / qmax;                    // correctly rounded fp32 divide
        inv = qmax / a;
    }
}

}  // namespace quant_rule
}  // namespace w8a8
