// Load-time repack of an int8 weight [N, K] (out x in) into MFMA fragments
// (page "Issue 5 probe: int8 quantized DiT serve paths on the RTX 3090
// (24 GB)", "Round two" kernel-path paragraph: load, transpose-repack, apply).
//
// Layout: fragment F[nb][kb] (kb fastest) is 1024 bytes; byte 16*l + j holds
// W[16*nb + l%16][64*kb + 16*(l/16) + j], zero outside [N, K]. Lane l of a
// wavefront therefore finds its 16-byte operand of v_mfma_i32_16x16x64_i8
// at offset 16*l: one fragment is one fully coalesced dwordx4 load, and the
// same bytes read as four 256-byte runs serve v_mfma_i32_32x32x32_i8.
// Each thread moves one 16-byte unit; this runs once per layer.
//
// quant_prepack_kernel is the online (load-time) weight quantization (page
// "Online Quantization", Overview: weights and scales computed while the
// model loads, from a BF16 or FP32 checkpoint): the per-output-channel rule
// of quant.hip applied to a bf16 or fp32 weight and written straight into
// the fragment layout above, so the int8 weight never exists unpacked (or,
// for the e4m3 twin, the same with e4m3 codes and scale absmax / 448).
#include <algorithm>

#include "internal.hpp"
#include "quant_rule.hpp"

namespace w8a8 {
namespace {

__global__ __launch_bounds__(256) void prepack_kernel(const int8_t *__restrict__ wq, int N, int K,
                                                      int64_t ldw, uint4 *__restrict__ packed,
                                                      int64_t units, int kblocks, int64_t u0)
{
    const int64_t u = u0 + (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= units)
        return;
    const int lane = (int)(u & 63);
    const int64_t frag = u >> 6;
    const int kb = (int)(frag % kblocks);
    const int64_t nb = frag / kblocks;
    const int64_t n = nb * kFragN + (lane & 15);
    const int64_t k0 = (int64_t)kb * kFragK + (lane >> 4) * 16;
    unsigned w[4] = {0, 0, 0, 0};
    if (n < N) {
        const int8_t *src = wq + n * ldw + k0;
        for (int j = 0; j < 16; ++j)
            if (k0 + j < K)
                w[j >> 2] |= ((unsigned)(uint8_t)src[j]) << (8 * (j & 3));
    }
    packed[u] = make_uint4(w[0], w[1], w[2], w[3]);
}

__global__ __launch_bounds__(256) void unpack_kernel(const uint4 *__restrict__ packed, int N, int K,
                                                     int8_t *__restrict__ wq, int64_t ldw,
                                                     int64_t units, int kblocks, int64_t u0)
{
    const int64_t u = u0 + (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= units)
        return;
    const int lane = (int)(u & 63);
    const int64_t frag = u >> 6;
    const int kb = (int)(frag % kblocks);
    const int64_t nb = frag / kblocks;
    const int64_t n = nb * kFragN + (lane & 15);
    const int64_t k0 = (int64_t)kb * kFragK + (lane >> 4) * 16;
    if (n >= N)
        return;
    const uint4 v = packed[u];
    const unsigned w[4] = {v.x, v.y, v.z, v.w};
    int8_t *dst = wq + n * ldw + k0;
    for (int j = 0; j < 16; ++j)
        if (k0 + j < K)
            dst[j] = (int8_t)((w[j >> 2] >> (8 * (j & 3))) & 0xffu);
}

// One workgroup per 16-channel fragment row nb. Phase 1: the absmax of each
// of its 16 rows (wave w takes rows 4w .. 4w+3, lanes stride along K).
// Phase 2: the codes of fragment F[nb][kb] for every kb, four fragments
// per pass, thread t writing unit t % 64 of fragment t / 64; each unit is 16
// weights of one row, re-read (from L2) and quantized with the row's
// scale. Rows past N and columns past K give zero codes (load_chunk
// zero-fills past K; code(0) = 0).
template <bool F32, bool FP8>
__global__ __launch_bounds__(256) void quant_prepack_kernel(const char *__restrict__ w, int N, int K,
                                                            int64_t ldw, uint4 *__restrict__ packed,
                                                            float *__restrict__ w_scale, int kblocks,
                                                            int nb0)
{
    using namespace quant_rule;
    constexpr int VEC = Elem<F32>::VEC, B = Elem<F32>::BYTES;
    __shared__ u32 rowmax[16];
    const int nb = nb0 + (int)blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = wave * 4 + i, n = nb * 16 + r;
        u32 mx = 0;
        if (n < N) {
            const char *row = w + (int64_t)n * ldw * B;
#pragma unroll 4
            for (int64_t e = (int64_t)lane * VEC; e < K; e += 64 * VEC)
                mx = max(mx, chunk_absmax<F32>(load_chunk<F32>(row, e, K)));
        }
        mx = wave_max(mx);
        if (lane == 0)
            rowmax[r] = mx;
    }
    __syncthreads();

    const int l = lane, r = l & 15, n = nb * 16 + r;
    float sc, inv;
    scale_of(rowmax[r], F32, sc, inv, FP8);
    if (threadIdx.x < 16 && nb * 16 + (int)threadIdx.x < N)
        w_scale[nb * 16 + threadIdx.x] = sc;
    const char *row = w + (int64_t)min(n, N - 1) * ldw * B;
    for (int kb = wave; kb < kblocks; kb += 4) {
        const int64_t k0 = (int64_t)kb * 64 + (l >> 4) * 16;
        u32 q[4] = {0, 0, 0, 0};
        if (n < N) {
            if (F32) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    u32 hi;
                    chunk_codes<kF32, FP8>(load_chunk<true>(row, k0 + 4 * c, K), inv, q[c], hi);
                }
            } else {
#pragma unroll
                for (int c = 0; c < 2; ++c)
                    chunk_codes<kBF16, FP8>(load_chunk<false>(row, k0 + 8 * c, K), inv, q[2 * c],
                                            q[2 * c + 1]);
            }
        }
        packed[((int64_t)nb * kblocks + kb) * 64 + l] = make_uint4(q[0], q[1], q[2], q[3]);
    }
}

}  // namespace

hipError_t launch_quant_prepack(const void *w, bool w_f32, int64_t N, int64_t K, int64_t ldw,
                                void *packed, float *w_scale, hipStream_t stream, bool fp8)
{
    const int64_t kblocks = ceil_div(K, kFragK);
    const int64_t nblocks = ceil_div(N, kFragN);
    auto fn = w_f32 ? (fp8 ? quant_prepack_kernel<true, true> : quant_prepack_kernel<true, false>)
                    : (fp8 ? quant_prepack_kernel<false, true> : quant_prepack_kernel<false, false>);
    // A launch's workgroups times threads must fit in 32 bits: large
    // weights go in slices of fragment rows.
    for (int64_t nb0 = 0; nb0 < nblocks; nb0 += kMaxBlocksPerLaunch) {
        const int64_t blocks = std::min(nblocks - nb0, kMaxBlocksPerLaunch);
        hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(256), 0, stream,
                           reinterpret_cast<const char *>(w), (int)N, (int)K, ldw,
                           reinterpret_cast<uint4 *>(packed), w_scale, (int)kblocks, (int)nb0);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    return hipSuccess;
}

hipError_t launch_prepack(const int8_t *wq, int64_t N, int64_t K, int64_t ldw, void *packed,
                          hipStream_t stream)
{
    const int64_t kblocks = ceil_div(K, kFragK);
    const int64_t units = ceil_div(N, kFragN) * kblocks * 64;
    for (int64_t u0 = 0; u0 < units; u0 += kMaxBlocksPerLaunch * 256) {
        const int64_t blocks = std::min(ceil_div(units - u0, 256), kMaxBlocksPerLaunch);
        hipLaunchKernelGGL(prepack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, wq, (int)N,
                           (int)K, ldw, reinterpret_cast<uint4 *>(packed), units, (int)kblocks, u0);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    return hipSuccess;
}

hipError_t launch_unpack(const void *packed, int64_t N, int64_t K, int8_t *wq, int64_t ldw,
                         hipStream_t stream)
{
    const int64_t kblocks = ceil_div(K, kFragK);
    const int64_t units = ceil_div(N, kFragN) * kblocks * 64;
    for (int64_t u0 = 0; u0 < units; u0 += kMaxBlocksPerLaunch * 256) {
        const int64_t blocks = std::min(ceil_div(units - u0, 256), kMaxBlocksPerLaunch);
        hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                           reinterpret_cast<const uint4 *>(packed), (int)N, (int)K, wq, ldw, units,
                           (int)kblocks, u0);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    return hipSuccess;
}

}  // namespace w8a8
