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
#include "internal.hpp"

namespace w8a8 {
namespace {

__global__ __launch_bounds__(256) void prepack_kernel(const int8_t *__restrict__ wq, int N, int K,
                                                      int64_t ldw, uint4 *__restrict__ packed,
                                                      int64_t units, int kblocks)
{
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
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
                                                     int64_t units, int kblocks)
{
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
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

}  // namespace

hipError_t launch_prepack(const int8_t *wq, int64_t N, int64_t K, int64_t ldw, void *packed,
                          hipStream_t stream)
{
    const int64_t kblocks = ceil_div(K, kFragK);
    const int64_t units = ceil_div(N, kFragN) * kblocks * 64;
    hipLaunchKernelGGL(prepack_kernel, dim3((unsigned)ceil_div(units, 256)), dim3(256), 0, stream,
                       wq, (int)N, (int)K, ldw, reinterpret_cast<uint4 *>(packed), units,
                       (int)kblocks);
    return hipGetLastError();
}

hipError_t launch_unpack(const void *packed, int64_t N, int64_t K, int8_t *wq, int64_t ldw,
                         hipStream_t stream)
{
    const int64_t kblocks = ceil_div(K, kFragK);
    const int64_t units = ceil_div(N, kFragN) * kblocks * 64;
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)ceil_div(units, 256)), dim3(256), 0, stream,
                       reinterpret_cast<const uint4 *>(packed), (int)N, (int)K, wq, ldw, units,
                       (int)kblocks);
    return hipGetLastError();
}

}  // namespace w8a8
