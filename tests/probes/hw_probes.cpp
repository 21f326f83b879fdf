// Measurement probes of the MI355X memory paths that bound the matmul and
// the decode kernels (not part of the library; built by
// __graft_entry__.build() into tests/probes/hw_probes, run by
// `python bench.py --hw-probes`). Each prints one line of JSON.
//
//   l2_stream   read bandwidth per CU from the XCD's L2 (a 1 MiB window that
//               every workgroup re-reads, so after the first pass every
//               load hits in L2), for 4 or 16 waves per CU and 1-16 loads in
//               flight per wave;
//   l1_stream   the same from a 16 KiB window per workgroup (L1 hits: the
//               ceiling of the path from the vector cache to registers);
//   lds_read    LDS read bandwidth per CU (ds_read_b128), 4 or 8 waves;
//   hbm_floor   back-to-back launches that each read S bytes once from HBM
//               (rotating over buffers larger than the last-level cache):
//               the time one streaming kernel of that size takes.
//   mfma_only   the fused-QKV matmul's MFMA work with no memory traffic: 256
//               workgroups of 4 waves, each wave 768 v_mfma_i32_32x32x32_i8
//               on 12 accumulators (and 16 times that), back to back, with
//               the shader clock read inside the kernel.
//
// Every global index is taken modulo a power-of-two window inside its
// buffer and every LDS index modulo the array, so no access leaves its
// allocation. Loaded values are summed (not xor-ed: repeated addresses
// would cancel) and the sum is stored only under a condition the data never
// meets, which keeps the loads from being optimized away.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

typedef int v4i __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                   \
    do {                                                                           \
        hipError_t e_ = (x);                                                       \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "%s:%d %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
            exit(1);                                                               \
        }                                                                          \
    } while (0)

// Workgroup w reads iters * U wave-loads of 1 KiB per wave from its own
// window start (w * wg_stride16, in 16-byte units) within the region.
template <int U>
__global__ __launch_bounds__(256) void stream_kernel(const v4i *buf, unsigned long mask16, int iters,
                                                     unsigned long wg_stride16, int stride, int *out)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const unsigned long base = (unsigned long)blockIdx.x * wg_stride16;
    v4i acc = {0, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
        v4i v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = buf[(base + (unsigned long)(it * U + u) * stride + wave * 64 + lane) & mask16];
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc += v[u];
    }
    if (acc[0] == 0x7fffffff && acc[1] == 12345)
        out[blockIdx.x & 1023] = acc[2];
}

template <int NT>
__global__ __launch_bounds__(NT) void lds_kernel(int iters, int stride, int *out)
{
    __shared__ v4i buf[4096];
    for (int i = threadIdx.x; i < 4096; i += NT)
        buf[i] = v4i{i, i + 1, i + 2, i + 3};
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v4i acc = {0, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
            acc += buf[((it * 8 + u) * stride + wave * 64 + lane) & 4095];
    }
    if (acc[0] == 0x7fffffff && acc[1] == 12345)
        out[blockIdx.x & 1023] = acc[2];
}

__global__ __launch_bounds__(256) void floor_kernel(const v4i *buf, size_t n16, int *out)
{
    v4i acc = {0, 0, 0, 0};
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        v4i v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            acc += v[u];
    }
    for (; i < n16; i += stride)
        acc += buf[i];
    if (acc[0] == 0x7fffffff && acc[1] == 12345)
        out[blockIdx.x & 1023] = acc[2];
}

typedef int v16i __attribute__((ext_vector_type(16)));

// Each wave runs `steps` rounds of 12 independent MFMAs (one per
// accumulator, as a 128 x 192 tile's wave does per 32-deep k-step). Thread 0
// of workgroup 0 writes s_memtime and s_memrealtime at its start and end to
// clk[0..3].
__global__ __launch_bounds__(256) void mfma_kernel(int steps, int *out, long long *clk)
{
    const long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    const int lane = threadIdx.x & 63;
    v4i a = {lane, lane * 3, lane * 5, lane * 7};
    v4i b = {lane * 11, lane * 13, lane ^ 17, lane ^ 19};
    v16i acc[12];
#pragma unroll
    for (int i = 0; i < 12; ++i)
        acc[i] = v16i{};
    for (int s = 0; s < steps; ++s) {
#pragma unroll
        for (int i = 0; i < 12; ++i)
            acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[i], 0, 0, 0);
        a += 1;
    }
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 12; ++i)
        sum += acc[i][0] + acc[i][15];
    if (sum == 0x7fffffff)
        out[blockIdx.x & 1023] = sum;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        clk[0] = t0;
        clk[1] = r0;
        clk[2] = __builtin_amdgcn_s_memtime();
        clk[3] = __builtin_amdgcn_s_memrealtime();
    }
}

template <class F>
static double time_us(F launch, int reps)
{
    hipEvent_t a, b;
    CHECK(hipEventCreate(&a));
    CHECK(hipEventCreate(&b));
    for (int w = 0; w < 3; ++w)
        launch(w);
    CHECK(hipEventRecord(a));
    for (int r = 0; r < reps; ++r)
        launch(r);
    CHECK(hipEventRecord(b));
    CHECK(hipEventSynchronize(b));
    float ms = 0;
    CHECK(hipEventElapsedTime(&ms, a, b));
    CHECK(hipEventDestroy(a));
    CHECK(hipEventDestroy(b));
    return ms * 1e3 / reps;
}

int main()
{
    int cus = 0;
    CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
    int *out;
    CHECK(hipMalloc(&out, 1024 * sizeof(int)));
    const size_t l2_bytes = 1 << 20, l1_window = 16 << 10;
    v4i *buf;
    CHECK(hipMalloc(&buf, l2_bytes));
    CHECK(hipMemset(buf, 1, l2_bytes));
    auto stream_case = [&](const char *name, size_t region, size_t wg_stride, int wgs, int u) {
        const int loads = 2048;                   // wave-loads of 1 KiB per wave
        const int iters = loads / u;
        auto launch = [&](int) {
            const unsigned long mask = region / 16 - 1;
            switch (u) {
            case 1: hipLaunchKernelGGL(stream_kernel<1>, dim3(wgs), dim3(256), 0, 0, buf, mask, iters, wg_stride / 16, 256, out); break;
            case 4: hipLaunchKernelGGL(stream_kernel<4>, dim3(wgs), dim3(256), 0, 0, buf, mask, iters, wg_stride / 16, 256, out); break;
            case 8: hipLaunchKernelGGL(stream_kernel<8>, dim3(wgs), dim3(256), 0, 0, buf, mask, iters, wg_stride / 16, 256, out); break;
            default: hipLaunchKernelGGL(stream_kernel<16>, dim3(wgs), dim3(256), 0, 0, buf, mask, iters, wg_stride / 16, 256, out); break;
            }
        };
        const double us = time_us(launch, 10);
        const double bytes = (double)wgs * 4 * loads * 1024;
        printf("{\"probe\": \"%s\", \"waves_per_cu\": %d, \"loads_in_flight_per_wave\": %d, "
               "\"bytes_per_ns_per_cu\": %.1f, \"tb_per_s\": %.2f}\n",
               name, 4 * wgs / cus, u, bytes / (us * 1e3) / cus, bytes / (us * 1e-6) / 1e12);
    };
    for (int wgs : {cus, 4 * cus})
        for (int u : {1, 4, 8, 16})
            stream_case("l2_stream", l2_bytes, 64 << 10, wgs, u);
    for (int wgs : {cus, 4 * cus})
        stream_case("l1_stream", l1_window, l1_window, wgs, 8);
    // (l1_stream: every workgroup re-reads the same 16 KiB window, which its
    // CU's vector cache holds)
    for (int nt : {256, 512}) {
        const int iters = 4096;
        auto launch = [&](int) {
            if (nt == 256)
                hipLaunchKernelGGL(lds_kernel<256>, dim3(cus), dim3(256), 0, 0, iters, 256, out);
            else
                hipLaunchKernelGGL(lds_kernel<512>, dim3(cus), dim3(512), 0, 0, iters, 512, out);
        };
        const double us = time_us(launch, 10);
        const double bytes = (double)cus * nt * 16 * 8 * iters;
        printf("{\"probe\": \"lds_read\", \"waves_per_cu\": %d, \"bytes_per_ns_per_cu\": %.1f}\n",
               nt / 64, bytes / (us * 1e3) / cus);
    }
    CHECK(hipFree(buf));
    const int copies = 12;
    for (size_t mb : {17, 38, 50}) {
        const size_t bytes = mb * 1000000 / 1024 * 1024;
        std::vector<v4i *> b(copies);
        for (auto &p : b) {
            CHECK(hipMalloc(&p, bytes));
            CHECK(hipMemset(p, 1, bytes));
        }
        for (int grid : {cus, 2 * cus, 8 * cus}) {
            auto launch = [&](int i) {
                hipLaunchKernelGGL(floor_kernel, dim3(grid), dim3(256), 0, 0, b[i % copies], bytes / 16, out);
            };
            const double us = time_us(launch, 48);
            printf("{\"probe\": \"hbm_floor\", \"mb\": %zu, \"workgroups\": %d, \"us_per_launch\": %.2f, "
                   "\"gb_per_s\": %.0f}\n", mb, grid, us, bytes / us / 1e3);
        }
        for (auto &p : b)
            CHECK(hipFree(p));
    }
    long long *clk;
    CHECK(hipMalloc(&clk, 4 * sizeof(long long)));
    for (int mult : {1, 16}) {
        const int steps = 64 * mult;              // 12 * 64 = 768 MFMAs per wave at 1x
        auto launch = [&](int) {
            hipLaunchKernelGGL(mfma_kernel, dim3(cus), dim3(256), 0, 0, steps, out, clk);
        };
        const double us = time_us(launch, 100);
        long long c[4];
        CHECK(hipMemcpy(c, clk, sizeof(c), hipMemcpyDeviceToHost));
        const double ops = (double)cus * 4 * steps * 12 * (2.0 * 32 * 32 * 32);
        printf("{\"probe\": \"mfma_only\", \"workgroups\": %d, \"mfma_per_wave\": %d, "
               "\"us_per_launch\": %.2f, \"pops\": %.3f, \"sclk_ghz\": %.3f}\n",
               cus, steps * 12, us, ops / (us * 1e-6) / 1e15,
               (double)(c[2] - c[0]) / ((double)(c[3] - c[1]) * 10.0));
    }
    CHECK(hipFree(clk));
    CHECK(hipFree(out));
    return 0;
}
