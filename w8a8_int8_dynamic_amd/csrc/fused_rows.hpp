// Per-token quant inside a matmul launch: the producer and consumer sides of
// the one-launch path of int8_quant_scaled_mm (page "Issue 5 probe: int8
// quantized DiT serve paths on the RTX 3090 (24 GB)", "Round two"
// kernel-path paragraph: the per-token quant that precedes the scaled
// matmul, here run by the matmul's own workgroups).
//
// Protocol. Producer workgroup w quantizes rows [w*rpw, (w+1)*rpw) of x
// (rpw = rows_per_wg) with the rule of int8_quant_per_token and then stores
// the launch's epoch (a per-device launch number, never 0) in flag[w]. A
// consumer accepts the rows of its tile once every producer of those rows
// shows the current epoch, so nothing is ever reset. Flags are plain
// coherent stores and loads, one word per producer: no read-modify-write on
// a shared word, which would serialize at the memory side. The wait is
// bounded; past the bound a workgroup quantizes the rows it needs itself,
// writing the same bytes their producers write, so no wave can spin forever
// and launches that overlap on one device stay correct. The epoch is fixed
// when the launch is made, so a captured graph would replay it; the host
// therefore never uses this path on a stream under capture.
//
// Coherence. Codes and scales are written with agent-scope (relaxed atomic)
// stores, coherent across the XCDs once complete, so no write-back of the
// producer's L2 is needed before the flag goes up. No cache of a consumer's
// CU or XCD can hold an older copy of the rows: caches start each launch
// clean, no workgroup reads a tile's rows before its wait, and the host
// takes this path only when the codes and scales buffers are aligned so
// that no cache line holds rows of two row tiles (kFusedAlign).
#pragma once

#include <type_traits>

#include "internal.hpp"
#include "quant_rule.hpp"

namespace w8a8 {
namespace fused {

using quant_rule::u32;

// Producer flags. Every translation unit that includes this header has its
// own array, used only by its own kernels.
constexpr int kMaxProducers = 16384;
static __device__ unsigned g_flag[kMaxProducers];

// Default bound on the polls for a tile's rows (each ~1 us; a few ms in
// all): far beyond any real wait. A launch carries its bound in
// MmArgs::wait_limit, which the host can lower (0 makes every workgroup take
// its own-rows path at once, which tests use).
constexpr unsigned kDefaultWaitLimit = 1u << 12;

// Alignment (bytes) that the codes and scales buffers need for the
// one-launch path: at least a cache line (128 bytes on gfx950), with margin.
constexpr uintptr_t kFusedAlign = 256;

// Short rows (K <= 64 * 8 * CPL): one wavefront per row, CPL 16-byte chunks
// per lane, 8 / CPL rows per wavefront in flight (all their loads issued
// before the first reduction); the reduction stays inside the wavefront, so
// there is no barrier. Wave w takes row groups w, w + NW, ... of [ra, rb).
template <int THREADS, int CPL, int E, bool FP8>
__device__ __forceinline__ void quantize_rows_by_wave(const MmArgs &a, int ra, int rb)
{
    using namespace quant_rule;
    constexpr int NW = THREADS / 64, R = 8 / CPL;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int g = ra + wave * R; g < rb; g += NW * R) {
        uint4 v[R][CPL];
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const uint16_t *xrow = a.x + (int64_t)min(g + i, rb - 1) * a.ldx;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                // K is a multiple of 16: a chunk that starts inside the row is whole.
                const int e = (c * 64 + lane) * 8;
                v[i][c] = e < a.K ? *reinterpret_cast<const uint4 *>(xrow + e) : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < R; ++i) {
            if (g + i >= rb)
                break;
            u32 mx = 0;
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                mx = max(mx, chunk_absmax<E>(v[i][c]));
            mx = wave_max(mx);
            float sc, inv;
            scale_of(mx, E, sc, inv, FP8);
            int8_t *qrow = const_cast<int8_t *>(a.xq) + (int64_t)(g + i) * a.ldq;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int e = (c * 64 + lane) * 8;
                if (e < a.K) {
                    u32 lo, hi;
                    chunk_codes<E, FP8>(v[i][c], inv, lo, hi);
                    __hip_atomic_store(reinterpret_cast<uint64_t *>(qrow + e), (uint64_t)hi << 32 | lo,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            if (lane == 0)
                __hip_atomic_store(const_cast<float *>(a.xs) + g + i, sc, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Rows [ra, rb) of x (16-bit floats of kind E, bf16 or fp16, [M, ldx]) into
// xq / xs by the THREADS threads of a workgroup, with the rule of
// int8_quant_per_token. Rows of up to 4096
// elements go one per wavefront (quantize_rows_by_wave). Longer rows use the
// whole workgroup: a row of up to 8 * 8 * THREADS elements is held in
// registers (one read of x; two such rows at a time when they fit); longer
// still take an absmax pass and a codes pass that re-reads the row from L2.
// red: 2 * THREADS / 64 words of LDS. Every thread of the workgroup must
// call this (it may hold barriers). FP8: e4m3 codes and absmax / 448 scales.
template <int THREADS, int E, bool FP8 = false>
__device__ __forceinline__ void quantize_rows(const MmArgs &a, int ra, int rb, u32 *red)
{
    using namespace quant_rule;
    if (a.K <= 64 * 8) {
        quantize_rows_by_wave<THREADS, 1, E, FP8>(a, ra, rb);
        return;
    }
    if (a.K <= 64 * 8 * 2) {
        quantize_rows_by_wave<THREADS, 2, E, FP8>(a, ra, rb);
        return;
    }
    if (a.K <= 64 * 8 * 4) {
        quantize_rows_by_wave<THREADS, 4, E, FP8>(a, ra, rb);
        return;
    }
    if (a.K <= 64 * 8 * 8 && rb - ra > THREADS / 64) {
        quantize_rows_by_wave<THREADS, 8, E, FP8>(a, ra, rb);
        return;
    }
    constexpr int NW = THREADS / 64;
    constexpr int QCH = 8;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    // K is a multiple of 16, so every 8-code chunk is whole.
    auto put_codes = [&](int8_t *qrow, int e, u32 lo, u32 hi) __attribute__((always_inline)) {
        __hip_atomic_store(reinterpret_cast<uint64_t *>(qrow + e), (uint64_t)hi << 32 | lo,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    auto put_scale = [&](int r, float sc) __attribute__((always_inline)) {
        if (threadIdx.x == 0)
            __hip_atomic_store(const_cast<float *>(a.xs) + r, sc, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    };
    // One row group (1 or 2 rows) held in registers: every load of the group
    // is issued before the reductions.
    auto rows_in_regs = [&](auto nr_c, int r) __attribute__((always_inline)) {
        constexpr int NR = decltype(nr_c)::value;
        constexpr int CH = QCH / NR;
        uint4 v[NR][CH];
        u32 mx[NR];
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            const char *xrow = reinterpret_cast<const char *>(a.x + (int64_t)(r + k) * a.ldx);
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int e = (c * THREADS + (int)threadIdx.x) * 8;
                v[k][c] = e < a.K ? load_chunk<E>(xrow, e, a.K) : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            mx[k] = 0;
#pragma unroll
            for (int c = 0; c < CH; ++c)
                mx[k] = max(mx[k], chunk_absmax<E>(v[k][c]));
            mx[k] = wave_max(mx[k]);
            if (lane == 0)
                red[k * NW + wave] = mx[k];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < NR; ++k)
#pragma unroll
            for (int w = 0; w < NW; ++w)
                mx[k] = max(mx[k], red[k * NW + w]);
        __syncthreads();                               // red is rewritten by the next group
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            float sc, inv;
            scale_of(mx[k], E, sc, inv, FP8);
            int8_t *qrow = const_cast<int8_t *>(a.xq) + (int64_t)(r + k) * a.ldq;
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int e = (c * THREADS + (int)threadIdx.x) * 8;
                if (e < a.K) {
                    u32 lo, hi;
                    chunk_codes<E, FP8>(v[k][c], inv, lo, hi);
                    put_codes(qrow, e, lo, hi);
                }
            }
            put_scale(r + k, sc);
        }
    };
    auto row_looped = [&](int r) __attribute__((always_inline)) {
        const char *xrow = reinterpret_cast<const char *>(a.x + (int64_t)r * a.ldx);
        int8_t *qrow = const_cast<int8_t *>(a.xq) + (int64_t)r * a.ldq;
        u32 mx = 0;
        for (int e = (int)threadIdx.x * 8; e < a.K; e += THREADS * 8)
            mx = max(mx, chunk_absmax<E>(load_chunk<E>(xrow, e, a.K)));
        mx = wave_max(mx);
        if (lane == 0)
            red[wave] = mx;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < NW; ++w)
            mx = max(mx, red[w]);
        __syncthreads();
        float sc, inv;
        scale_of(mx, E, sc, inv, FP8);
        for (int e = (int)threadIdx.x * 8; e < a.K; e += THREADS * 8) {
            u32 lo, hi;
            chunk_codes<E, FP8>(load_chunk<E>(xrow, e, a.K), inv, lo, hi);
            put_codes(qrow, e, lo, hi);
        }
        put_scale(r, sc);
    };
    int r = ra;
    if (a.K <= (QCH / 2) * 8 * THREADS)
        for (; r + 2 <= rb; r += 2)
            rows_in_regs(std::integral_constant<int, 2>{}, r);
    for (; r < rb; ++r) {
        if (a.K <= QCH * 8 * THREADS)
            rows_in_regs(std::integral_constant<int, 1>{}, r);
        else
            row_looped(r);
    }
}

// Producer: once every thread's stores have completed, raise this
// workgroup's flag (when it had rows to quantize). Every thread calls this.
__device__ __forceinline__ void publish(const MmArgs &a, bool had_rows)
{
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0 && had_rows)
        __hip_atomic_store(&g_flag[blockIdx.x], a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Consumer: wave 0 polls the flags of producers p0 .. p0+count-1 until all
// show this launch's epoch, or the bound runs out. Returns, in every thread,
// true when it ran out (the caller then quantizes the rows itself).
// decision: one word of LDS that no other phase writes meanwhile. Every
// thread calls this.
__device__ __forceinline__ bool wait_producers(const MmArgs &a, int p0, int count, u32 *decision)
{
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const unsigned limit = a.wait_limit;
        unsigned it = 0;
        for (; it < limit; ++it) {
            bool ready = true;
            for (int i = lane; i < count; i += 64)
                ready &= __hip_atomic_load(&g_flag[p0 + i], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT) == a.epoch;
            if (__all(ready))
                break;
            __builtin_amdgcn_s_sleep(2);
        }
        if (lane == 0)
            decision[0] = it == limit;
    }
    __syncthreads();
    return decision[0] != 0;
}

}  // namespace fused
}  // namespace w8a8
