// Small-M int8 x int8 -> int32 matmul with the fused scale epilogue, for
// gfx950: the decode-shaped case, a handful of token rows against a large
// weight. Same results as the main kernel (scaled_mm.hip), bit for bit.
//
// With few token rows each weight byte meets only a few tokens, so the
// matmul is bound by streaming the weight out of HBM (page "INT8 Quant for
// Dual-Max Recipe", the soak-run analysis: decode is bandwidth-bound, and
// 8-bit weights move the same bytes whatever their format). The main
// kernel's tiles (64 or more channels and the whole of K per workgroup)
// leave most CUs without work when N is a few thousand, so this kernel
// spreads the weight stream over as many wavefronts as it can:
//   - A workgroup owns 16*FN output channels and 16*FM token rows. Its WK
//     wavefronts split K: wave w takes k-blocks w, w+WK, w+2WK, ..., so at
//     any moment the workgroup reads one contiguous run of each weight
//     column.
//   - A k-block is one v_mfma_i32_16x16x64_i8 per (row block, fragment).
//     The prepacked 1 KB weight fragment is the MFMA A operand exactly as
//     stored (lane l: the 16 bytes at 16*l), one coalesced load that skips
//     the caches' retention (every weight byte is read once). The token rows
//     are the B operand (lane l: row l%16, the 16 bytes at 16*(l/16) of the
//     k-block); they are small and every workgroup reads them, from L2.
//     Accumulator register r of lane l is channel 4*(l/16)+r, token l%16.
//   - U k-blocks form a load group: all its loads are issued before its
//     first MFMA, so each wave keeps U fragments in flight.
//   - The WK partial sums meet in LDS and wave 0 applies the epilogue in the
//     main kernel's fixed operation order.
//   - Fused per-token quant (int8_quant_scaled_mm), for tiles of one or
//     two rows that fit four 16-byte chunks per thread: every workgroup
//     quantizes its own tile's rows into LDS (the rows are small and sit in
//     L2, so repeating the work is cheap at this size) with the rule of
//     int8_quant_per_token, and reads its token operands from there; nothing
//     waits on another workgroup.
//     The first load group of weights goes out before the rows are read, so
//     the quant's latency hides behind the weight stream. The workgroup of
//     the first channel fragment also writes the codes and scales out.
// Ragged tails as in the main kernel: token rows past M read row M-1,
// fragments past N read the last fragment, token chunks past K read the last
// chunk (which meets zero weights); stores are masked.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "internal.hpp"
#include "quant_rule.hpp"

namespace w8a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Fused quant: every workgroup converts its tile's rows itself, about ten
// VALU operations per element, which only pays below a few rows: tiles of
// at most kQuantRows rows, and at most kQuantSlots 16-byte chunks of x per
// thread (held in registers between the absmax and the codes).
constexpr int kQuantRows = 2;
constexpr int kQuantSlots = 4;

// FM blocks of 16 token rows and FN fragments of 16 channels per
// workgroup; WK wavefronts split K; U k-blocks per load group.
template <int FM_, int FN_, int WK_, int U_>
struct Skinny {
    static constexpr int FM = FM_, FN = FN_, WK = WK_, U = U_;
    static constexpr int BM = 16 * FM, BN = 16 * FN, THREADS = 64 * WK;
    static_assert(WK >= 2 && WK <= 16, "two to sixteen wavefronts");
    static_assert(U * (FM + FN) * 4 <= 128, "operand registers");
};

// Rows m0 .. m0+rows-1 of x quantized by one workgroup of THREADS threads
// with the rule of int8_quant_per_token: codes into tok (row r at r*pitch),
// scales into rowscale; with `writer` also codes and scales to xq / xs. The
// rows are read once: thread t holds chunk c of row r (elements
// (c*THREADS + t)*8 ..+8) in slot r*cpr + c, at most kQuantSlots of them.
// Every thread calls this (it holds barriers).
template <int THREADS, int E, bool FP8>
__device__ __forceinline__ void quantize_tile(const MmArgs &a, int m0, int rows, int pitch,
                                              bool writer, int8_t *tok, quant_rule::u32 *rowmax,
                                              float *rowscale)
{
    using namespace quant_rule;
    const int lane = threadIdx.x & 63;
    const int cpr = (a.K / 8 + THREADS - 1) / THREADS;
    const int slots = rows * cpr;
    uint4 v[kQuantSlots];
#pragma unroll
    for (int s = 0; s < kQuantSlots; ++s) {
        if (s < slots) {
            const int r = s / cpr, e = ((s - r * cpr) * THREADS + (int)threadIdx.x) * 8;
            // K is a multiple of 16: a chunk that starts inside the row is whole.
            const uint16_t *xrow = a.x + (int64_t)(m0 + r) * a.ldx;
            v[s] = e < a.K ? *reinterpret_cast<const uint4 *>(xrow + e) : make_uint4(0, 0, 0, 0);
        }
    }
    if ((int)threadIdx.x < rows)
        rowmax[threadIdx.x] = 0;
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kQuantSlots; ++s) {
        if (s < slots) {
            const u32 m = wave_max(chunk_absmax<E>(v[s]));
            if (lane == 0)
                atomicMax(&rowmax[s / cpr], m);
        }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kQuantSlots; ++s) {
        if (s < slots) {
            const int r = s / cpr, e = ((s - r * cpr) * THREADS + (int)threadIdx.x) * 8;
            float sc, inv;
            scale_of(rowmax[r], E, sc, inv, FP8);
            if (e < a.K) {
                u32 lo, hi;
                chunk_codes<E, FP8>(v[s], inv, lo, hi);
                *reinterpret_cast<v2u *>(tok + r * pitch + e) = v2u{lo, hi};
                if (writer)
                    *reinterpret_cast<v2u *>(const_cast<int8_t *>(a.xq) + (int64_t)(m0 + r) * a.ldq + e) =
                        v2u{lo, hi};
            }
        }
    }
    if ((int)threadIdx.x < rows) {
        float sc, inv;
        scale_of(rowmax[threadIdx.x], E, sc, inv, FP8);
        rowscale[threadIdx.x] = sc;
        if (writer)
            const_cast<float *>(a.xs)[m0 + threadIdx.x] = sc;
    }
    __syncthreads();
}

// At least 16 wavefronts per CU (128 registers each): the kernel lives on
// the loads it keeps in flight, so occupancy counts more than ILP.
// FP8: the e4m3 twin. Two k-blocks (the 1 KB fragments of k-blocks kb and
// the next of this wave's) make one v_mfma_scale_f32_16x16x128_f8f6f4 on the
// concatenated 16-byte halves of both operands (unit block scales), fp32
// accumulators; a lone last k-block pairs with zero weights.
template <class S, int OUT, bool FUSED, bool FP8 = false>
__global__ __launch_bounds__(S::THREADS, 1024 / S::THREADS) void skinny_mm_kernel(const MmArgs a)
{
    using Acc = std::conditional_t<FP8, f32x4, v4i>;
    constexpr bool OUT_I32 = OUT == kOutI32, OUT_F16 = OUT == kOutF16;
    // The fused form reads x in the output's 16-bit type (bf16 for int32).
    constexpr int IN = OUT_F16 ? kElemF16 : kElemBF16;
    // Waves 1 .. WK-1 hand their partial sums to wave 0.
    __shared__ v4i part[S::WK - 1][S::FM * S::FN][64];
    // Fused quant: the tile's codes (rows of K + 16 bytes, sized at launch),
    // row maxima (bit patterns of |x|) and scales.
    extern __shared__ __attribute__((aligned(16))) int8_t tok[];
    __shared__ quant_rule::u32 rowmax[FUSED ? S::BM : 1];
    __shared__ float rowscale[FUSED ? S::BM : 1];

    const int lane = threadIdx.x & 63;
    const int wk = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tiles_m = (a.M + S::BM - 1) / S::BM;
    const int tiles_n = (a.nblocks + S::FN - 1) / S::FN;
    // Split of K (int8 only): the nsplit workgroups of a tile are neighbours
    // in the logical order, each with its own run of kbs k-blocks.
    const int nsplit = !FP8 && a.ksplit > 1 ? a.ksplit : 1;
    // The row tiles of one weight column run on one XCD, next to each other.
    const int tl = xcd_remap(blockIdx.x, tiles_m * tiles_n * nsplit);
    const int t = tl / nsplit, ks = tl - t * nsplit;
    const int m0 = (t % tiles_m) * S::BM, nb0 = (t / tiles_m) * S::FN;
    const int KB = a.kblocks;
    const int kbeg = nsplit > 1 ? min(ks * a.kbs, KB) : 0;
    const int kend = nsplit > 1 ? min(kbeg + a.kbs, KB) : KB;
    const int klast = a.K - 16;

    const v4i *wsrc[S::FN];
#pragma unroll
    for (int j = 0; j < S::FN; ++j)
        wsrc[j] = reinterpret_cast<const v4i *>(a.wp) + (int64_t)min(nb0 + j, a.nblocks - 1) * KB * 64 +
                  lane;
    // Token operand rows: from xq, or from the LDS codes when fused.
    const int rows = min(S::BM, a.M - m0);
    const int pitch = a.K + 16;
    const int8_t *tsrc[S::FM];
#pragma unroll
    for (int f = 0; f < S::FM; ++f) {
        const int r = min(16 * f + (lane & 15), rows - 1);
        tsrc[f] = FUSED ? tok + r * pitch : a.xq + (int64_t)(m0 + r) * a.ldq;
    }
    const int kc = 16 * (lane >> 4);

    Acc acc[S::FM][S::FN];
#pragma unroll
    for (int f = 0; f < S::FM; ++f)
#pragma unroll
        for (int j = 0; j < S::FN; ++j)
            acc[f][j] = Acc{};

    auto wload = [&](int kb, v4i (&w)[S::FN]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < S::FN; ++j)
            w[j] = __builtin_nontemporal_load(wsrc[j] + (int64_t)kb * 64);
    };
    auto tload = [&](int kb, v4i (&x)[S::FM]) __attribute__((always_inline)) {
#pragma unroll
        for (int f = 0; f < S::FM; ++f)
            x[f] = *reinterpret_cast<const v4i *>(tsrc[f] + min(kb * 64 + kc, klast));
    };
    auto block = [&](int kb, v4i (&w)[S::FN], v4i (&x)[S::FM]) __attribute__((always_inline)) {
        wload(kb, w);
        tload(kb, x);
    };
    auto mma = [&](const v4i (&w)[S::FN], const v4i (&x)[S::FM]) __attribute__((always_inline)) {
#pragma unroll
        for (int f = 0; f < S::FM; ++f)
#pragma unroll
            for (int j = 0; j < S::FN; ++j) {
                if constexpr (!FP8)
                    acc[f][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[j], x[f], acc[f][j], 0, 0, 0);
            }
    };
    auto mma2 = [&](const v4i (&w0)[S::FN], const v4i (&x0)[S::FM], const v4i (&w1)[S::FN],
                    const v4i (&x1)[S::FM]) __attribute__((always_inline)) {
#pragma unroll
        for (int f = 0; f < S::FM; ++f)
#pragma unroll
            for (int j = 0; j < S::FN; ++j) {
                if constexpr (FP8) {
                    const v8i ww = __builtin_shufflevector(w0[j], w1[j], 0, 1, 2, 3, 4, 5, 6, 7);
                    const v8i xx = __builtin_shufflevector(x0[f], x1[f], 0, 1, 2, 3, 4, 5, 6, 7);
                    acc[f][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ww, xx, acc[f][j], 0, 0,
                                                                               0, 127, 0, 127);
                }
            }
    };
    // The MFMAs of a load group's first n k-blocks (n is wave-uniform).
    auto mma_group = [&](const v4i (&w)[S::U][S::FN], const v4i (&x)[S::U][S::FM], int n)
                         __attribute__((always_inline)) {
        if constexpr (FP8) {
            static_assert(S::U % 2 == 0, "k-blocks go to the fp8 MFMA in pairs");
            const v4i zero[S::FN] = {};
#pragma unroll
            for (int u = 0; u < S::U; u += 2) {
                if (u + 1 < n)
                    mma2(w[u], x[u], w[u + 1], x[u + 1]);
                else if (u < n)
                    mma2(w[u], x[u], zero, x[u]);
            }
        } else {
#pragma unroll
            for (int u = 0; u < S::U; ++u)
                if (u < n)
                    mma(w[u], x[u]);
        }
    };

    // This wave's k-blocks: wk, wk+WK, ... (mine of them). Full load groups,
    // then one partial group; within a group every load is issued before the
    // first MFMA waits on any of them. Each workgroup starts its walk at its
    // own offset (rot), which spreads the workgroups of an XCD over the
    // token bytes.
    // The split's ticket is taken as the workgroup starts (by wave 0, which
    // finishes the tile), so its round trip overlaps the K loop.
    unsigned ticket0 = 0;
    if (nsplit > 1 && wk == 0 && lane == 0)
        ticket0 = __hip_atomic_fetch_add(a.split_count + 2 * t, 1u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    const int span = kend - kbeg;
    const int mine = wk < span ? (span - 1 - wk) / S::WK + 1 : 0;
    const int rot = mine > 0 ? t % mine : 0;
    auto kb_of = [&](int i) __attribute__((always_inline)) {
        i += rot;
        return kbeg + wk + (i >= mine ? i - mine : i) * S::WK;
    };
    int g = 0;
    if (FUSED) {
        // The first load group's weights go out before the token rows exist
        // (always issued, clamped into the weight, so that no branch joins a
        // path without them; unused when this wave has fewer k-blocks).
        const bool pre = mine >= S::U;
        v4i w[S::U][S::FN];
#pragma unroll
        for (int u = 0; u < S::U; ++u)
            wload(min(kb_of(u), KB - 1), w[u]);
        quantize_tile<S::THREADS, IN, FP8>(a, m0, rows, pitch, nb0 == 0 && ks == 0, tok, rowmax,
                                           rowscale);
        if (pre) {
            v4i x[S::U][S::FM];
#pragma unroll
            for (int u = 0; u < S::U; ++u)
                tload(kb_of(u), x[u]);
            __builtin_amdgcn_sched_barrier(0);
            mma_group(w, x, S::U);
            __builtin_amdgcn_sched_barrier(0);
            g = S::U;
        }
    }
#pragma unroll 1
    for (; g + S::U <= mine; g += S::U) {
        v4i w[S::U][S::FN], x[S::U][S::FM];
#pragma unroll
        for (int u = 0; u < S::U; ++u)
            block(kb_of(g + u), w[u], x[u]);
        __builtin_amdgcn_sched_barrier(0);
        mma_group(w, x, S::U);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (g < mine) {
        v4i w[S::U][S::FN], x[S::U][S::FM];
#pragma unroll
        for (int u = 0; u < S::U; ++u)
            if (g + u < mine)
                block(kb_of(g + u), w[u], x[u]);
        __builtin_amdgcn_sched_barrier(0);
        mma_group(w, x, mine - g);
    }

    if (wk > 0) {
#pragma unroll
        for (int f = 0; f < S::FM; ++f)
#pragma unroll
            for (int j = 0; j < S::FN; ++j)
                part[wk - 1][f * S::FN + j][lane] = __builtin_bit_cast(v4i, acc[f][j]);
    }
    __syncthreads();
    if (wk != 0)
        return;
    // One wave's partials at a time (all of them at once would not fit in
    // registers).
#pragma unroll 1
    for (int w = 0; w < S::WK - 1; ++w)
#pragma unroll
        for (int f = 0; f < S::FM; ++f)
#pragma unroll
            for (int j = 0; j < S::FN; ++j)
                acc[f][j] += __builtin_bit_cast(Acc, part[w][f * S::FN + j][lane]);

    if (nsplit > 1) {
        // The tile's nsplit workgroups meet through the workspace: each
        // took a ticket from the tile's arrival word as it started (in start
        // order, so the last ticket may go to a workgroup that finishes
        // early; it then waits for the others); all but the last
        // write their int32 partial sums (write-through stores, coherent
        // across the XCDs once complete) and then count themselves in the
        // tile's done word. The last waits until done shows the others,
        // reads their partial sums with coherent loads, adds them (exact in
        // int32, whatever the order), finishes the tile and sets both words
        // back to 0. It only ever waits for workgroups that hold a ticket,
        // so are running and never wait themselves: the wait always ends.
        unsigned *words = a.split_count + 2 * t;     // [0] arrivals, [1] done
        const unsigned ticket = (unsigned)__builtin_amdgcn_readfirstlane((int)ticket0);
        uint64_t *part_all = reinterpret_cast<uint64_t *>(a.split_part) +
                             (int64_t)t * nsplit * (S::FM * S::FN * 64 * 2);
        if (ticket != (unsigned)(nsplit - 1)) {
            uint64_t *mine_part = part_all + (int64_t)ks * (S::FM * S::FN * 64 * 2);
#pragma unroll
            for (int f = 0; f < S::FM; ++f)
#pragma unroll
                for (int j = 0; j < S::FN; ++j) {
                    const v4i v = __builtin_bit_cast(v4i, acc[f][j]);
                    uint64_t *d = mine_part + ((f * S::FN + j) * 64 + lane) * 2;
                    __hip_atomic_store(d, (uint64_t)(unsigned)v[1] << 32 | (unsigned)v[0],
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(d + 1, (uint64_t)(unsigned)v[3] << 32 | (unsigned)v[2],
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            __builtin_amdgcn_s_waitcnt(0);             // every store above has completed
            __atomic_signal_fence(__ATOMIC_SEQ_CST);   // and the compiler keeps them above
            if (lane == 0)
                __hip_atomic_fetch_add(words + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        while (__hip_atomic_load(words + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) !=
               (unsigned)(nsplit - 1))
            __builtin_amdgcn_s_sleep(1);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);       // no partial load moves above the wait
#pragma unroll 1
        for (int o = 0; o < nsplit; ++o) {
            if (o == ks)
                continue;
            const uint64_t *src = part_all + (int64_t)o * (S::FM * S::FN * 64 * 2);
#pragma unroll
            for (int f = 0; f < S::FM; ++f)
#pragma unroll
                for (int j = 0; j < S::FN; ++j) {
                    const uint64_t *q = src + ((f * S::FN + j) * 64 + lane) * 2;
                    const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    const v4i v = {(int)(unsigned)lo, (int)(unsigned)(lo >> 32), (int)(unsigned)hi,
                                   (int)(unsigned)(hi >> 32)};
                    acc[f][j] += __builtin_bit_cast(Acc, v);
                }
        }
        if (lane == 0) {
            __hip_atomic_store(words, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(words + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    const bool has_bias = !OUT_I32 && a.bias != nullptr;
#pragma unroll
    for (int f = 0; f < S::FM; ++f) {
        const int m = m0 + 16 * f + (lane & 15);
        if (m >= a.M)
            continue;
        const float xr = OUT_I32 ? 0.0f : FUSED ? rowscale[16 * f + (lane & 15)] : a.xs[m];
#pragma unroll
        for (int j = 0; j < S::FN; ++j) {
            const int n = 16 * (nb0 + j) + 4 * (lane >> 4);
            if (n >= a.N)
                continue;
            const Acc c = acc[f][j];
            const bool whole = a.vec_store && n + 3 < a.N;
            if (OUT_I32) {
                int *o = reinterpret_cast<int *>(a.out) + (int64_t)m * a.ldo + n;
                if (whole) {
                    *reinterpret_cast<v4i *>(o) = __builtin_bit_cast(v4i, c);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < a.N)
                            o[r] = __builtin_bit_cast(v4i, c)[r];
                }
                continue;
            }
            // The epilogue's fixed order per output: acc * xs, then * ws,
            // then + bias, each rounded to fp32; then round to nearest even
            // bf16.
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int nr = min(n + r, a.N - 1);
                v[r] = (float)c[r] * xr;
                v[r] = v[r] * a.ws[nr];
                if (has_bias) {
                    const unsigned b = a.bias[nr];
                    v[r] = v[r] + (OUT_F16 ? quant_rule::f16_to_float(b) : __uint_as_float(b << 16));
                }
            }
            v2u pk;
            if (OUT_F16) {
                const f16x2 lo = __builtin_convertvector((f32x2){v[0], v[1]}, f16x2);
                const f16x2 hi = __builtin_convertvector((f32x2){v[2], v[3]}, f16x2);
                pk = v2u{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
            } else {
                const bf16x2 lo = __builtin_convertvector((f32x2){v[0], v[1]}, bf16x2);
                const bf16x2 hi = __builtin_convertvector((f32x2){v[2], v[3]}, bf16x2);
                pk = v2u{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
            }
            uint16_t *o = reinterpret_cast<uint16_t *>(a.out) + (int64_t)m * a.ldo + n;
            if (whole) {
                *reinterpret_cast<v2u *>(o) = pk;
            } else {
                const unsigned hv[4] = {pk[0] & 0xffffu, pk[0] >> 16, pk[1] & 0xffffu, pk[1] >> 16};
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < a.N)
                        o[r] = (uint16_t)hv[r];
            }
        }
    }
}

template <class S>
constexpr TileEntry skinny(const char *name)
{
    static_assert(S::U == 4, "skinny_split counts load groups of 4 k-blocks");
    return TileEntry{name, S::BM, S::BN, S::THREADS, true,
                     {skinny_mm_kernel<S, kOutBF16, false>, skinny_mm_kernel<S, kOutI32, false>,
                      skinny_mm_kernel<S, kOutF16, false>},
                     {skinny_mm_kernel<S, kOutBF16, true>, skinny_mm_kernel<S, kOutI32, true>,
                      skinny_mm_kernel<S, kOutF16, true>}};
}

// 16*FM token rows x 16*FN channels / WK waves along K / U k-blocks per
// load group.
const TileEntry kSkinny[] = {
    skinny<Skinny<1, 1, 8, 4>>("s16x16/k8/u4"),
    skinny<Skinny<1, 1, 4, 4>>("s16x16/k4/u4"),
    skinny<Skinny<1, 2, 8, 4>>("s16x32/k8/u4"),
    skinny<Skinny<2, 1, 8, 4>>("s32x16/k8/u4"),
};


template <class S>
constexpr TileEntry skinny_fp8(const char *name)
{
    return TileEntry{name, S::BM, S::BN, S::THREADS, true,
                     {skinny_mm_kernel<S, kOutBF16, false, true>,
                      skinny_mm_kernel<S, kOutI32, false, true>,
                      skinny_mm_kernel<S, kOutF16, false, true>},
                     {skinny_mm_kernel<S, kOutBF16, true, true>,
                      skinny_mm_kernel<S, kOutI32, true, true>,
                      skinny_mm_kernel<S, kOutF16, true, true>}};
}

// The e4m3 twin's small-M configurations, in the same order.
const TileEntry kSkinnyFp8[] = {
    skinny_fp8<Skinny<1, 1, 8, 4>>("s16x16/k8/u4"),
    skinny_fp8<Skinny<1, 1, 4, 4>>("s16x16/k4/u4"),
    skinny_fp8<Skinny<1, 2, 8, 4>>("s16x32/k8/u4"),
    skinny_fp8<Skinny<2, 1, 8, 4>>("s32x16/k8/u4"),
};
static_assert(sizeof(kSkinnyFp8) == sizeof(kSkinny), "the twin has the same configurations");

}  // namespace

int skinny_tile_count() { return (int)(sizeof(kSkinny) / sizeof(kSkinny[0])); }
const TileEntry &skinny_tile(int i) { return kSkinny[i]; }
const TileEntry &skinny_tile_fp8(int i) { return kSkinnyFp8[i]; }

hipError_t launch_skinny_quant_mm(const MmArgs &a, const TileEntry &e, int mode,
                                  hipStream_t stream)
{
    const int64_t rows = std::min<int64_t>(a.M, e.bm);
    const int64_t cpr = ceil_div(a.K / 8, e.threads);
    if (rows > kQuantRows || rows * cpr > kQuantSlots)
        return hipErrorNotSupported;
    const size_t lds = (size_t)(rows * (a.K + 16));
    const int64_t tiles = ceil_div(a.M, e.bm) * ceil_div(a.N, e.bn) * (a.ksplit > 1 ? a.ksplit : 1);
    hipLaunchKernelGGL(e.fused[mode], dim3((unsigned)tiles), dim3(e.threads),
                       lds, stream, a);
    return hipGetLastError();
}

// The workspace of int8_quant_scaled_mm_noalloc: the split counters
// (zero when the code object loads; every call leaves them zero) and the
// partial sums. Host code never passes this name to a kernel: it is a
// host-side stand-in, and scratch_address() gives the device address.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_address(void **ptr)
{
    constexpr int kDevices = 64;
    static std::mutex lock;
    static void *addr[kDevices];
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return err;
    if (dev < 0 || dev >= kDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> guard(lock);
    if (addr[dev] == nullptr) {
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess)
            return err;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

SkinnySplit skinny_split(int64_t tiles, int fm, int fn, int wk, int kblocks)
{
    // A wave walks its k-blocks in load groups of kGroup, one memory round
    // trip each, so an unsplit tile takes about kblocks / (wk * kGroup)
    // round trips; meeting the other workgroups of a split through memory
    // costs about three (measured on MI355X: 3-5 us). Split only where the
    // chain is long (at least 12 groups: K of 24576 and more on eight
    // waves), into as many as 8 ways that leave at least 4 groups each and
    // at most about two workgroups per CU. Measured: K 131056, N 16: 48.4 ->
    // 12.1 us; K 65536, N 512: 27.1 -> 13.3 us; K 32768, N 1024, 4 rows:
    // 16.8 -> 14.6 us; K 12288, N 3072 (6 groups): 9.3 us unsplit against
    // 15.9 split, so no split there.
    constexpr int kGroup = 4;               // every small-M configuration's U
    const int64_t chain = ceil_div(kblocks, (int64_t)wk * kGroup);
    SkinnySplit r{1, kblocks, 0, 0};
    if (chain >= 12) {
        for (int s = 2; s <= 8; s *= 2) {
            if (tiles * (s / 2) >= 512 || chain / s < 4)
                break;
            r.ksplit = s;
        }
    }
    r.kbs = (int)ceil_div(kblocks, r.ksplit);
    r.count_bytes = (size_t)round_up(tiles * 8, 256);
    r.part_bytes = (size_t)tiles * r.ksplit * fm * fn * 1024;
    return r;
}

}  // namespace w8a8
