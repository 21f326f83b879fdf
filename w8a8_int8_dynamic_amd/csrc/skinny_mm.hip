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
// Ragged tails as in the main kernel: token rows past M read row M-1,
// fragments past N read the last fragment, token chunks past K read the last
// chunk (which meets zero weights); stores are masked.
#include "internal.hpp"

namespace w8a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// FM blocks of 16 token rows and FN fragments of 16 channels per
// workgroup; WK wavefronts split K; U k-blocks per load group.
template <int FM_, int FN_, int WK_, int U_>
struct Skinny {
    static constexpr int FM = FM_, FN = FN_, WK = WK_, U = U_;
    static constexpr int BM = 16 * FM, BN = 16 * FN, THREADS = 64 * WK;
    static_assert(WK >= 2 && WK <= 16, "two to sixteen wavefronts");
    static_assert(U * (FM + FN) * 4 <= 128, "operand registers");
};

// At least 16 wavefronts per CU (128 registers each): the kernel lives on
// the loads it keeps in flight, so occupancy counts more than ILP.
template <class S, bool OUT_I32>
__global__ __launch_bounds__(S::THREADS, 1024 / S::THREADS) void skinny_mm_kernel(const MmArgs a)
{
    // Waves 1 .. WK-1 hand their partial sums to wave 0.
    __shared__ v4i part[S::WK - 1][S::FM * S::FN][64];

    const int lane = threadIdx.x & 63;
    const int wk = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tiles_m = (a.M + S::BM - 1) / S::BM;
    const int tiles_n = (a.nblocks + S::FN - 1) / S::FN;
    // The row tiles of one weight column run on one XCD, next to each other.
    const int t = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    const int m0 = (t % tiles_m) * S::BM, nb0 = (t / tiles_m) * S::FN;
    const int KB = a.kblocks;
    const int klast = a.K - 16;

    const v4i *wsrc[S::FN];
#pragma unroll
    for (int j = 0; j < S::FN; ++j)
        wsrc[j] = reinterpret_cast<const v4i *>(a.wp) + (int64_t)min(nb0 + j, a.nblocks - 1) * KB * 64 +
                  lane;
    const int8_t *tsrc[S::FM];
#pragma unroll
    for (int f = 0; f < S::FM; ++f)
        tsrc[f] = a.xq + (int64_t)min(m0 + 16 * f + (lane & 15), a.M - 1) * a.ldq;
    const int kc = 16 * (lane >> 4);

    v4i acc[S::FM][S::FN];
#pragma unroll
    for (int f = 0; f < S::FM; ++f)
#pragma unroll
        for (int j = 0; j < S::FN; ++j)
            acc[f][j] = v4i{};

    auto block = [&](int kb, v4i (&w)[S::FN], v4i (&x)[S::FM]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < S::FN; ++j)
            w[j] = __builtin_nontemporal_load(wsrc[j] + (int64_t)kb * 64);
#pragma unroll
        for (int f = 0; f < S::FM; ++f)
            x[f] = *reinterpret_cast<const v4i *>(tsrc[f] + min(kb * 64 + kc, klast));
    };
    auto mma = [&](const v4i (&w)[S::FN], const v4i (&x)[S::FM]) __attribute__((always_inline)) {
#pragma unroll
        for (int f = 0; f < S::FM; ++f)
#pragma unroll
            for (int j = 0; j < S::FN; ++j)
                acc[f][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[j], x[f], acc[f][j], 0, 0, 0);
    };

    // This wave's k-blocks: wk, wk+WK, ... (mine of them). Full load groups,
    // then one partial group; within a group every load is issued before the
    // first MFMA waits on any of them.
    // Each workgroup starts its walk at its own offset (rot), so that the
    // workgroups of an XCD do not all ask one L2 channel for the same token
    // bytes at once.
    const int mine = wk < KB ? (KB - 1 - wk) / S::WK + 1 : 0;
    const int rot = mine > 0 ? t % mine : 0;
    auto kb_of = [&](int i) __attribute__((always_inline)) {
        i += rot;
        return wk + (i >= mine ? i - mine : i) * S::WK;
    };
    int g = 0;
#pragma unroll 1
    for (; g + S::U <= mine; g += S::U) {
        v4i w[S::U][S::FN], x[S::U][S::FM];
#pragma unroll
        for (int u = 0; u < S::U; ++u)
            block(kb_of(g + u), w[u], x[u]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < S::U; ++u)
            mma(w[u], x[u]);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (g < mine) {
        v4i w[S::U][S::FN], x[S::U][S::FM];
#pragma unroll
        for (int u = 0; u < S::U; ++u)
            if (g + u < mine)
                block(kb_of(g + u), w[u], x[u]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < S::U; ++u)
            if (g + u < mine)
                mma(w[u], x[u]);
    }

    if (wk > 0) {
#pragma unroll
        for (int f = 0; f < S::FM; ++f)
#pragma unroll
            for (int j = 0; j < S::FN; ++j)
                part[wk - 1][f * S::FN + j][lane] = acc[f][j];
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
                acc[f][j] += part[w][f * S::FN + j][lane];

    const bool has_bias = !OUT_I32 && a.bias != nullptr;
#pragma unroll
    for (int f = 0; f < S::FM; ++f) {
        const int m = m0 + 16 * f + (lane & 15);
        if (m >= a.M)
            continue;
        const float xr = OUT_I32 ? 0.0f : a.xs[m];
#pragma unroll
        for (int j = 0; j < S::FN; ++j) {
            const int n = 16 * (nb0 + j) + 4 * (lane >> 4);
            if (n >= a.N)
                continue;
            const v4i c = acc[f][j];
            const bool whole = a.vec_store && n + 3 < a.N;
            if (OUT_I32) {
                int *o = reinterpret_cast<int *>(a.out) + (int64_t)m * a.ldo + n;
                if (whole) {
                    *reinterpret_cast<v4i *>(o) = c;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < a.N)
                            o[r] = c[r];
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
                if (has_bias)
                    v[r] = v[r] + __uint_as_float((unsigned)a.bias[nr] << 16);
            }
            const bf16x2 lo = __builtin_convertvector((f32x2){v[0], v[1]}, bf16x2);
            const bf16x2 hi = __builtin_convertvector((f32x2){v[2], v[3]}, bf16x2);
            const v2u pk = v2u{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
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
    return TileEntry{name, S::BM, S::BN, S::THREADS, true, skinny_mm_kernel<S, false>,
                     skinny_mm_kernel<S, true>, nullptr, nullptr};
}

// 16*FM token rows x 16*FN channels / WK waves along K / U k-blocks per
// load group.
const TileEntry kSkinny[] = {
    skinny<Skinny<1, 1, 8, 4>>("s16x16/k8/u4"),
    skinny<Skinny<1, 1, 4, 4>>("s16x16/k4/u4"),
    skinny<Skinny<1, 2, 8, 4>>("s16x32/k8/u4"),
    skinny<Skinny<2, 1, 8, 4>>("s32x16/k8/u4"),
};

}  // namespace

int skinny_tile_count() { return (int)(sizeof(kSkinny) / sizeof(kSkinny[0])); }
const TileEntry &skinny_tile(int i) { return kSkinny[i]; }

}  // namespace w8a8
