// int8 x int8 -> int32 matmul with the fused scale epilogue, for gfx950.
//
// What it computes (page "Issue 5 probe: int8 quantized DiT serve paths on
// the RTX 3090 (24 GB)", "Round two" kernel-path paragraph; page "INT8 Quant
// for Dual-Max Recipe": int8 x int8 on the matrix cores, no dequantization):
//   acc[m,n] = sum_k xq[m,k] * wq[n,k]                    exact int32
//   out[m,n] = bf16_rne(fl(fl(fl(acc) * xs[m]) * ws[n]) [+ bias[n]])
// or the raw accumulators in the int32 debug mode.
//
// Design (a dense contraction: the int8 MFMA roofline bounds it). Measured
// on MI355X, the limits that shape it are the rate of the MFMA itself, the
// LDS bandwidth shared by MFMA operand reads and global->LDS copies, and the
// cost of a workgroup barrier when each SIMD runs a single wavefront.
//   - v_mfma_i32_32x32x32_i8, the full-rate int8 MFMA on gfx950 (the
//     16x16x64 form runs at about half its rate). The weight fragment is the
//     MFMA "A" operand (32 output channels x 32 k), the token fragment the
//     "B" operand (32 tokens x 32 k): each lane's accumulators come in runs
//     of four consecutive output channels of one token.
//   - Four wavefronts split a BM x BN tile into WN column groups and WK
//     k-groups: wave (wn, wk) owns all BM rows and BN/WN columns, and takes
//     every WK-th 64-deep k-block. No weight fragment is used by two waves,
//     so weights skip LDS: each wave loads its operands straight from the
//     prepacked weight into a ring of LW+1 register sets (each load is 64
//     lanes x 16 bytes in four contiguous 256-byte runs).
//   - Token rows are shared by the WN waves of a k-group, so they go
//     through LDS: a ring of LT+1 stages (WK k-blocks each), filled straight
//     from memory by buffer_load_dwordx4 ... lds (no staging registers, no
//     LDS write instructions), LT stages ahead of the operand reads; one
//     barrier per stage. The MUBUF form of the LDS load matters: the
//     compiler takes a FLAT-encoded one (global_load_lds) as possibly
//     completing out of order and then turns every later wait into a full
//     vmcnt(0). Against the earlier scheme (ordinary loads into registers,
//     then ds_write_b128), measured on MI355X: 1.9 % faster on the
//     fused-QKV shape, 5-6 % on the 256-row tiles, outputs bit-identical.
//   - A 16-row x 64-k token image is loaded with lane 4r+j reading k-chunk
//     j ^ swz(r) of row r into slot 4r+j: every 4-lane quad reads one row's 64 contiguous
//     bytes (one memory sector per quad, several times faster than a
//     row-per-lane gather), and the swizzle keeps the later MFMA operand
//     reads (row l%32, chunk c: slot 4r + (c ^ swz(r))) on distinct banks.
//   - The WK k-groups' int32 partial sums meet in LDS after the K loop; the
//     scaled bf16 tile is staged in LDS and written back in whole rows
//     (consecutive lanes on consecutive 8-byte pieces: full cache lines).
//   - Workgroup ids are remapped so consecutive tiles (the M tiles that
//     share one N stripe of the weight) land on one XCD and share its L2.
// Ragged tails: token rows past M and weight images past N read the last
// valid row/image (their results are never stored); token k-chunks past K
// read the last valid chunk, which meets zero weights (the prepacked weight
// is zero beyond K); k-blocks past the end of K are skipped. Every load
// stays inside its operand; stores are masked.
#pragma once

#include <array>
#include <tuple>
#include <type_traits>
#include <utility>

#include "fused_rows.hpp"
#include "internal.hpp"
#include "quant_rule.hpp"
#include "timeline.hpp"

namespace w8a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Four fp32 values rounded to nearest-even 16-bit floats (fp16 when F16,
// else bf16), packed in order into two words.
template <bool F16>
__device__ __forceinline__ v2u pack4(const float (&t)[4])
{
    if (F16) {
        const f16x2 lo = __builtin_convertvector((f32x2){t[0], t[1]}, f16x2);
        const f16x2 hi = __builtin_convertvector((f32x2){t[2], t[3]}, f16x2);
        return v2u{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
    }
    const bf16x2 lo = __builtin_convertvector((f32x2){t[0], t[1]}, bf16x2);
    const bf16x2 hi = __builtin_convertvector((f32x2){t[2], t[3]}, bf16x2);
    return v2u{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
}

// Logical tile id -> (tm, tn): bands of kBandM M-tiles; inside a band the
// M index runs fastest. The 32 tiles an XCD runs at once then form a block
// of at most 4 x 8 output tiles, whose token rows and weight columns its L2
// holds together, instead of one weight stripe against every token row.
constexpr int kBandM = 4;
__device__ __forceinline__ void tile_of(int t, int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int band = t / (kBandM * tiles_n);
    const int r = t - band * kBandM * tiles_n;
    const int gm = min(kBandM, tiles_m - band * kBandM);   // M-tiles in this band
    tm = band * kBandM + r % gm;
    tn = r / gm;
}

// s_waitcnt lgkmcnt(0) only (vmcnt and expcnt untouched; gfx9 encoding):
// this wave's LDS reads and writes have completed.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F & ~0x0F00); }

// s_waitcnt vmcnt(VM) lgkmcnt(0).
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0()
{
    static_assert(VM >= 0 && VM < 64, "vmcnt out of range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));
}

// 16 bytes per lane from base + voff straight into LDS
// (buffer_load_dwordx4 ... lds): lane l's bytes land at lds_dst + 16*l
// (lds_dst wave-uniform). The buffer resource covers [base, base + 2 GiB)
// with the gfx9-family raw-buffer configuration word, so offsets are 32-bit
// and one past the range would read zeros rather than fault. The resource
// type exists only in the device pass (the host pass would otherwise drop
// the kernels' launch stubs).
__device__ __forceinline__ void dma16(const void *base, int voff, void *lds_dst)
{
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_dst, 16, voff, 0, 0, 0);
#endif
}

__device__ __forceinline__ int tok_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// A kernel argument held in scalar registers from here on. Left alone, the
// compiler re-reads kernel arguments from memory wherever it needs them
// (each re-read a scalar load plus a wait) instead of keeping them.
template <class V>
__device__ __forceinline__ V pinned(V v)
{
    asm volatile("" : "+s"(v));
    return v;
}
// The same for a global-memory pointer: the value passes through an
// integer, so it is converted back through the global address space, which
// keeps its loads and stores global (not flat) instructions.
template <class P>
__device__ __forceinline__ P *pinned_ptr(P *p)
{
    typedef __attribute__((address_space(1))) P GP;
    return (P *)(GP *)pinned(reinterpret_cast<uintptr_t>(p));
}

// f(std::integral_constant<int, u>) for u = 0 .. N-1: compile-time indices
// into the register rings, whatever the compiler decides about unrolling.
template <class F, int... U>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, U...>)
{
    (f(std::integral_constant<int, U>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

constexpr int cgcd(int a, int b) { return b == 0 ? a : cgcd(b, a % b); }
constexpr int clcm(int a, int b) { return a / cgcd(a, b) * b; }

// BM x BN output tile; WM row groups x WN column groups x WK k-groups of
// wavefronts; token images loaded into LDS LT stages ahead of the step that
// reads them (a ring of LT+1 LDS stages), weights into registers LW stages
// ahead of their use. WL: the weights go through LDS as well (whole images
// in the token stages), so that row groups sharing a weight fragment
// (WM = 2) fetch it once; LW is then unused. MP: memory instructions placed
// after each MFMA of a step's interleave (int8; the e4m3 twin spreads them
// evenly over its MFMAs).
template <int BM_, int BN_, int WM_, int WN_, int WK_, int LT_, int LW_, bool WL_ = false,
          int MP_ = 1>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, WK = WK_, LT = LT_, LW = LW_;
    static constexpr bool WLDS = WL_;
    static constexpr int MP = MP_;
    static constexpr int NW = WM * WN * WK;            // wavefronts per workgroup
    static constexpr int THREADS = NW * 64;
    static constexpr int MB = BM / 16;                 // 16-row token images per k-block
    static constexpr int FM = BM / WM / 32;            // 32x32 MFMA tiles per wave, rows
    static constexpr int FN = BN / WN / 32;            // ... and columns
    static constexpr int AIMG = WK * MB;               // token images per stage
    static constexpr int WIMG = WLDS ? WK * (BN / 16) : 0;  // weight images per stage in LDS
    static constexpr int LA = AIMG / NW;               // token image loads per wave per stage
    static constexpr int LW8 = WIMG / NW;              // weight image loads per wave (LDS path)
    static constexpr int LB = WLDS ? 0 : 2 * FN;       // weight register loads per wave per stage
    static constexpr int LPW = LA + LW8 + LB;          // loads per wave per stage
    static constexpr int NS = LT + 1;                  // LDS stages
    static constexpr int NB = WLDS ? 1 : LW + 1;       // weight register sets
    static constexpr int GROUP = clcm(clcm(NB, 2), NS);     // steps per unrolled loop body
    static constexpr int AHEAD = WLDS ? LT + 1 : cmax(LT + 1, LW);  // furthest stage fetched
    // Steady-state wait at the top of step s: stage s+1's images (the first
    // loads of step s-LT; on the LDS path the weight images follow the
    // tokens) and the weights of stage s (the last loads of step s-LW) have
    // landed.
    static constexpr int VM = WLDS ? (LT - 1) * LPW
                                   : (LB + (LT - 1) * LPW < (LW - 1) * LPW ? LB + (LT - 1) * LPW
                                                                           : (LW - 1) * LPW);
    static constexpr int STAGE = (AIMG + WIMG) * 64;   // 16-byte slots per LDS stage
    static constexpr int RING = NS * STAGE * 16;       // LDS ring, bytes
    static constexpr int PART = (WK - 1) * BM * BN * 4;     // k-group partial sums
    static constexpr int PITCH = BN * 2 + 16;          // staged bf16 row, bytes
    static constexpr int OUTB = BM * PITCH;
    // The bf16 tile goes after the k-group partials (which it meets in the
    // epilogue); with one k-group it reuses the ring, idle by then.
    static constexpr int TILE_OFF = WK > 1 ? cmax(RING, PART) : 0;
    static constexpr int MAIN = cmax(TILE_OFF + OUTB, RING);
    static constexpr int SIDE = 2 * BN + BM;           // fp32 ws, bias, xs of the tile
    static constexpr int SIDE_PER_THREAD = (SIDE + THREADS - 1) / THREADS;
    static constexpr int FLAG = MAIN + SIDE * 4;        // one word: fused-path decision
    static constexpr int LDS = FLAG + 16;
    static_assert(NW == 4 || NW == 8, "four or eight wavefronts per workgroup");
    static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "tile/wave mismatch");
    static_assert(AIMG % NW == 0, "token loads must split evenly over waves");
    static_assert(WIMG % NW == 0, "weight image loads must split evenly over waves");
    static_assert(LT >= 1 && (NS & (NS - 1)) == 0, "LDS ring of a power-of-two stages");
    static_assert(WLDS || LW >= LT, "weight lead >= token lead");
    static_assert(VM < 64 && (LT + 1) * LPW < 64 && (LW + 1) * LPW < 64, "vmcnt range");
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert(FM * FN * 16 <= 1024 / NW, "accumulators must leave room for operands");
    static_assert(WK <= 2 && FM % WK == 0, "k-groups split the row tiles evenly");
};

// OUT: kOutBF16, kOutI32 or kOutF16. The fused form reads x in the output's
// 16-bit type (bf16 for the int32 debug mode).
// FP8: the e4m3 twin (operands are e4m3 codes in the same layout; one
// v_mfma_scale_f32_32x32x64_f8f6f4 per k-block with unit block scales,
// fp32 accumulators; kOutI32 then stores the raw fp32 accumulators; the
// fused form writes e4m3 codes).
template <class T, int OUT, bool FUSED, bool FP8 = false>
__global__ __launch_bounds__(T::THREADS) void scaled_mm_kernel(const MmArgs args)
{
    constexpr bool OUT_I32 = OUT == kOutI32, OUT_F16 = OUT == kOutF16;
    using Acc = std::conditional_t<FP8, v16f, v16i>;
    constexpr int IN = OUT_F16 ? kElemF16 : kElemBF16;
    __shared__ uint4 lds[T::LDS / 16];
    W8A8_STAMP(0);

    MmArgs a;
    a.xq = pinned_ptr(args.xq);
    a.xs = pinned_ptr(args.xs);
    a.wp = pinned_ptr(args.wp);
    a.ws = pinned_ptr(args.ws);
    a.bias = pinned_ptr(args.bias);
    a.out = pinned_ptr(args.out);
    a.ldq = pinned(args.ldq);
    a.ldo = pinned(args.ldo);
    a.M = pinned(args.M);
    a.N = pinned(args.N);
    a.K = pinned(args.K);
    a.kblocks = pinned(args.kblocks);
    a.nblocks = pinned(args.nblocks);
    a.vec_store = pinned(args.vec_store);
    a.vec16 = pinned(args.vec16);
    if (FUSED) {
        a.x = pinned_ptr(args.x);
        a.ldx = pinned(args.ldx);
        a.rows_per_wg = pinned(args.rows_per_wg);
        a.epoch = pinned(args.epoch);
        a.wait_limit = pinned(args.wait_limit);
    }

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave % T::WN, wm = (wave / T::WN) % T::WM, wk = wave / (T::WN * T::WM);

    const int tiles_m = (a.M + T::BM - 1) / T::BM;
    const int tiles_n = (a.N + T::BN - 1) / T::BN;
    int tm, tn;
    tile_of(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const int S = (a.kblocks + T::WK - 1) / T::WK;     // ring stages: WK k-blocks each
    const int klast = a.K - 16;                        // last valid 16-byte k-chunk
    const int kblast = a.kblocks - 1;

    // Token sources of this lane: stage image g = i*NW + wave is k-block
    // g / MB of the stage and rows m0 + 16*(g % MB) .. +16; lane 4r+j reads
    // row r (clamped to M-1), k-chunk j ^ swz(r), and stores it to slot 4r+j.
    const int drow = lane >> 2;
    const int dchunk = ((lane & 3) ^ tok_swz(drow)) * 16;
    const int8_t *arow[T::LA];
    int aks[T::LA];
#pragma unroll
    for (int i = 0; i < T::LA; ++i) {
        const int g = i * T::NW + wave;
        aks[i] = g / T::MB;
        const int row = min(m0 + (g % T::MB) * 16 + drow, a.M - 1);
        arow[i] = a.xq + (int64_t)row * a.ldq;
    }
    // Weight operand sources: 32-channel group j of this wave is images
    // n0/16 + 2*(wn*FN + j) + {0,1}; lane l reads image (l>>4)&1, slot
    // 16*(2h + l/32) + l%16 of k-block kb.
    const v4i *bsrc[T::FN];
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
        const int img = min(n0 / 16 + (wn * T::FN + j) * 2 + ((lane >> 4) & 1), a.nblocks - 1);
        bsrc[j] = reinterpret_cast<const v4i *>(a.wp) + (int64_t)img * a.kblocks * 64 +
                  (lane >> 5) * 16 + (lane & 15);
    }
    // LDS slots of this lane's token operand (pair of images, per k-half).
    int xslot[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r16 = lane & 15, c = 2 * h + (lane >> 5);
        xslot[h] = ((lane >> 4) & 1) * 64 + 4 * r16 + (c ^ tok_swz(r16));
    }

    Acc acc[T::FN][T::FM];
    // Accumulator registers 4q .. 4q+3 as raw 32-bit words (for the LDS
    // exchange and the raw output), and one accumulator plus the other
    // k-group's partial (raw bits) as fp32: an exact int32 sum converted
    // once, or an fp32 sum.
    auto quad_bits = [](const Acc &c, int q) __attribute__((always_inline)) {
        if constexpr (FP8)
            return __builtin_bit_cast(v4i, f32x4{c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]});
        else
            return v4i{c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]};
    };
    auto acc_plus = [](const Acc &c, int k, int other) __attribute__((always_inline)) {
        if constexpr (FP8)
            return c[k] + __int_as_float(other);
        else
            return (float)(c[k] + other);
    };
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
            acc[j][i] = Acc{};
    v4i bq[T::NB][T::FN][2];                           // weight operand ring (direct path)
    v4i xf[2][T::FM][2];                               // token operands, this and next stage
    v4i bf[T::WLDS ? 2 : 1][T::FN][2];                 // weight operands from LDS, this and next

    // Weights of stage t into ring set t % NB. Addresses are clamped into
    // the operands, so a load of a stage past the end is harmless.
    auto load_b = [&](int t, v4i (&bset)[T::FN][2]) __attribute__((always_inline)) {
        const int kb = min(t * T::WK + wk, kblast);
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                bset[j][h] = bsrc[j][(int64_t)kb * 64 + h * 32];
    };
    // The token images (and, on the LDS path, the weight images) of stage t
    // straight from memory into LDS stage t % NS: image g of the stage to its
    // 1 KB slot, lane l to 16-byte slot l. Token image g = i*NW + wave is
    // k-block g / MB of the stage, rows 16*(g % MB) ..; weight image g is
    // k-block g / (BN/16), channel image g % (BN/16) of the tile. Offsets are
    // from the tile's first token row and first weight image (32-bit).
    // Addresses are clamped into the operands, so a load of a stage past the
    // end is harmless.
    const int8_t *xb = a.xq + (int64_t)m0 * a.ldq;
    const char *wb = reinterpret_cast<const char *>(a.wp) + (int64_t)(n0 / 16) * a.kblocks * 1024;
    int aoff[T::LA];
#pragma unroll
    for (int i = 0; i < T::LA; ++i)
        aoff[i] = (int)(arow[i] - xb);
    auto dma = [&](int t) __attribute__((always_inline)) {
        char *st = reinterpret_cast<char *>(lds) + (t & (T::NS - 1)) * T::STAGE * 16;
#pragma unroll
        for (int i = 0; i < T::LA; ++i) {
            const int g = i * T::NW + wave;
            const int kc = min((t * T::WK + aks[i]) * 64 + dchunk, klast);
            dma16(xb, aoff[i] + kc, st + g * 1024);
        }
#pragma unroll
        for (int i = 0; i < T::LW8; ++i) {
            const int g = i * T::NW + wave;
            const int kb = min(t * T::WK + g / (T::BN / 16), kblast);
            const int img = min(n0 / 16 + g % (T::BN / 16), a.nblocks - 1) - n0 / 16;
            dma16(wb, (img * a.kblocks + kb) * 1024 + lane * 16, st + (T::AIMG + g) * 1024);
        }
    };
    // LDS path: this wave's weight operands of stage t (its k-group's
    // k-block): for 32-channel group j the images 2*(wn*FN+j) + (l>>4 & 1),
    // slot 16*(2h + l/32) + l%16, as the direct path loads them.
    auto bread = [&](int t, v4i (&b)[T::FN][2]) __attribute__((always_inline)) {
        const v4i *st = reinterpret_cast<const v4i *>(lds) + (t & (T::NS - 1)) * T::STAGE +
                        (T::AIMG + wk * (T::BN / 16)) * 64;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < T::FN; ++j)
                b[j][h] = st[(2 * (wn * T::FN + j) + ((lane >> 4) & 1)) * 64 + 16 * (2 * h + (lane >> 5)) +
                             (lane & 15)];
    };
    // This wave's token operands of stage t (its k-group's k-block) from LDS.
    auto read = [&](int t, v4i (&x)[T::FM][2]) __attribute__((always_inline)) {
        const v4i *st = reinterpret_cast<const v4i *>(lds) + (t & (T::NS - 1)) * T::STAGE + wk * T::MB * 64 +
                        wm * (2 * T::FM) * 64;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
                x[i][h] = st[(2 * i) * 64 + xslot[h]];
    };
    // MFMAs number q0 .. q1-1 of a stage, in the order (h, j, i): a wave's 2*FN*FM
    // MFMAs per stage touch every accumulator twice, FN*FM apart. The e4m3
    // twin takes both halves of a k-block in one MFMA, in the order (j, i).
    auto mma = [&](auto q0_c, auto q1_c, const v4i (&x)[T::FM][2], const v4i (&b)[T::FN][2])
                   __attribute__((always_inline)) {
        constexpr int q0 = decltype(q0_c)::value, q1 = decltype(q1_c)::value;
        static_for<q1 - q0>([&](auto Q) __attribute__((always_inline)) {
            constexpr int q = q0 + decltype(Q)::value;
            if constexpr (FP8) {
                constexpr int j = q / T::FM, i = q % T::FM;
                const v8i bb = __builtin_shufflevector(b[j][0], b[j][1], 0, 1, 2, 3, 4, 5, 6, 7);
                const v8i xx = __builtin_shufflevector(x[i][0], x[i][1], 0, 1, 2, 3, 4, 5, 6, 7);
                acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bb, xx, acc[j][i], 0, 0,
                                                                            0, 127, 0, 127);
            } else {
                constexpr int h = q / (T::FN * T::FM), j = (q / T::FM) % T::FN, i = q % T::FM;
                acc[j][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b[j][h], x[i][h], acc[j][i], 0, 0, 0);
            }
        });
    };
    constexpr int NMMA = (FP8 ? 1 : 2) * T::FN * T::FM;   // MFMAs per wave per stage
    constexpr int PRE = FP8 ? 1 : 2;                   // of them issued before the barrier
    // Memory instructions placed after each MFMA of the interleave: the
    // tile's MP for int8 (one where a step has about as many memory
    // instructions as MFMAs; two or three on the tiles with two or three
    // times as many, measured on MI355X); the e4m3 twin has half as many
    // (twice as long) MFMAs, so its memory instructions are spread over them.
    constexpr int DS_READS = 2 * T::FM + (T::WLDS ? 2 * T::FN : 0);
    constexpr int MEM_OPS = DS_READS + T::LPW;
    constexpr int PER = FP8 ? (MEM_OPS + NMMA - PRE - 1) / (NMMA - PRE) : T::MP;

    // Step s. On entry this wave's operands of stage s are in xf[s & 1], the
    // images of stages s+1 .. s+LT are landing in LDS and the weights of
    // stage s are in ring set s % NB. The step: wait until stage s+1's images
    // and stage s's weights have landed; the first MFMAs of stage s (they keep
    // the matrix core busy across the barrier); barrier (stage s+1 visible to
    // every wave; every read of stage s done); read stage s+1's operands; load
    // stage s+1+LT's images into the LDS stage that stage s used and the
    // weights of stage s+LW, interleaved (PER at a time) with the rest of
    // stage s's MFMAs so that they issue while the matrix core is busy.
    // The compiler does not order LDS reads after these loads: the explicit
    // waits and the barrier do.
    auto step = [&](auto full, int s, auto u_c) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full)::value;
        constexpr int u = decltype(u_c)::value;        // s modulo GROUP
        const bool run = FULL || s * T::WK + wk < a.kblocks;
        // The steady state waits for exactly what it needs; the last steps
        // (where fewer loads follow) drain.
        if (FULL)
            wait_vm_lgkm0<T::VM>();
        else
            wait_vm_lgkm0<0>();
        auto &wcur = [&]() -> auto & {
            if constexpr (T::WLDS)
                return bf[u & 1];
            else
                return bq[u % T::NB];
        }();
        if (run)
            mma(std::integral_constant<int, 0>{}, std::integral_constant<int, PRE>{}, xf[u & 1], wcur);
        __builtin_amdgcn_s_barrier();
        if (FULL || s + 1 < S) {
            read(s + 1, xf[(u + 1) & 1]);
            if constexpr (T::WLDS)
                bread(s + 1, bf[(u + 1) & 1]);
        }
        if (FULL || s + 1 + T::LT < S)
            dma(s + 1 + T::LT);
        if constexpr (!T::WLDS) {
            if (FULL || s + T::LW < S)
                load_b(s + T::LW, bq[(u + T::LW) % T::NB]);
        }
        if (run)
            mma(std::integral_constant<int, PRE>{}, std::integral_constant<int, NMMA>{}, xf[u & 1], wcur);
        if (FULL) {
            // PER memory instructions after each MFMA: the operand reads
            // first, then the loads.
            static_for<(DS_READS + PER - 1) / PER>([&](auto) __attribute__((always_inline)) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, PER, 0); // DS read
            });
            static_for<(T::LPW + PER - 1) / PER>([&](auto) __attribute__((always_inline)) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, PER, 0); // VMEM read
            });
        }
        // Keep each step's loads in program order relative to the next
        // step, so the load counter pattern repeats exactly.
        __builtin_amdgcn_sched_barrier(0);
    };
    using Full = std::integral_constant<bool, true>;
    using Part = std::integral_constant<bool, false>;

    if (FUSED) {
        // Fused quant: this workgroup quantizes rows [r0, r1) of x and
        // publishes them (rows_per_wg divides BM, so the rows belong to one
        // M-tile), then waits for the producers of its own tile's rows.
        quant_rule::u32 *red = reinterpret_cast<quant_rule::u32 *>(lds);
        // A word no other phase writes: every wave reads it after the
        // wait's barrier while others may already be filling the ring.
        quant_rule::u32 *decision =
            reinterpret_cast<quant_rule::u32 *>(reinterpret_cast<char *>(lds) + T::FLAG);
        const int r0 = (int)blockIdx.x * a.rows_per_wg;
        const int r1 = min(r0 + a.rows_per_wg, a.M);
        fused::quantize_rows<T::THREADS, IN, FP8>(a, r0, r1, red);
        W8A8_STAMP(1);
        fused::publish(a, r0 < r1);
        W8A8_STAMP(2);
        const int rows = min(T::BM, a.M - m0);
        const int producers = (rows + a.rows_per_wg - 1) / a.rows_per_wg;
        if (fused::wait_producers(a, m0 / a.rows_per_wg, producers, decision)) {
            fused::quantize_rows<T::THREADS, IN, FP8>(a, m0, m0 + rows, red);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    }

    W8A8_STAMP(3);

    // Scales (and bias) of the tile, fetched now into a couple of registers
    // per thread and parked in LDS for the epilogue, so that their latency
    // hides behind the K loop: entries [0, BN) ws, [BN, 2BN) bias as fp32
    // (zero without bias), [2BN, 2BN+BM) xs; rows/channels past M/N repeat
    // the last valid one.
    float side_v[T::SIDE_PER_THREAD];
    if (!OUT_I32) {
#pragma unroll
        for (int u = 0; u < T::SIDE_PER_THREAD; ++u) {
            const int p = u * T::THREADS + (int)threadIdx.x;
            float v = 0.0f;
            if (p < T::BN)
                v = a.ws[min(n0 + p, a.N - 1)];
            else if (p < 2 * T::BN) {
                if (a.bias) {
                    const unsigned b = a.bias[min(n0 + p - T::BN, a.N - 1)];
                    v = OUT_F16 ? quant_rule::f16_to_float(b) : __uint_as_float(b << 16);
                }
            } else if (p < T::SIDE)
                v = a.xs[min(m0 + p - 2 * T::BN, a.M - 1)];
            side_v[u] = v;
        }
    }

    // Prologue: the weights of the stages before the first virtual step's,
    // stage 0's images, then the loads that steps -LT .. -1 would have
    // issued, then stage 0's operands into xf[0]. Every load is issued even
    // when its stage does not exist (its addresses are clamped and its LDS
    // stage is never read), so the load counter state at the loop entry
    // matches the one at the back-edge. Stage 0 has landed once no more than
    // the virtual steps' loads are in flight.
    if constexpr (!T::WLDS)
        static_for<T::LW - T::LT>([&](auto U) __attribute__((always_inline)) {
            constexpr int t = decltype(U)::value;
            load_b(t, bq[t % T::NB]);
        });
    dma(0);
    static_for<T::LT>([&](auto U) __attribute__((always_inline)) {
        constexpr int v = decltype(U)::value - T::LT;  // virtual step -LT .. -1
        dma(v + 1 + T::LT);
        if constexpr (!T::WLDS)
            load_b(v + T::LW, bq[(v + T::LW) % T::NB]);
    });
    wait_vm_lgkm0<T::LT * T::LPW>();
    __builtin_amdgcn_s_barrier();
    read(0, xf[0]);
    if constexpr (T::WLDS)
        bread(0, bf[0]);

    W8A8_STAMP(4);

    // Steady state: GROUP unconditional steps while every stage they fetch
    // exists.
    int s0 = 0;
    for (; s0 + T::GROUP + T::AHEAD <= S; s0 += T::GROUP) {
        static_for<T::GROUP>([&](auto U) __attribute__((always_inline)) {
            step(Full{}, s0 + decltype(U)::value, U);
        });
    }
    // Tail: fewer than GROUP + AHEAD stages, each step guarded.
    static_for<T::GROUP + T::AHEAD>([&](auto U) __attribute__((always_inline)) {
        if (s0 + decltype(U)::value < S)
            step(Part{}, s0 + decltype(U)::value, U);
    });

    W8A8_STAMP(5);

    // ---- epilogue ----
    // Accumulator layout: acc[j][i] register 4q+r of lane l holds channel
    // n = 32*(wn*FN+j) + 8q + 4*(l/32) + r and token m = 32*i + l%32 of the tile.
    // k-group wk finishes row tiles i in [wk*FMH, (wk+1)*FMH): it receives the
    // other k-group's partial sums of those through LDS and hands over its own
    // partial sums of the rest, so all four waves share the scaling and stores.
    constexpr int FMH = T::FM / T::WK;
    // The accumulator registers of a wave's rows must be named at compile
    // time, so the epilogue is instantiated once per k-group.
    auto epilogue = [&](auto wk_c) __attribute__((always_inline)) {
        constexpr int WKI = decltype(wk_c)::value;
        constexpr int i0 = WKI * FMH;
        float *side = reinterpret_cast<float *>(reinterpret_cast<char *>(lds) + T::MAIN);
        const bool has_bias = !OUT_I32 && a.bias != nullptr;
        if (!OUT_I32) {
#pragma unroll
            for (int u = 0; u < T::SIDE_PER_THREAD; ++u) {
                const int p = u * T::THREADS + (int)threadIdx.x;
                if (p < T::SIDE)
                    side[p] = side_v[u];
            }
        }
        wait_vm_lgkm0<0>();                            // no image still landing in the ring
        __builtin_amdgcn_s_barrier();                  // every wave is done with the ring

        // Hand over the partial sums of the other k-group's rows: one 16-byte
        // slot per (j, i % FMH, q, lane) of each (row group, column group,
        // owner k-group).
        v4i *part = reinterpret_cast<v4i *>(lds);
        constexpr int PW = T::FN * FMH * 4 * 64;
        const int pbase = ((wm * T::WN + wn) * T::WK + WKI) * PW;
        if (T::WK > 1) {
#pragma unroll
            for (int i = 0; i < T::FM; ++i) {
                if (i / FMH == WKI)
                    continue;
#pragma unroll
                for (int j = 0; j < T::FN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        part[((wm * T::WN + wn) * T::WK + i / FMH) * PW + ((j * FMH + i % FMH) * 4 + q) * 64 + lane] =
                            quad_bits(acc[j][i], q);
                    }
            }
            wait_lgkm0();
            __builtin_amdgcn_s_barrier();
        }
        // The other k-group's partial sums of row tile i0+i of this wave, read
        // one row tile at a time (they are independent loads, issued together).
        auto partials = [&](int i, v4i (&pv)[T::FN][4]) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < T::FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    pv[j][q] = T::WK > 1 ? part[pbase + ((j * FMH + i) * 4 + q) * 64 + lane] : v4i{};
        };

        if (OUT_I32) {
            // Debug mode: raw int32 sums (fp32 sums in the e4m3 twin, as
            // their bits) straight from registers.
#pragma unroll
            for (int i = 0; i < FMH; ++i) {
                v4i pv[T::FN][4];
                partials(i, pv);
                const int m = m0 + wm * (T::BM / T::WM) + (i0 + i) * 32 + (lane & 31);
                if (m >= a.M)
                    continue;
#pragma unroll
                for (int j = 0; j < T::FN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int n = n0 + (wn * T::FN + j) * 32 + q * 8 + (lane >> 5) * 4;
                        if (n >= a.N)
                            continue;
                        const Acc &c = acc[j][i0 + i];
                        v4i v;
                        if constexpr (FP8)
                            v = __builtin_bit_cast(
                                v4i, __builtin_bit_cast(f32x4, quad_bits(c, q)) + __builtin_bit_cast(f32x4, pv[j][q]));
                        else
                            v = quad_bits(c, q) + pv[j][q];
                        int *o = reinterpret_cast<int *>(a.out) + (int64_t)m * a.ldo + n;
                        if (a.vec_store && n + 3 < a.N) {
                            *reinterpret_cast<v4i *>(o) = v;
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (n + r < a.N)
                                    o[r] = v[r];
                        }
                    }
            }
            return;
        }

        // bf16 output. Scales of this wave's columns and rows from LDS, then
        // the epilogue's fixed order per output: acc * xs, then * ws, then
        // + bias, each step rounded to fp32, and a round-to-nearest-even pair
        // conversion to bf16. The BM x BN bf16 tile is staged in LDS (its own
        // region, row pitch BN*2+16 bytes) ...
        f32x4 w4[T::FN][4];
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                w4[j][q] = *reinterpret_cast<const f32x4 *>(side + (wn * T::FN + j) * 32 + q * 8 + (lane >> 5) * 4);
        char *tile_lds = reinterpret_cast<char *>(lds) + T::TILE_OFF;
        auto scale = [&](auto with_bias) __attribute__((always_inline)) {
            constexpr bool B = decltype(with_bias)::value;
#pragma unroll
            for (int i = 0; i < FMH; ++i) {
                v4i pv[T::FN][4];
                partials(i, pv);
                const int ml = wm * (T::BM / T::WM) + (i0 + i) * 32 + (lane & 31);
                const float xr = side[2 * T::BN + ml];
#pragma unroll
                for (int j = 0; j < T::FN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int nl = (wn * T::FN + j) * 32 + q * 8 + (lane >> 5) * 4;
                        const f32x4 b4 = B ? *reinterpret_cast<const f32x4 *>(side + T::BN + nl) : f32x4{};
                        const Acc &c = acc[j][i0 + i];
                        float t[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            t[r] = acc_plus(c, 4 * q + r, pv[j][q][r]) * xr;
                            t[r] = t[r] * w4[j][q][r];
                            if (B)
                                t[r] = t[r] + b4[r];
                        }
                        *reinterpret_cast<v2u *>(tile_lds + ml * T::PITCH + nl * 2) =
                            pack4<OUT_F16>(t);
                    }
            }
        };
        if (has_bias)
            scale(std::true_type{});
        else
            scale(std::false_type{});
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();

        // ... then write whole rows: consecutive lanes store consecutive
        // pieces, so every store instruction fills complete cache lines. All
        // LDS reads are issued before the first store. A tile inside the
        // output with 16-byte aligned rows takes 16-byte pieces with
        // addresses stepped by a constant, as streaming (nontemporal) stores:
        // the tile goes out while later workgroups still compute instead of
        // waiting in L2 for the end of the launch (measured on MI355X: the
        // fused-QKV matmul 2.5 % faster, the other shapes level); other tiles
        // go piece by piece.
        constexpr int P16 = T::BN / 8;                 // 16-byte pieces per row
        constexpr int RPP = T::THREADS / P16;          // rows per pass
        constexpr int PASSES = (T::BM + RPP - 1) / RPP;
        if (a.vec16 && m0 + T::BM <= a.M && n0 + T::BN <= a.N) {
            const int t = threadIdx.x;
            if (t < RPP * P16) {
                const int r0 = t / P16, c = t % P16;
                v4u val[PASSES];
#pragma unroll
                for (int ps = 0; ps < PASSES; ++ps)
                    if (T::BM % RPP == 0 || r0 + ps * RPP < T::BM)
                        val[ps] = *reinterpret_cast<const v4u *>(tile_lds + (r0 + ps * RPP) * T::PITCH + c * 16);
                uint16_t *o = reinterpret_cast<uint16_t *>(a.out) + (int64_t)(m0 + r0) * a.ldo + n0 + c * 8;
                const int64_t step = (int64_t)RPP * a.ldo;
#pragma unroll
                for (int ps = 0; ps < PASSES; ++ps)
                    if (T::BM % RPP == 0 || r0 + ps * RPP < T::BM)
                        __builtin_nontemporal_store(val[ps], reinterpret_cast<v4u *>(o + ps * step));
            }
            return;
        }
        constexpr int QPR = T::BN / 4;                 // 8-byte pieces per row
        for (int p = threadIdx.x; p < T::BM * QPR; p += T::THREADS) {
            const int m = m0 + p / QPR, n = n0 + (p % QPR) * 4;
            if (m >= a.M || n >= a.N)
                continue;
            const v2u v = *reinterpret_cast<const v2u *>(tile_lds + (p / QPR) * T::PITCH + (p % QPR) * 8);
            uint16_t *o = reinterpret_cast<uint16_t *>(a.out) + (int64_t)m * a.ldo + n;
            if (a.vec_store && n + 3 < a.N) {
                *reinterpret_cast<v2u *>(o) = v;
            } else {
                const unsigned hv[4] = {v[0] & 0xffffu, v[0] >> 16, v[1] & 0xffffu, v[1] >> 16};
                for (int r = 0; r < 4; ++r)
                    if (n + r < a.N)
                        o[r] = (uint16_t)hv[r];
            }
        }
    };
    static_for<T::WK>([&](auto W) __attribute__((always_inline)) {
        if (wk == decltype(W)::value)
            epilogue(W);
    });
    W8A8_STAMP(6);
}

// The main kernel's tile configurations in tile-number order (the int8
// kernel and its e4m3 twin use the same list): BM x BN output tile / WM row
// groups x WN column groups x WK k-groups of waves / token and weight fetch
// leads in stages ("l3lds": weights through LDS with the tokens, three
// stages ahead; measured on MI355X 6-9 % faster than fetching them straight
// into registers, where the two row groups each load every fragment). The
// 256x256 tile takes all 512 registers of a lane (256 of them accumulators;
// its epilogue spills 8 bytes) and 138 KB of LDS; it reads the fewest L2
// bytes per MFMA op of the list and wins on large shapes whose tiles fill
// whole rounds of 256 CUs.
using MainTiles = std::tuple<Tile<64, 64, 1, 2, 2, 3, 3>, Tile<64, 128, 1, 2, 2, 3, 3, false, 2>,
                             Tile<128, 64, 1, 2, 2, 3, 3, false, 3>, Tile<128, 128, 1, 2, 2, 3, 3>,
                             Tile<128, 192, 1, 2, 2, 3, 3>, Tile<256, 128, 2, 2, 1, 3, 3, true, 2>,
                             Tile<256, 192, 2, 2, 1, 3, 3, true>, Tile<256, 256, 2, 2, 1, 3, 3, true>>;
constexpr const char *kMainTileNames[] = {
    "64x64/m1n2k2/l33",   "64x128/m1n2k2/l33",    "128x64/m1n2k2/l33",    "128x128/m1n2k2/l33",
    "128x192/m1n2k2/l33", "256x128/m2n2k1/l3lds", "256x192/m2n2k1/l3lds", "256x256/m2n2k1/l3lds"};
constexpr int kNumMainTiles = (int)std::tuple_size<MainTiles>::value;
static_assert(sizeof(kMainTileNames) / sizeof(kMainTileNames[0]) == kNumMainTiles, "tile names");

// A table of TileEntry, one per main tile, built by Make<T>(name).
template <template <class> class Make, size_t... I>
constexpr std::array<TileEntry, sizeof...(I)> main_table(std::index_sequence<I...>)
{
    return {{Make<std::tuple_element_t<I, MainTiles>>::entry(kMainTileNames[I])...}};
}

}  // namespace
}  // namespace w8a8
