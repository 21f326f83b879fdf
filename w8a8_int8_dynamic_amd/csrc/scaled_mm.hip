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
//     so weights skip LDS entirely: each wave loads its operands straight
//     from the prepacked weight into a ring of NS register sets (each load
//     is 64 lanes x 16 bytes in four contiguous 256-byte runs).
//   - Token rows are shared by the WN waves of a k-group, so they go
//     through LDS: a ring of NS stages (WK k-blocks each). Every load is an
//     ordinary global load the compiler tracks: token data is fetched NS-1
//     stages ahead into a small register staging ring and written to LDS
//     (ds_write_b128) one stage before use; one barrier per stage. (Direct
//     global->LDS loads were tried: the compiler either drains them with a
//     full vmcnt(0) before each LDS read, or, issued from inline asm, loses
//     count of them and over-waits on the weight loads.)
//   - A 16-row x 64-k token image is loaded with lane 4r+j reading k-chunk
//     j ^ swz(r) of row r and storing it to slot 4r+j: every 4-lane quad reads one row's 64 contiguous
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
#include <type_traits>
#include <utility>

#include "internal.hpp"

namespace w8a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kXcds = 8;

// Physical workgroup id -> logical tile id such that each XCD (which takes
// ids pid % 8 round-robin) receives one contiguous run of logical ids.
__device__ __forceinline__ int xcd_remap(int pid, int tiles)
{
    const int q = tiles / kXcds, r = tiles % kXcds;
    const int xcd = pid % kXcds, local = pid / kXcds;
    return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

__device__ __forceinline__ unsigned bf16_bits(float f)
{
    return (unsigned)__builtin_bit_cast(unsigned short, (__bf16)f);   // RNE
}

// s_waitcnt lgkmcnt(0) only (vmcnt and expcnt untouched; gfx9 encoding):
// this wave's LDS reads and writes have completed.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F & ~0x0F00); }

// s_waitcnt for everything.
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }

// s_waitcnt vmcnt(VM) lgkmcnt(0).
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0()
{
    static_assert(VM >= 0 && VM < 64, "vmcnt out of range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));
}

__device__ __forceinline__ int tok_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

__device__ __forceinline__ v4i as_v4i(const uint4 &v)
{
    return v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
}

constexpr int cmax(int a, int b) { return a > b ? a : b; }

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

template <int BM_, int BN_, int WN_, int WK_, int NS_>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, WN = WN_, WK = WK_, NS = NS_;
    static constexpr int NW = WN * WK;                 // wavefronts per workgroup
    static constexpr int THREADS = NW * 64;
    static constexpr int MB = BM / 16;                 // 16-row token images per k-block
    static constexpr int FM = BM / 32;                 // 32x32 MFMA tiles per wave, rows
    static constexpr int FN = BN / WN / 32;            // ... and columns
    static constexpr int AIMG = WK * MB;               // token images per stage
    static constexpr int LA = AIMG / NW;               // token DMA loads per wave per stage
    static constexpr int LB = 2 * FN;                  // weight loads per wave per stage
    static constexpr int LPW = LA + LB;                // global loads per wave per stage
    static constexpr int STAGE = AIMG * 64;            // uint4 slots per ring stage
    static constexpr int RING = NS * STAGE * 16;       // bytes
    static constexpr int PART = (WK - 1) * BM * BN * 4;     // k-group partial sums
    static constexpr int PITCH = BN * 2 + 8;           // staged bf16 row, bytes
    static constexpr int OUTB = BM * PITCH;
    static constexpr int LDS = cmax(RING, cmax(PART, OUTB));
    static_assert(NW == 4, "four wavefronts per workgroup");
    static_assert(BM % 32 == 0 && BN % (32 * WN) == 0, "tile/wave mismatch");
    static_assert(AIMG % NW == 0, "token loads must split evenly over waves");
    static_assert(NS == 3 || NS == 4, "pipeline depth: 3 or 4 stages");
    static_assert(LA * 0 + (2 * (BN / WN / 32) + (WK * (BM / 16)) / (WN * WK)) * (NS - 2) < 64,
                  "vmcnt range");
    static constexpr int NA = NS - 2;                  // token staging register sets
    static constexpr int GROUP = NS == 4 ? 4 : 3;      // lcm(NS, NA): steps per unrolled group
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert(FM * FN * 16 <= 256, "accumulators must fit the AGPR file");
};

template <class T, bool OUT_I32>
__global__ __launch_bounds__(T::THREADS) void scaled_mm_kernel(const MmArgs a)
{
    __shared__ uint4 lds[T::LDS / 16];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave % T::WN, wk = wave / T::WN;

    const int tiles_m = (a.M + T::BM - 1) / T::BM;
    const int tiles_n = (a.N + T::BN - 1) / T::BN;
    const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    const int tn = tile / tiles_m, tm = tile % tiles_m;
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

    v16i acc[T::FN][T::FM];
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
            acc[j][i] = v16i{};
    v4i bq[T::NS][T::FN][2];                           // weight operand ring
    v4i ast[T::NA][T::LA];                             // token staging ring
    v4i xf[T::FM][2];                                  // token operands of one stage

    // Global loads of stage t: token rows into staging set t % NA, weights
    // into ring set t % NS.
    auto load = [&](int t, v4i (&aset)[T::LA], v4i (&bset)[T::FN][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < T::LA; ++i) {
            const int kc = min((t * T::WK + aks[i]) * 64 + dchunk, klast);
            aset[i] = *reinterpret_cast<const v4i *>(arow[i] + kc);
        }
        const int kb = min(t * T::WK + wk, kblast);
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                bset[j][h] = bsrc[j][(int64_t)kb * 64 + h * 32];
    };
    // Token rows of stage t from staging registers into LDS ring buffer t % NS.
    auto store = [&](int t, const v4i (&aset)[T::LA]) __attribute__((always_inline)) {
        v4i *st = reinterpret_cast<v4i *>(lds) + (t % T::NS) * T::STAGE;
#pragma unroll
        for (int i = 0; i < T::LA; ++i)
            st[(i * T::NW + wave) * 64 + lane] = aset[i];
    };

    // One stage s: barrier (stage s is in LDS and stage s-2's buffer is
    // free), move stage s+1 into LDS, fetch stage s+NS-1, read this wave's
    // token operands of stage s, run its MFMAs. In the steady state (FULL)
    // every step is unconditional.
    auto step = [&](auto full, int s, v4i (&anext)[T::LA], v4i (&bcur)[T::FN][2],
                    v4i (&bnext)[T::FN][2]) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full)::value;
        // Stage s's weights were fetched NS-1 steps ago; LPW*(NS-2) loads of
        // later stages may still be in flight. (Stated explicitly: at the
        // loop back-edge the compiler's own count otherwise degrades to a
        // full drain.)
        if (FULL)
            wait_vm_lgkm0<T::LPW * (T::NS - 2)>();
        else
            wait_lgkm0();
        __builtin_amdgcn_s_barrier();
        if (FULL || s + 1 < S)
            store(s + 1, anext);
        if (FULL || s + T::NS - 1 < S)
            load(s + T::NS - 1, anext, bnext);
        const v4i *st = reinterpret_cast<const v4i *>(lds) + (s % T::NS) * T::STAGE + wk * T::MB * 64;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
                xf[i][h] = st[(2 * i) * 64 + xslot[h]];
        if (FULL || s * T::WK + wk < a.kblocks) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int j = 0; j < T::FN; ++j)
#pragma unroll
                    for (int i = 0; i < T::FM; ++i)
                        acc[j][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bcur[j][h], xf[i][h],
                                                                          acc[j][i], 0, 0, 0);
        }
        // Keep each step's loads in program order relative to the next
        // step, so the load counter state at the loop back-edge matches the
        // prologue's and the compiler's waits stay exact.
        __builtin_amdgcn_sched_barrier(0);
    };
    using Full = std::integral_constant<bool, true>;
    using Part = std::integral_constant<bool, false>;

    // Prologue: stage 0 into LDS; stages 1 .. NS-2 in flight.
    load(0, ast[0], bq[0]);
    store(0, ast[0]);
    static_for<T::NS - 2>([&](auto U) __attribute__((always_inline)) {
        constexpr int t = decltype(U)::value + 1;
        if (t < S)
            load(t, ast[t % T::NA], bq[t]);
    });
    // Steady state: groups of GROUP steps whose loads (stage s+NS-1 < S)
    // and k-blocks (stage s < S-1) all exist. Step s moves stage s+1 out of
    // staging set (s+1) % NA and refills that same set with stage s+NS-1.
    int s0 = 0;
    for (; s0 + T::GROUP + T::NS - 1 <= S; s0 += T::GROUP) {
        static_for<T::GROUP>([&](auto U) __attribute__((always_inline)) {
            constexpr int u = decltype(U)::value;
            step(Full{}, s0 + u, ast[(u + 1) % T::NA], bq[u % T::NS], bq[(u + T::NS - 1) % T::NS]);
        });
    }
    // Tail: fewer than GROUP + NS - 1 stages, each guarded.
    static_for<T::GROUP + T::NS - 1>([&](auto U) __attribute__((always_inline)) {
        constexpr int u = decltype(U)::value;
        if (s0 + u < S)
            step(Part{}, s0 + u, ast[(u + 1) % T::NA], bq[u % T::NS], bq[(u + T::NS - 1) % T::NS]);
    });

    // ---- epilogue ----
    // Accumulator layout: acc[j][i] register 4q+r of lane l holds channel
    // n = 32*(wn*FN+j) + 8q + 4*(l/32) + r and token m = 32*i + l%32 of the tile.
    wait_all();
    __builtin_amdgcn_s_barrier();                      // ring fully consumed
    if (T::WK > 1) {
        uint4 *part = lds;
        constexpr int PW = T::FN * T::FM * 4 * 64;     // uint4 slots per wave's partials
        if (wk > 0) {
#pragma unroll
            for (int j = 0; j < T::FN; ++j)
#pragma unroll
                for (int i = 0; i < T::FM; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const v16i &c = acc[j][i];
                        part[((wk - 1) * T::WN + wn) * PW + ((j * T::FM + i) * 4 + q) * 64 + lane] =
                            make_uint4(c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]);
                    }
        }
        wait_all();
        __builtin_amdgcn_s_barrier();
        if (wk == 0) {
#pragma unroll
            for (int g = 1; g < T::WK; ++g)
#pragma unroll
                for (int j = 0; j < T::FN; ++j)
#pragma unroll
                    for (int i = 0; i < T::FM; ++i)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const uint4 v =
                                part[((g - 1) * T::WN + wn) * PW + ((j * T::FM + i) * 4 + q) * 64 + lane];
                            acc[j][i][4 * q] += (int)v.x;
                            acc[j][i][4 * q + 1] += (int)v.y;
                            acc[j][i][4 * q + 2] += (int)v.z;
                            acc[j][i][4 * q + 3] += (int)v.w;
                        }
        }
        wait_all();
        __builtin_amdgcn_s_barrier();                  // partials consumed: LDS reusable
    }

    if (OUT_I32) {
        // Debug mode: raw accumulators straight from registers.
        if (wk == 0) {
#pragma unroll
            for (int j = 0; j < T::FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = n0 + (wn * T::FN + j) * 32 + q * 8 + (lane >> 5) * 4;
                    if (n >= a.N)
                        continue;
                    const bool full = a.vec_store && n + 3 < a.N;
#pragma unroll
                    for (int i = 0; i < T::FM; ++i) {
                        const int m = m0 + i * 32 + (lane & 31);
                        if (m >= a.M)
                            continue;
                        const v16i &c = acc[j][i];
                        int *o = reinterpret_cast<int *>(a.out) + (int64_t)m * a.ldo + n;
                        if (full) {
                            *reinterpret_cast<int4 *>(o) =
                                make_int4(c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]);
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (n + r < a.N)
                                    o[r] = c[4 * q + r];
                        }
                    }
                }
        }
        return;
    }

    // bf16 output: scale in registers, stage the BM x BN tile in LDS (row
    // pitch BN*2+8 bytes keeps the 8-byte writes of 32 rows on distinct
    // banks), then write whole rows: consecutive lanes store consecutive
    // 8-byte pieces, so every store instruction fills complete cache lines.
    char *tile_lds = reinterpret_cast<char *>(lds);
    if (wk == 0) {
#pragma unroll
        for (int i = 0; i < T::FM; ++i) {
            const int ml = i * 32 + (lane & 31);
            const float xs = a.xs[min(m0 + ml, a.M - 1)];
#pragma unroll
            for (int j = 0; j < T::FN; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int nl = (wn * T::FN + j) * 32 + q * 8 + (lane >> 5) * 4;
                    const v16i &c = acc[j][i];
                    unsigned h[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int nn = min(n0 + nl + r, a.N - 1);
                        float t = (float)c[4 * q + r] * xs;
                        t = t * a.ws[nn];
                        if (a.bias)
                            t = t + __uint_as_float((unsigned)a.bias[nn] << 16);
                        h[r] = bf16_bits(t);
                    }
                    *reinterpret_cast<uint2 *>(tile_lds + ml * T::PITCH + nl * 2) =
                        make_uint2(h[0] | h[1] << 16, h[2] | h[3] << 16);
                }
            }
        }
    }
    wait_all();
    __builtin_amdgcn_s_barrier();
    constexpr int QPR = T::BN / 4;                     // 8-byte pieces per row
    for (int p = threadIdx.x; p < T::BM * QPR; p += T::THREADS) {
        const int ml = p / QPR, nl = (p % QPR) * 4;
        const int m = m0 + ml, n = n0 + nl;
        if (m >= a.M || n >= a.N)
            continue;
        const uint2 v = *reinterpret_cast<const uint2 *>(tile_lds + ml * T::PITCH + nl * 2);
        uint16_t *o = reinterpret_cast<uint16_t *>(a.out) + (int64_t)m * a.ldo + n;
        if (a.vec_store && n + 3 < a.N) {
            *reinterpret_cast<uint2 *>(o) = v;
        } else {
            const unsigned hv[4] = {v.x & 0xffffu, v.x >> 16, v.y & 0xffffu, v.y >> 16};
            for (int r = 0; r < 4; ++r)
                if (n + r < a.N)
                    o[r] = (uint16_t)hv[r];
        }
    }
}

typedef void (*MmFn)(const MmArgs);

struct TileEntry {
    const char *name;
    int bm, bn;
    MmFn bf16, i32;
};

template <class T>
constexpr TileEntry entry(const char *name)
{
    return TileEntry{name, T::BM, T::BN, scaled_mm_kernel<T, false>, scaled_mm_kernel<T, true>};
}

// BM x BN output tile / WN column groups x WK k-groups of waves / NS stages
const TileEntry kTiles[] = {
    entry<Tile<64, 64, 2, 2, 4>>("64x64/n2k2/s4"),
    entry<Tile<64, 128, 2, 2, 4>>("64x128/n2k2/s4"),
    entry<Tile<128, 64, 2, 2, 4>>("128x64/n2k2/s4"),
    entry<Tile<128, 128, 2, 2, 4>>("128x128/n2k2/s4"),
    entry<Tile<128, 192, 2, 2, 3>>("128x192/n2k2/s3"),
    entry<Tile<128, 192, 2, 2, 4>>("128x192/n2k2/s4"),
};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

}  // namespace

int mm_tile_count() { return kNumTiles; }

const char *mm_tile_name(int tile)
{
    return (tile >= 0 && tile < kNumTiles) ? kTiles[tile].name : "";
}

// Automatic choice: fewest full-machine rounds of tiles, weighted by how
// much output each round covers and a penalty for the higher load traffic
// per op of small tiles.
int mm_tile_auto(int64_t M, int64_t N, int64_t K)
{
    (void)K;
    const int cus = 256;
    int best = 0;
    double best_cost = 1e300;
    for (int t = 0; t < kNumTiles; ++t) {
        const TileEntry &e = kTiles[t];
        const int64_t tiles = ceil_div(M, e.bm) * ceil_div(N, e.bn);
        const double rounds = (double)ceil_div(tiles, cus);
        const double per_op = 1.0 + 48.0 / e.bm + 48.0 / e.bn;
        const double cost = rounds * e.bm * e.bn * per_op;
        if (cost < best_cost) {
            best_cost = cost;
            best = t;
        }
    }
    return best;
}

hipError_t launch_scaled_mm(const MmArgs &a, bool out_i32, int tile, hipStream_t stream)
{
    const TileEntry &e = kTiles[tile];
    const int64_t tiles = ceil_div(a.M, e.bm) * ceil_div(a.N, e.bn);
    const int threads = 256;
    hipLaunchKernelGGL(out_i32 ? e.i32 : e.bf16, dim3((unsigned)tiles), dim3(threads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace w8a8
