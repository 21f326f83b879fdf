// int8 x int8 -> int32 matmul with the fused scale epilogue, for gfx950.
//
// What it computes (page "Issue 5 probe: int8 quantized DiT serve paths on
// the RTX 3090 (24 GB)", "Round two" kernel-path paragraph; page "INT8 Quant
// for Dual-Max Recipe": int8 x int8 on the matrix cores, no dequantization):
//   acc[m,n] = sum_k xq[m,k] * wq[n,k]                    exact int32
//   out[m,n] = bf16_rne(fl(fl(fl(acc) * xs[m]) * ws[n]) [+ bias[n]])
// or the raw accumulators in the int32 debug mode.
//
// Design (a dense contraction: the int8 MFMA roofline bounds it):
//   - v_mfma_i32_16x16x64_i8. The weight fragment is the MFMA "A" operand
//     (16 output channels x 64 k) and the token fragment the "B" operand
//     (16 tokens x 64 k), so each lane's four accumulators are four
//     consecutive output channels of one token: the epilogue packs them
//     into one 8-byte bf16 store.
//   - A workgroup computes a BM x BN output tile with WM x WN wavefronts;
//     each wave owns (BM/WM) x (BN/WN) and keeps FM x FN accumulator tiles.
//   - The K loop moves KS 64-deep k-blocks per stage through LDS, double
//     buffered: the global loads of stage t+1 are in flight while stage t
//     feeds the MFMAs; one barrier per stage.
//   - LDS holds "fragment images": 1 KiB per 16 rows x 64 k, lane l's 16
//     bytes at offset 16*l. Token rows are gathered into that order on the
//     way in (lane l loads row l%16, k-chunk l/16: the same 64-byte row
//     pieces a plain row-major copy would touch), and the prepacked weight
//     already is in it. Every ds_write_b128 and ds_read_b128 is therefore
//     64 consecutive 16-byte slots: no bank conflicts, no swizzle.
//   - Workgroup ids are remapped so consecutive tiles (the M tiles that
//     share one N stripe of the weight) land on one XCD and share its L2.
// Ragged M, N and K tails are masked at the loads (zero fill) and stores.
#include "internal.hpp"

namespace w8a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

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

// 16-byte global load, or zeros when the fragment lies outside the operand.
__device__ __forceinline__ uint4 load_or_zero(bool ok, const uint4 *p)
{
    uint4 v = make_uint4(0, 0, 0, 0);
    if (ok)
        v = *p;
    return v;
}

template <int BM_, int BN_, int KS_, int WM_, int WN_>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, KS = KS_, WM = WM_, WN = WN_;
    static constexpr int NW = WM * WN;                 // wavefronts per workgroup
    static constexpr int THREADS = NW * 64;
    static constexpr int MB = BM / 16, NB = BN / 16;   // fragments per tile edge
    static constexpr int FM = MB / WM, FN = NB / WN;   // fragments per wave edge
    static constexpr int NA = MB * KS, NBW = NB * KS;  // fragment blocks per stage
    static constexpr int LA = NA / NW, LB = NBW / NW;  // blocks each wave loads
    static constexpr int STAGE = (NA + NBW) * 64;      // uint4 slots per stage
    static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "tile/wave mismatch");
    static_assert(NA % NW == 0 && NBW % NW == 0, "loads must split evenly over waves");
};

template <class T, bool OUT_I32>
__global__ __launch_bounds__(T::THREADS) void scaled_mm_kernel(const MmArgs a)
{
    __shared__ uint4 lds[2 * T::STAGE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / T::WN, wn = wave % T::WN;

    const int tiles_m = (a.M + T::BM - 1) / T::BM;
    const int tiles_n = (a.N + T::BN - 1) / T::BN;
    const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    const int tn = tile / tiles_m, tm = tile % tiles_m;
    const int m0 = tm * T::BM, n0 = tn * T::BN;

    // Per-lane global sources. Token block b = mb*KS + ks: row m0+16*mb+l%16,
    // k-chunk 16*(l/16) of k-block (stage*KS + ks).
    const int lrow = lane & 15, lkc = (lane >> 4) * 16;
    const int8_t *__restrict__ xq = a.xq;
    const uint4 *__restrict__ wp = reinterpret_cast<const uint4 *>(a.wp);

    uint4 ra[T::LA], rb[T::LB];

    auto gload = [&](int st) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < T::LA; ++i) {
            const int b = i * T::NW + wave;
            const int mb = b / T::KS, ks = b % T::KS;
            const int row = m0 + mb * 16 + lrow;
            const int kc = (st * T::KS + ks) * 64 + lkc;
            ra[i] = load_or_zero(row < a.M && kc < a.K,
                                 reinterpret_cast<const uint4 *>(xq + (int64_t)row * a.ldq + kc));
        }
#pragma unroll
        for (int i = 0; i < T::LB; ++i) {
            const int b = i * T::NW + wave;
            const int nb = b / T::KS, ks = b % T::KS;
            const int nblk = n0 / 16 + nb, kblk = st * T::KS + ks;
            rb[i] = load_or_zero(nblk < a.nblocks && kblk < a.kblocks,
                                 wp + ((int64_t)nblk * a.kblocks + kblk) * 64 + lane);
        }
    };
    auto lstore = [&](int buf) __attribute__((always_inline)) {
        uint4 *s = lds + buf * T::STAGE;
#pragma unroll
        for (int i = 0; i < T::LA; ++i)
            s[(i * T::NW + wave) * 64 + lane] = ra[i];
#pragma unroll
        for (int i = 0; i < T::LB; ++i)
            s[(T::NA + i * T::NW + wave) * 64 + lane] = rb[i];
    };

    v4i acc[T::FN][T::FM];
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
            acc[j][i] = v4i{0, 0, 0, 0};

    auto compute = [&](int buf) __attribute__((always_inline)) {
        const uint4 *s = lds + buf * T::STAGE;
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) {
            v4i xf[T::FM], wf[T::FN];
#pragma unroll
            for (int i = 0; i < T::FM; ++i) {
                const uint4 v = s[((wm * T::FM + i) * T::KS + ks) * 64 + lane];
                xf[i] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
            }
#pragma unroll
            for (int j = 0; j < T::FN; ++j) {
                const uint4 v = s[(T::NA + (wn * T::FN + j) * T::KS + ks) * 64 + lane];
                wf[j] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
            }
#pragma unroll
            for (int j = 0; j < T::FN; ++j)
#pragma unroll
                for (int i = 0; i < T::FM; ++i)
                    acc[j][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[j], xf[i], acc[j][i], 0, 0, 0);
        }
    };

    const int stages = (a.kblocks + T::KS - 1) / T::KS;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int st = 0; st < stages; ++st) {
        const int cur = st & 1;
        if (st + 1 < stages)
            gload(st + 1);
        compute(cur);
        if (st + 1 < stages)
            lstore(cur ^ 1);
        __syncthreads();
    }

    // Epilogue. acc[j][i] lane l: channel n = n0 + 16*(wn*FN+j) + 4*(l/16) + r,
    // token m = m0 + 16*(wm*FM+i) + l%16, r = 0..3.
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
        const int n = n0 + (wn * T::FN + j) * 16 + (lane >> 4) * 4;
        if (n >= a.N)
            continue;
        const bool full = a.vec_store && n + 3 < a.N;
        float ws4[4], b4[4];
        if (!OUT_I32) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool ok = n + r < a.N;
                ws4[r] = ok ? a.ws[n + r] : 0.0f;
                b4[r] = (ok && a.bias) ? __uint_as_float((unsigned)a.bias[n + r] << 16) : 0.0f;
            }
        }
#pragma unroll
        for (int i = 0; i < T::FM; ++i) {
            const int m = m0 + (wm * T::FM + i) * 16 + lrow;
            if (m >= a.M)
                continue;
            const v4i c = acc[j][i];
            if (OUT_I32) {
                int *o = reinterpret_cast<int *>(a.out) + (int64_t)m * a.ldo + n;
                if (full) {
                    *reinterpret_cast<int4 *>(o) = make_int4(c[0], c[1], c[2], c[3]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < a.N)
                            o[r] = c[r];
                }
            } else {
                const float xs = a.xs[m];
                unsigned h[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float t = (float)c[r] * xs;
                    t = t * ws4[r];
                    if (a.bias)
                        t = t + b4[r];
                    h[r] = bf16_bits(t);
                }
                uint16_t *o = reinterpret_cast<uint16_t *>(a.out) + (int64_t)m * a.ldo + n;
                if (full) {
                    *reinterpret_cast<uint2 *>(o) = make_uint2(h[0] | h[1] << 16, h[2] | h[3] << 16);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < a.N)
                            o[r] = (uint16_t)h[r];
                }
            }
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

// BM x BN x (64*KS) / WM x WN
const TileEntry kTiles[] = {
    entry<Tile<64, 64, 2, 2, 2>>("64x64x128/2x2"),
    entry<Tile<64, 128, 2, 2, 2>>("64x128x128/2x2"),
    entry<Tile<128, 64, 2, 2, 2>>("128x64x128/2x2"),
    entry<Tile<128, 128, 2, 2, 2>>("128x128x128/2x2"),
    entry<Tile<128, 192, 2, 2, 2>>("128x192x128/2x2"),
    entry<Tile<128, 256, 2, 2, 2>>("128x256x128/2x2"),
    entry<Tile<256, 128, 2, 2, 2>>("256x128x128/2x2"),
    entry<Tile<128, 128, 1, 2, 2>>("128x128x64/2x2"),
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
