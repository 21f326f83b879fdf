// The e4m3 (FP8) twin of the matmul: the main kernel (mm_kernel.hpp) with
// e4m3 operands and fp32 accumulation, over the same tile configurations
// as the int8 kernel (page "Online Quantization": FP8 W8A8 with dynamic
// activation scaling, the sibling of Int8 W8A8 in its method tables).
//   acc[m,n] = sum_k e4m3(xq[m,k]) * e4m3(wq[n,k])       (fp32 MFMA sums)
//   out[m,n] = 16-bit float of fl(fl(acc * xs[m]) * ws[n]) [+ bias[n]]
// The weight is prepacked exactly as the int8 weight (a byte permutation),
// with e4m3 codes in place of int8 ones. The tiles are the int8 ones, in the
// same order: the main kernel's here, then the small-M kernel's e4m3 twin
// (skinny_mm.hip); both have the fused quant forms of the int8 path.
#include "mm_kernel.hpp"

namespace w8a8 {
namespace {

template <class T>
struct Fp8Entry {
    static constexpr TileEntry entry(const char *name)
    {
        return TileEntry{name, T::BM, T::BN, T::THREADS, false,
                         {scaled_mm_kernel<T, kOutBF16, false, true>,
                          scaled_mm_kernel<T, kOutI32, false, true>,
                          scaled_mm_kernel<T, kOutF16, false, true>},
                         {scaled_mm_kernel<T, kOutBF16, true, true>,
                          scaled_mm_kernel<T, kOutI32, true, true>,
                          scaled_mm_kernel<T, kOutF16, true, true>}};
    }
};

const auto kFp8Tiles = main_table<Fp8Entry>(std::make_index_sequence<kNumMainTiles>{});

const TileEntry &fp8_entry(int tile)
{
    return tile < kNumMainTiles ? kFp8Tiles[tile] : skinny_tile_fp8(tile - kNumMainTiles);
}

// Keys of the e4m3 twin in the capacity cache come after the int8 tiles'
// (keys past the cache's size are simply not cached).
constexpr int kCapKeyBase = 16;

}  // namespace

int fp8_tile_count() { return kNumMainTiles + skinny_tile_count(); }

bool fp8_launch_fits(int tile, int64_t M, int64_t N)
{
    const TileEntry &e = fp8_entry(tile);
    return mm_grid_fits(ceil_div(M, e.bm) * ceil_div(N, e.bn), e.threads);
}

hipError_t launch_quant_scaled_mm_fp8(MmArgs a, int mode, int tile, hipStream_t stream)
{
    return launch_quant_scaled_mm_entry(a, mode, fp8_entry(tile), kCapKeyBase + tile, stream);
}

hipError_t launch_scaled_mm_fp8(const MmArgs &a, int mode, int tile, hipStream_t stream)
{
    const TileEntry &e = fp8_entry(tile);
    const int64_t tiles = ceil_div(a.M, e.bm) * ceil_div(a.N, e.bn);
    hipLaunchKernelGGL(e.plain[mode], dim3((unsigned)tiles), dim3(e.threads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace w8a8
