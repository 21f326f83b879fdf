// The e4m3 (FP8) twin of the matmul: the main kernel (mm_kernel.hpp) with
// e4m3 operands and fp32 accumulation, over the same tile configurations
// as the int8 kernel (page "Online Quantization": FP8 W8A8 with dynamic
// activation scaling, the sibling of Int8 W8A8 in its method tables).
//   acc[m,n] = sum_k e4m3(xq[m,k]) * e4m3(wq[n,k])       (fp32 MFMA sums)
//   out[m,n] = 16-bit float of fl(fl(acc * xs[m]) * ws[n]) [+ bias[n]]
// The weight is prepacked exactly as the int8 weight (a byte permutation),
// with e4m3 codes in place of int8 ones. No fused quant and no small-M
// configurations: int8_quant_scaled_mm's single-launch paths are int8 only.
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
                         {nullptr, nullptr, nullptr}};
    }
};

const auto kFp8Tiles = main_table<Fp8Entry>(std::make_index_sequence<kNumMainTiles>{});

}  // namespace

int fp8_tile_count() { return kNumMainTiles; }

hipError_t launch_scaled_mm_fp8(const MmArgs &a, int mode, int tile, hipStream_t stream)
{
    const TileEntry &e = kFp8Tiles[tile];
    const int64_t tiles = ceil_div(a.M, e.bm) * ceil_div(a.N, e.bn);
    hipLaunchKernelGGL(e.plain[mode], dim3((unsigned)tiles), dim3(e.threads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace w8a8
