// The int8 tile configurations of the main matmul kernel (mm_kernel.hpp),
// the automatic tile choice over them and the small-M configurations
// (skinny_mm.hip), and the launchers of int8_scaled_mm and the fused
// quant + matmul.
#include <algorithm>
#include <atomic>
#include <cmath>

#include "mm_kernel.hpp"

namespace w8a8 {
namespace {

template <class T>
struct Int8Entry {
    static constexpr TileEntry entry(const char *name)
    {
        return TileEntry{name, T::BM, T::BN, T::THREADS, false,
                         {scaled_mm_kernel<T, kOutBF16, false>, scaled_mm_kernel<T, kOutI32, false>,
                          scaled_mm_kernel<T, kOutF16, false>},
                         {scaled_mm_kernel<T, kOutBF16, true>, scaled_mm_kernel<T, kOutI32, true>,
                          scaled_mm_kernel<T, kOutF16, true>}};
    }
};

const auto kTiles = main_table<Int8Entry>(std::make_index_sequence<kNumMainTiles>{});
constexpr int kNumTiles = kNumMainTiles;

const TileEntry &tile_entry(int tile)
{
    return tile < kNumTiles ? kTiles[tile] : skinny_tile(tile - kNumTiles);
}

}  // namespace

const TileEntry &mm_tile_entry(int tile) { return tile_entry(tile); }

int mm_tile_count() { return kNumTiles + skinny_tile_count(); }

bool mm_launch_fits(int tile, int64_t M, int64_t N)
{
    const TileEntry &e = tile_entry(tile);
    return mm_grid_fits(ceil_div(M, e.bm) * ceil_div(N, e.bn), e.threads);
}

const char *mm_tile_name(int tile)
{
    return (tile >= 0 && tile < mm_tile_count()) ? tile_entry(tile).name : "";
}

// Automatic choice: the smallest modelled time (rates measured on MI355X
// under full load). Workgroups run in rounds of one per CU (256 CUs).
//   Main kernel: a tile costs the largest of its MFMA time, the time to
//   stream its operands from L2 and, where few row tiles share its weight
//   columns (small M), the time to stream its weight columns from HBM, plus
//   a fixed cost (prologue and epilogue). About 16000 int8 MFMA ops per ns
//   per CU (the shader clock drops to ~2 GHz), about 80 bytes per ns of L2
//   reads per CU (~20 TB/s in all), and about 22 bytes per ns per CU from
//   HBM for its four waves; the row tiles of one band (up to 4) share each
//   weight fetch.
//   Small-M kernel, for up to 32 token rows (beyond that each weight byte
//   meets enough tokens for the main kernel's tiles): the weight stream, at
//   about 38 bytes per ns from HBM per busy CU, in rounds (each tile streams
//   its BN weight columns over all of K), or the L2 reads of all workgroups
//   if more: each k-block brings the weight fragments and one 128-byte line
//   per token row, ~16 TB/s in all; plus a fixed cost. Fitted on MI355X to
//   the measured best tile of nine decode shapes (M 1-32, N 3072-12288, K
//   4096-12288, weights streamed from HBM), all within 0.5 % of the best.
int mm_tile_auto(int64_t M, int64_t N, int64_t K)
{
    const double cus = 256.0;
    const double kk = (double)round_up(K, 64), kblocks = kk / 64.0;
    int best = 0;
    double best_cost = 1e300;
    for (int t = 0; t < mm_tile_count(); ++t) {
        const TileEntry &e = tile_entry(t);
        if (e.skinny && M > 32)
            continue;
        const int64_t tiles_m = ceil_div(M, e.bm);
        const int64_t tiles = tiles_m * ceil_div(N, e.bn);
        const double rounds = std::ceil((double)tiles / cus);
        double cost;
        if (!e.skinny) {
            const double t_mma = 2.0 * e.bm * e.bn * kk / 16000.0;
            const double t_l2 = (double)(e.bm + e.bn) * kk / 80.0;
            const double t_hbm = (double)e.bn * kk / (double)std::min<int64_t>(tiles_m, 4) / 22.0;
            cost = rounds * (std::max({t_mma, t_l2, t_hbm}) + 3000.0);
        } else {
            const double t_hbm = rounds * (double)e.bn * kk / 38.0;
            const double rows = (double)std::min<int64_t>(M, e.bm);
            const double t_l2 = (double)tiles * kblocks * (e.bn / 16 * 1024.0 + rows * 128.0) / 16000.0;
            cost = std::max(t_hbm, t_l2) + 3000.0;
        }
        if (cost < best_cost * 0.999) {
            best_cost = cost;
            best = t;
        }
    }
    return best;
}

hipError_t launch_scaled_mm(const MmArgs &a, int mode, int tile, hipStream_t stream)
{
    const TileEntry &e = tile_entry(tile);
    const int64_t tiles = ceil_div(a.M, e.bm) * ceil_div(a.N, e.bn) *
                          (e.skinny && a.ksplit > 1 ? a.ksplit : 1);
    const int threads = e.threads;
    hipLaunchKernelGGL(e.plain[mode], dim3((unsigned)tiles), dim3(threads), 0, stream, a);
    return hipGetLastError();
}

// Workgroups of a fused kernel that the device holds at once (CUs times
// occupancy), per device, tile and output mode; 0 until first asked. The
// runtime's occupancy query costs tens of microseconds, far more than the
// small launches this path serves, so it runs once.
constexpr int kCapDevices = 64, kCapTiles = 32;
static std::atomic<int> g_capacity[kCapDevices][kCapTiles][3];

static hipError_t fused_capacity(int dev, int tile, int mode, MmKernel fn, int threads, int &cap)
{
    const bool cached = dev >= 0 && dev < kCapDevices && tile < kCapTiles;
    if (cached && (cap = g_capacity[dev][tile][mode].load(std::memory_order_relaxed)) > 0)
        return hipSuccess;
    int cus = 0, per_cu = 0;
    hipError_t err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err == hipSuccess)
        err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(fn),
                                                           threads, 0);
    if (err != hipSuccess)
        return err;
    cap = cus * per_cu;
    if (cached && cap > 0)
        g_capacity[dev][tile][mode].store(cap, std::memory_order_relaxed);
    return hipSuccess;
}

namespace {
std::atomic<unsigned> g_wait_limit{fused::kDefaultWaitLimit};
}  // namespace

unsigned set_fused_wait_limit(unsigned polls) { return g_wait_limit.exchange(polls); }

unsigned fused_wait_limit() { return g_wait_limit.load(); }

hipError_t launch_quant_scaled_mm(MmArgs a, int mode, int tile, hipStream_t stream)
{
    return launch_quant_scaled_mm_entry(a, mode, tile_entry(tile), tile, stream);
}

hipError_t launch_quant_scaled_mm_entry(MmArgs a, int mode, const TileEntry &e, int cap_key,
                                        hipStream_t stream)
{
    const int64_t tiles = ceil_div(a.M, e.bm) * ceil_div(a.N, e.bn);
    MmKernel fn = e.fused[mode];
    if (fn == nullptr)
        return hipErrorNotSupported;
    if (e.skinny)
        return launch_skinny_quant_mm(a, e, mode, stream);
    // Rows per workgroup: enough to cover M with one workgroup per tile,
    // rounded up to a power of two so that it divides BM.
    int rpw = 1;
    while ((int64_t)rpw * tiles < a.M)
        rpw *= 2;
    if (e.bm % rpw != 0 || ceil_div(a.M, rpw) > fused::kMaxProducers)
        return hipErrorNotSupported;
    // Consumers read the codes and scales of their own row tile with plain
    // loads once its producers have published, with no cache invalidation.
    // That is only sound when no cache line holds rows of two row tiles: a
    // consumer could otherwise pull in (and its XCD's L2 keep) a line whose
    // other part a later producer still has to write. A row tile's codes
    // span BM * ldq bytes (a multiple of 1024) and its scales BM * 4 (a
    // multiple of 256), so bases aligned to kFusedAlign keep every tile on
    // whole lines; other buffers take the two launches.
    if (reinterpret_cast<uintptr_t>(a.xq) % fused::kFusedAlign != 0 ||
        reinterpret_cast<uintptr_t>(a.xs) % fused::kFusedAlign != 0)
        return hipErrorNotSupported;
    // The flags carry an epoch fixed when the launch is made. A captured graph
    // would replay one epoch forever, and a replay could then take the flags
    // its predecessor raised for its own rows; so under stream capture the
    // caller runs the two launches instead.
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    hipError_t err = hipStreamIsCapturing(stream, &capture);
    if (err != hipSuccess)
        return err;
    if (capture != hipStreamCaptureStatusNone)
        return hipErrorNotSupported;
    int dev = 0;
    err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return err;
    // Every workgroup waits for rows that other workgroups produce, so the
    // path is only taken when the whole grid fits the device at once at this
    // kernel's occupancy. (A cooperative launch would guarantee residency,
    // but costs tens of microseconds on this runtime; the bounded wait with
    // its own-rows fallback keeps an ordinary launch correct even where the
    // grid does not all run at once.)
    int cap = 0;
    err = fused_capacity(dev, cap_key, mode, fn, e.threads, cap);
    if (err != hipSuccess)
        return err;
    if (tiles > cap)
        return hipErrorNotSupported;
    a.rows_per_wg = rpw;
    // A fresh epoch per launch on this device (0 is the flags' initial value).
    static std::atomic<unsigned> epochs[64];
    std::atomic<unsigned> &ep = epochs[dev & 63];
    unsigned v = ++ep;
    if (v == 0)
        v = ++ep;
    a.epoch = v;
    a.wait_limit = g_wait_limit.load();
    hipLaunchKernelGGL(fn, dim3((unsigned)tiles), dim3(e.threads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace w8a8

#ifdef W8A8_TIMELINE
// Measurement builds only (libw8a8_timeline.so): copies the first `bytes`
// bytes of the int8 kernels' timeline records (timeline.hpp) on the current
// device to host memory `dst`, synchronously; returns the hipError_t.
extern "C" __attribute__((visibility("default"))) int w8a8_timeline_read(void *dst, size_t bytes)
{
    if (bytes > sizeof(w8a8::timeline::g_stamp))
        return (int)hipErrorInvalidValue;
    return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(w8a8::timeline::g_stamp), bytes, 0,
                                    hipMemcpyDeviceToHost);
}
#endif
