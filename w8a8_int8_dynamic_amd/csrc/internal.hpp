// Internal declarations shared by the HIP translation units of libw8a8.
// Not part of the public ABI (include/w8a8.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

// Sizes of the prepacked weight fragments (see int8_prepack_weight).
constexpr int kFragN = 16;      // output channels per fragment
constexpr int kFragK = 64;      // reduction elements per fragment
constexpr int kFragBytes = 1024;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// A launch's workgroups times threads per workgroup must fit in 32 bits.
// Launchers whose grid grows with the data split it into launches of at
// most this many workgroups (2^30 threads at 256 per workgroup); the matmul
// launchers, whose grid is fixed by the tile, report a grid that cannot fit
// (mm_grid_fits).
constexpr int64_t kMaxBlocksPerLaunch = int64_t(1) << 22;
inline bool mm_grid_fits(int64_t workgroups, int threads)
{
    return workgroups <= INT32_MAX && workgroups * threads <= (int64_t)UINT32_MAX;
}

// Element kinds of rows and outputs (the quant rule's kBF16 / kF32 / kF16).
constexpr int kElemBF16 = 0, kElemF32 = 1, kElemF16 = 2;

// ---- per-row quantization (quant.hip) ----
// kind: x is bf16 bits, fp32 or fp16 bits [rows, ldx]. fp8: e4m3 codes
// (bf16 or fp32 rows only) instead of int8. keep_codes: the codes are read
// by the next launch, so they are stored to stay in the caches (activation
// rows only; otherwise they are streamed out).
hipError_t launch_quant_rows(const void *x, int kind, int64_t rows, int64_t K, int64_t ldx,
                             int8_t *q, int64_t ldq, float *scale, hipStream_t stream,
                             bool fp8 = false, bool keep_codes = false);

// ---- weight repack (prepack.hip) ----
hipError_t launch_prepack(const int8_t *wq, int64_t N, int64_t K, int64_t ldw, void *packed,
                          hipStream_t stream);
hipError_t launch_unpack(const void *packed, int64_t N, int64_t K, int8_t *wq, int64_t ldw,
                         hipStream_t stream);
// Per-channel quant of a bf16 (w_f32 false) or fp32 weight [N, ldw] straight
// into the packed layout, with the fp32 scales.
hipError_t launch_quant_prepack(const void *w, bool w_f32, int64_t N, int64_t K, int64_t ldw,
                                void *packed, float *w_scale, hipStream_t stream,
                                bool fp8 = false);

// ---- scaled matmul (scaled_mm.hip) ----
struct MmArgs {
    const int8_t *xq;
    const float *xs;
    const int8_t *wp;
    const float *ws;
    const uint16_t *bias;
    void *out;
    int64_t ldq;
    int64_t ldo;
    int M, N, K;
    int kblocks;     // round_up(K, 64) / 64: fragments along K in the packed weight
    int nblocks;     // round_up(N, 16) / 16: fragments along N in the packed weight
    int vec_store;   // 1 when out rows allow stores of 4 consecutive elements
    int vec16;       // 1 when out rows start on 16-byte boundaries
    // Fused quant: when x is set, the launch first quantizes x [M, ldx] (bf16)
    // into xq / xs, rows_per_wg rows per workgroup, then runs the matmul.
    const uint16_t *x;
    int64_t ldx;
    int rows_per_wg;
    unsigned epoch;       // this launch's number on its device, never 0
    unsigned wait_limit;  // bound on a workgroup's polls for its producers' flags
    // Split of K over workgroups (small-M kernel only; ksplit <= 1: none).
    // Each tile's ksplit workgroups take kbs k-blocks each; two words per
    // tile in split_count (arrivals, partial sums written) and the partial
    // sums in split_part let the last to arrive add them up and apply the
    // epilogue; it sets both words back to 0.
    int ksplit;
    int kbs;
    unsigned *split_count;
    int *split_part;
};

// Split of K for the small-M kernel: how many workgroups share a tile's K
// (1: no split) and the workspace the split needs (counters, then the
// partial sums), for `tiles` tiles of fm x fn 16 x 16 fragments and kblocks
// k-blocks spread over wk waves per workgroup.
struct SkinnySplit {
    int ksplit, kbs;
    size_t count_bytes, part_bytes;
    size_t bytes() const { return ksplit > 1 ? count_bytes + part_bytes : 0; }
};
SkinnySplit skinny_split(int64_t tiles, int fm, int fn, int wk, int kblocks);

// The library's own workspace for callers that cannot allocate: a static
// device array of kScratchBytes per device (skinny_mm.hip). *ptr is its
// device address on the current device, looked up once per device.
constexpr size_t kScratchBytes = size_t(4) << 20;
hipError_t scratch_address(void **ptr);

// Output kinds, the ABI's W8A8_OUT_* values: they index TileEntry's kernels.
constexpr int kOutBF16 = 0, kOutI32 = 1, kOutF16 = 2, kOutKinds = 3;

// One tile configuration: its output tile (bm x bn), block size and
// kernels per output kind (plain, and the fused quant + matmul forms, which
// read x in the output's 16-bit type, bf16 for int32; null where the
// configuration has none). skinny marks the small-M kernel.
typedef void (*MmKernel)(const MmArgs);
struct TileEntry {
    const char *name;
    int bm, bn, threads;
    bool skinny;
    MmKernel plain[kOutKinds], fused[kOutKinds];
};

// Small-M configurations (skinny_mm.hip); they follow the main kernel's in
// the tile numbering.
int skinny_tile_count();
const TileEntry &skinny_tile(int i);
const TileEntry &skinny_tile_fp8(int i);     // the e4m3 twin's, same order
// Fused quant + small-M matmul (each workgroup quantizes its own rows);
// hipErrorNotSupported (nothing launched) when the rows are too long.
hipError_t launch_skinny_quant_mm(const MmArgs &a, const TileEntry &e, int mode,
                                  hipStream_t stream);

// Physical workgroup id -> logical tile id such that each XCD (which takes
// ids pid % 8 round-robin) receives one contiguous run of logical ids.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_remap(int pid, int tiles)
{
    const int q = tiles / kXcds, r = tiles % kXcds;
    const int xcd = pid % kXcds, local = pid / kXcds;
    return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

int mm_tile_count();
const TileEntry &mm_tile_entry(int tile);     // int8 tiles: main, then small-M
const char *mm_tile_name(int tile);
int mm_tile_auto(int64_t M, int64_t N, int64_t K);
// Whether the grid of tile `tile` over an M x N output fits one launch
// (mm_grid_fits); fp8_launch_fits is the same for the e4m3 twin's tiles.
bool mm_launch_fits(int tile, int64_t M, int64_t N);
bool fp8_launch_fits(int tile, int64_t M, int64_t N);

// ---- the e4m3 twin of the matmul (scaled_mm_fp8.hip) ----
// Tiles are numbered as the int8 ones (main, then small-M); mode kOutI32
// stores the raw fp32 accumulators. The fused form returns
// hipErrorNotSupported (nothing launched) as launch_quant_scaled_mm does.
int fp8_tile_count();
hipError_t launch_scaled_mm_fp8(const MmArgs &a, int mode, int tile, hipStream_t stream);
hipError_t launch_quant_scaled_mm_fp8(MmArgs a, int mode, int tile, hipStream_t stream);
hipError_t launch_scaled_mm(const MmArgs &a, int mode, int tile, hipStream_t stream);
// Fused quant + matmul in one launch. Returns hipErrorNotSupported (nothing
// launched) when the shape's workgroups cannot all be resident at once; the
// caller then runs the two steps as separate launches.
hipError_t launch_quant_scaled_mm(MmArgs a, int mode, int tile, hipStream_t stream);
// The bound on the polls of the fused launches made from now on (process
// wide); returns the previous bound.
unsigned set_fused_wait_limit(unsigned polls);
unsigned fused_wait_limit();
// The same for any tile entry; cap_key (< 32) names it in the per-device
// cache of resident-workgroup capacities.
hipError_t launch_quant_scaled_mm_entry(MmArgs a, int mode, const TileEntry &e, int cap_key,
                                        hipStream_t stream);

}  // namespace w8a8
