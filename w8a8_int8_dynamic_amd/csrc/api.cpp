// C ABI of libw8a8 (declared in include/w8a8.h): argument checks, device
// check, and dispatch to the HIP kernels. Every check that can be made on
// the host runs before the first HIP call, so a bad argument never reaches
// the device and can be tested without one.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <limits>
#include <string>

#include "w8a8.h"   // include/ is on the include path
#include "internal.hpp"

#define W8A8_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

w8a8_status_t fail(w8a8_status_t s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
w8a8_status_t fail(w8a8_status_t s, const char *fmt, ...)
{
    char buf[256];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

w8a8_status_t ok()
{
    g_last_error.clear();
    return W8A8_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxRows = std::numeric_limits<int32_t>::max();

// Per-device cache of "is gfx950": 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_ok[kMaxDevices];

int query_supported(int device)
{
    if (device < 0 || device >= kMaxDevices) {
        fail(W8A8_ERR_DEVICE, "device %d out of range", device);
        return 0;
    }
    int c = g_dev_ok[device].load(std::memory_order_relaxed);
    if (c == 0) {
        hipDeviceProp_t prop;
        hipError_t e = hipGetDeviceProperties(&prop, device);
        if (e != hipSuccess) {   // not cached: the device may become usable later
            fail(W8A8_ERR_DEVICE, "hipGetDeviceProperties(%d): %s", device, hipGetErrorString(e));
            return 0;
        }
        c = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        if (c == 2)
            fail(W8A8_ERR_DEVICE, "device %d is %s, not gfx950", device, prop.gcnArchName);
        g_dev_ok[device].store(c, std::memory_order_relaxed);
    }
    return c == 1;
}

w8a8_status_t check_device()
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(W8A8_ERR_DEVICE, "no current HIP device: %s", hipGetErrorString(e));
    if (!query_supported(dev))
        return W8A8_ERR_DEVICE;   // query_supported recorded the reason
    return W8A8_OK;
}

w8a8_status_t launched(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(W8A8_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

w8a8_status_t quant_common(const void *x, int kind, int64_t M, int64_t K, int64_t ldx, int8_t *q,
                           int64_t ldq, float *s, void *stream, const char *what, bool fp8 = false)
{
    const bool f32 = kind == w8a8::kElemF32;
    if (M < 0 || M > kMaxRows)
        return fail(W8A8_ERR_SHAPE, "%s: rows %lld out of range", what, (long long)M);
    if (K < 1 || K > kMaxRows)
        return fail(W8A8_ERR_SHAPE, "%s: K %lld out of range", what, (long long)K);
    if (ldx < K || ldq < K)
        return fail(W8A8_ERR_SHAPE, "%s: leading dimension smaller than K", what);
    if (M == 0)
        return ok();
    if (!x || !q || !s)
        return fail(W8A8_ERR_NULL, "%s: NULL tensor pointer", what);
    const int64_t vec = f32 ? 4 : 8;
    if (!aligned(x, 16) || ldx % vec != 0)
        return fail(W8A8_ERR_ALIGN, "%s: input must be 16-byte aligned with ld a multiple of %lld",
                    what, (long long)vec);
    if (!aligned(q, 8) || ldq % 8 != 0)
        return fail(W8A8_ERR_ALIGN, "%s: codes must be 8-byte aligned with ld a multiple of 8", what);
    if (!aligned(s, 4))
        return fail(W8A8_ERR_ALIGN, "%s: scales must be 4-byte aligned", what);
    w8a8_status_t st = check_device();
    if (st != W8A8_OK)
        return st;
    return launched(w8a8::launch_quant_rows(x, kind, M, K, ldx, q, ldq, s,
                                            reinterpret_cast<hipStream_t>(stream), fp8),
                    what);
}

w8a8_status_t pack_common(int64_t N, int64_t K, int64_t ldw, const void *a, const void *b,
                          const void *packed, const char *what, bool device = true)
{
    if (N < 1 || N > kMaxRows || K < 1 || K > kMaxRows)
        return fail(W8A8_ERR_SHAPE, "%s: N and K must be in [1, 2^31)", what);
    if (ldw < K)
        return fail(W8A8_ERR_SHAPE, "%s: ldw smaller than K", what);
    if (int8_prepack_weight_bytes(N, K) == 0)
        return fail(W8A8_ERR_SHAPE, "%s: packed size overflows", what);
    if (!a || !b)
        return fail(W8A8_ERR_NULL, "%s: NULL tensor pointer", what);
    if (!aligned(packed, 16))
        return fail(W8A8_ERR_ALIGN, "%s: packed weight must be 16-byte aligned", what);
    return device ? check_device() : ok();
}

}  // namespace

W8A8_API w8a8_status_t int8_quant_per_token(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                                            int8_t *xq, int64_t ldq, float *x_scale, void *stream)
{
    return quant_common(x, w8a8::kElemBF16, M, K, ldx, xq, ldq, x_scale, stream,
                        "int8_quant_per_token");
}

W8A8_API w8a8_status_t int8_quant_per_token_f16(const uint16_t *x, int64_t M, int64_t K,
                                                int64_t ldx, int8_t *xq, int64_t ldq,
                                                float *x_scale, void *stream)
{
    return quant_common(x, w8a8::kElemF16, M, K, ldx, xq, ldq, x_scale, stream,
                        "int8_quant_per_token_f16");
}

W8A8_API w8a8_status_t int8_quant_per_channel(const float *w, int64_t N, int64_t K, int64_t ldw,
                                              int8_t *wq, int64_t ldq, float *w_scale,
                                              void *stream)
{
    return quant_common(w, w8a8::kElemF32, N, K, ldw, wq, ldq, w_scale, stream,
                        "int8_quant_per_channel");
}

W8A8_API size_t int8_prepack_weight_bytes(int64_t N, int64_t K)
{
    if (N < 1 || K < 1 || N > kMaxRows || K > kMaxRows)
        return 0;
    const unsigned __int128 n = (unsigned __int128)w8a8::round_up(N, w8a8::kFragN);
    const unsigned __int128 k = (unsigned __int128)w8a8::round_up(K, w8a8::kFragK);
    const unsigned __int128 bytes = n * k;
    if (bytes > (unsigned __int128)std::numeric_limits<size_t>::max() / 2)
        return 0;
    return (size_t)bytes;
}

W8A8_API w8a8_status_t int8_prepack_weight(const int8_t *wq, int64_t N, int64_t K, int64_t ldw,
                                           void *w_packed, void *stream)
{
    w8a8_status_t st = pack_common(N, K, ldw, wq, w_packed, w_packed, "int8_prepack_weight");
    if (st != W8A8_OK)
        return st;
    return launched(w8a8::launch_prepack(wq, N, K, ldw, w_packed,
                                         reinterpret_cast<hipStream_t>(stream)),
                    "int8_prepack_weight");
}

W8A8_API w8a8_status_t int8_quant_prepack_weight(const void *w, int w_dtype, int64_t N, int64_t K,
                                                 int64_t ldw, void *w_packed, float *w_scale,
                                                 void *stream)
{
    const char *what = "int8_quant_prepack_weight";
    if (w_dtype != W8A8_W_F32 && w_dtype != W8A8_W_BF16)
        return fail(W8A8_ERR_MODE, "%s: unknown weight dtype %d", what, w_dtype);
    const bool f32 = w_dtype == W8A8_W_F32;
    w8a8_status_t st = pack_common(N, K, ldw, w, w_packed, w_packed, what, false);
    if (st != W8A8_OK)
        return st;
    if (!w_scale)
        return fail(W8A8_ERR_NULL, "%s: NULL tensor pointer", what);
    if (!aligned(w, 16) || ldw % (f32 ? 4 : 8) != 0 || !aligned(w_scale, 4))
        return fail(W8A8_ERR_ALIGN, "%s: w must be 16-byte aligned with ldw a multiple of %d, "
                    "w_scale 4-byte aligned", what, f32 ? 4 : 8);
    st = check_device();
    if (st != W8A8_OK)
        return st;
    return launched(w8a8::launch_quant_prepack(w, f32, N, K, ldw, w_packed, w_scale,
                                               reinterpret_cast<hipStream_t>(stream)),
                    what);
}

W8A8_API w8a8_status_t int8_unpack_weight(const void *w_packed, int64_t N, int64_t K, int8_t *wq,
                                          int64_t ldw, void *stream)
{
    w8a8_status_t st = pack_common(N, K, ldw, w_packed, wq, w_packed, "int8_unpack_weight");
    if (st != W8A8_OK)
        return st;
    return launched(w8a8::launch_unpack(w_packed, N, K, wq, ldw,
                                        reinterpret_cast<hipStream_t>(stream)),
                    "int8_unpack_weight");
}

namespace {

// Checks the matmul arguments shared by int8_scaled_mm and the fused entry
// point and fills the kernel arguments. M == 0 passes (the callers return
// before launching). With need_xs the token scales are required in both
// output modes (the fused path writes them).
w8a8_status_t mm_args(const int8_t *xq, int64_t ldq, const float *x_scale, const void *w_packed,
                      const float *w_scale, const uint16_t *bias, int64_t M, int64_t N, int64_t K,
                      int mode, void *out, int64_t ldo, int tile, bool need_xs, const char *what,
                      w8a8::MmArgs &a, int &t, bool fp8 = false)
{
    if (mode != W8A8_OUT_BF16 && mode != W8A8_OUT_I32 && mode != W8A8_OUT_F16)
        return fail(W8A8_ERR_MODE, "%s: unknown output mode %d", what, mode);
    if (tile < -1 || tile >= (fp8 ? w8a8::fp8_tile_count() : w8a8::mm_tile_count()))
        return fail(W8A8_ERR_MODE, "%s: unknown tile %d", what, tile);
    if (M < 0 || M > kMaxRows || N < 1 || N > kMaxRows)
        return fail(W8A8_ERR_SHAPE, "%s: M or N out of range", what);
    if (K < 16 || K > W8A8_MAX_K || K % 16 != 0)
        return fail(W8A8_ERR_SHAPE, "%s: K must be a multiple of 16 in [16, %d]", what, W8A8_MAX_K);
    if (ldq < K || ldo < N)
        return fail(W8A8_ERR_SHAPE, "%s: leading dimension too small", what);
    if (ldq > W8A8_MAX_LDQ)
        return fail(W8A8_ERR_SHAPE, "%s: ldq above %d", what, W8A8_MAX_LDQ);
    a = w8a8::MmArgs{};
    t = -1;
    if (M == 0)
        return ok();
    const bool i32 = mode == W8A8_OUT_I32;
    if (!xq || !w_packed || !out || (!i32 && !w_scale) || ((need_xs || !i32) && !x_scale))
        return fail(W8A8_ERR_NULL, "%s: NULL tensor pointer", what);
    if (!aligned(xq, 16) || ldq % 16 != 0 || !aligned(w_packed, 16))
        return fail(W8A8_ERR_ALIGN, "%s: xq/w_packed must be 16-byte aligned, ldq a multiple of 16",
                    what);
    const uintptr_t esz = i32 ? 4 : 2;
    if (!aligned(out, esz))
        return fail(W8A8_ERR_ALIGN, "%s: out must be aligned to its element size", what);
    if ((x_scale && !aligned(x_scale, 4)) || (!i32 && (!aligned(w_scale, 4) || (bias && !aligned(bias, 2)))))
        return fail(W8A8_ERR_ALIGN, "%s: scales/bias misaligned", what);
    t = tile >= 0 ? tile : w8a8::mm_tile_auto(M, N, K);
    if (!(fp8 ? w8a8::fp8_launch_fits(t, M, N) : w8a8::mm_launch_fits(t, M, N)))
        return fail(W8A8_ERR_SHAPE, "%s: M x N needs more workgroups of tile %d than one launch holds",
                    what, t);
    a.xq = xq;
    a.xs = (i32 && !need_xs) ? nullptr : x_scale;
    a.wp = reinterpret_cast<const int8_t *>(w_packed);
    a.ws = i32 ? nullptr : w_scale;
    a.bias = i32 ? nullptr : bias;
    a.out = out;
    a.ldq = ldq;
    a.ldo = ldo;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.kblocks = (int)w8a8::ceil_div(K, w8a8::kFragK);
    a.nblocks = (int)w8a8::ceil_div(N, w8a8::kFragN);
    // 8-byte 16-bit / 16-byte int32 stores of 4 consecutive channels need every
    // row start (and channel multiples of 4) aligned to that width.
    const uintptr_t vw = 4 * esz;
    a.vec_store = aligned(out, vw) && ((uint64_t)ldo * esz) % vw == 0;
    a.vec16 = aligned(out, 16) && ((uint64_t)ldo * esz) % 16 == 0;
    a.x = nullptr;
    return ok();
}

}  // namespace

namespace {

// The split of K that tile t would use for an M x N x K product, and the
// workspace bytes it needs (0: no split for this shape and tile).
size_t split_need(int t, int64_t M, int64_t N, int64_t K, w8a8::SkinnySplit *split = nullptr)
{
    if (M < 1 || N < 1 || K < 1 || t < 0)
        return 0;
    const w8a8::TileEntry &e = w8a8::mm_tile_entry(t);
    if (!e.skinny)
        return 0;
    const int64_t tiles = w8a8::ceil_div(M, e.bm) * w8a8::ceil_div(N, e.bn);
    const w8a8::SkinnySplit sp = w8a8::skinny_split(tiles, e.bm / 16, e.bn / 16, e.threads / 64,
                                                    (int)w8a8::ceil_div(K, w8a8::kFragK));
    if (split)
        *split = sp;
    if (!w8a8::mm_grid_fits(tiles * sp.ksplit, e.threads))
        return 0;
    return sp.bytes();
}

// Hands the caller's workspace to the launch when tile t splits K for this
// shape and the workspace is large enough; otherwise the launch runs
// unsplit (same results).
w8a8_status_t take_workspace(w8a8::MmArgs &a, int t, void *workspace, size_t workspace_bytes,
                             const char *what)
{
    w8a8::SkinnySplit sp{};
    const size_t need = split_need(t, a.M, a.N, a.K, &sp);
    if (need == 0 || workspace == nullptr || workspace_bytes < need)
        return W8A8_OK;
    if (!aligned(workspace, 256))
        return fail(W8A8_ERR_ALIGN, "%s: workspace must be 256-byte aligned", what);
    a.ksplit = sp.ksplit;
    a.kbs = sp.kbs;
    a.split_count = reinterpret_cast<unsigned *>(workspace);
    a.split_part = reinterpret_cast<int *>(reinterpret_cast<char *>(workspace) + sp.count_bytes);
    return W8A8_OK;
}

w8a8_status_t scaled_mm_common(const int8_t *xq, int64_t ldq, const float *x_scale,
                               const void *w_packed, const float *w_scale, const uint16_t *bias,
                               int64_t M, int64_t N, int64_t K, int mode, void *out, int64_t ldo,
                               void *workspace, size_t workspace_bytes, void *stream, int tile,
                               const char *what)
{
    w8a8::MmArgs a;
    int t;
    w8a8_status_t st = mm_args(xq, ldq, x_scale, w_packed, w_scale, bias, M, N, K, mode, out, ldo,
                               tile, false, what, a, t);
    if (st != W8A8_OK || M == 0)
        return st;
    st = take_workspace(a, t, workspace, workspace_bytes, what);
    if (st != W8A8_OK)
        return st;
    st = check_device();
    if (st != W8A8_OK)
        return st;
    return launched(w8a8::launch_scaled_mm(a, mode, t, reinterpret_cast<hipStream_t>(stream)),
                    what);
}

}  // namespace

W8A8_API w8a8_status_t int8_scaled_mm_tile(const int8_t *xq, int64_t ldq, const float *x_scale,
                                           const void *w_packed, const float *w_scale,
                                           const uint16_t *bias, int64_t M, int64_t N, int64_t K,
                                           int mode, void *out, int64_t ldo, void *stream,
                                           int tile)
{
    return scaled_mm_common(xq, ldq, x_scale, w_packed, w_scale, bias, M, N, K, mode, out, ldo,
                            nullptr, 0, stream, tile, "int8_scaled_mm");
}

W8A8_API size_t int8_scaled_mm_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M < 1 || M > kMaxRows || N < 1 || N > kMaxRows || K < 16 || K > W8A8_MAX_K || K % 16 != 0)
        return 0;
    return split_need(w8a8::mm_tile_auto(M, N, K), M, N, K);
}

W8A8_API w8a8_status_t int8_scaled_mm_ws(const int8_t *xq, int64_t ldq, const float *x_scale,
                                         const void *w_packed, const float *w_scale,
                                         const uint16_t *bias, int64_t M, int64_t N, int64_t K,
                                         int mode, void *out, int64_t ldo, void *workspace,
                                         size_t workspace_bytes, void *stream)
{
    return scaled_mm_common(xq, ldq, x_scale, w_packed, w_scale, bias, M, N, K, mode, out, ldo,
                            workspace, workspace_bytes, stream, -1, "int8_scaled_mm_ws");
}

namespace {

// The fused entry points for bf16 and fp16 activations (x_kind).
w8a8_status_t quant_mm_common(const uint16_t *x, int x_kind, int64_t ldx, int8_t *xq, int64_t ldq,
                              float *x_scale, const void *w_packed, const float *w_scale,
                              const uint16_t *bias, int64_t M, int64_t N, int64_t K, int mode,
                              void *out, int64_t ldo, void *stream, int tile, const char *what,
                              void *workspace = nullptr, size_t workspace_bytes = 0)
{
    w8a8::MmArgs a;
    int t;
    w8a8_status_t st = mm_args(xq, ldq, x_scale, w_packed, w_scale, bias, M, N, K, mode, out, ldo,
                               tile, true, what, a, t);
    if (st != W8A8_OK)
        return st;
    if (ldx < K)
        return fail(W8A8_ERR_SHAPE, "%s: ldx smaller than K", what);
    if (M == 0)
        return ok();
    if (!x)
        return fail(W8A8_ERR_NULL, "%s: NULL tensor pointer", what);
    if (!aligned(x, 16) || ldx % 8 != 0)
        return fail(W8A8_ERR_ALIGN, "%s: x must be 16-byte aligned with ldx a multiple of 8", what);
    st = take_workspace(a, t, workspace, workspace_bytes, what);
    if (st != W8A8_OK)
        return st;
    st = check_device();
    if (st != W8A8_OK)
        return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    a.x = x;
    a.ldx = ldx;
    // The single-launch kernels read x in the output's 16-bit type (bf16 for
    // the int32 mode); other pairings take the two launches.
    const int fused_kind = mode == W8A8_OUT_F16 ? w8a8::kElemF16 : w8a8::kElemBF16;
    if (x_kind == fused_kind) {
        hipError_t err = w8a8::launch_quant_scaled_mm(a, mode, t, s);
        if (err != hipErrorNotSupported)
            return launched(err, what);
        (void)hipGetLastError();
    }
    // Two launches on the same stream (also when the grid cannot be
    // resident all at once); the codes stay in the caches for the matmul.
    a.x = nullptr;
    hipError_t err = w8a8::launch_quant_rows(x, x_kind, M, K, ldx, xq, ldq, x_scale, s, false, true);
    if (err != hipSuccess)
        return launched(err, what);
    return launched(w8a8::launch_scaled_mm(a, mode, t, s), what);
}

}  // namespace

W8A8_API w8a8_status_t int8_quant_scaled_mm_tile(const uint16_t *x, int64_t ldx, int8_t *xq,
                                                 int64_t ldq, float *x_scale,
                                                 const void *w_packed, const float *w_scale,
                                                 const uint16_t *bias, int64_t M, int64_t N,
                                                 int64_t K, int mode, void *out, int64_t ldo,
                                                 void *stream, int tile)
{
    return quant_mm_common(x, w8a8::kElemBF16, ldx, xq, ldq, x_scale, w_packed, w_scale, bias, M, N,
                           K, mode, out, ldo, stream, tile, "int8_quant_scaled_mm");
}

W8A8_API w8a8_status_t int8_quant_scaled_mm_f16_tile(const uint16_t *x, int64_t ldx, int8_t *xq,
                                                     int64_t ldq, float *x_scale,
                                                     const void *w_packed, const float *w_scale,
                                                     const uint16_t *bias, int64_t M, int64_t N,
                                                     int64_t K, int mode, void *out, int64_t ldo,
                                                     void *stream, int tile)
{
    return quant_mm_common(x, w8a8::kElemF16, ldx, xq, ldq, x_scale, w_packed, w_scale, bias, M, N,
                           K, mode, out, ldo, stream, tile, "int8_quant_scaled_mm_f16");
}

W8A8_API w8a8_status_t int8_quant_scaled_mm_f16(const uint16_t *x, int64_t ldx, int8_t *xq,
                                                int64_t ldq, float *x_scale, const void *w_packed,
                                                const float *w_scale, const uint16_t *bias,
                                                int64_t M, int64_t N, int64_t K, int mode,
                                                void *out, int64_t ldo, void *stream)
{
    return int8_quant_scaled_mm_f16_tile(x, ldx, xq, ldq, x_scale, w_packed, w_scale, bias, M, N,
                                         K, mode, out, ldo, stream, -1);
}

W8A8_API w8a8_status_t int8_quant_scaled_mm(const uint16_t *x, int64_t ldx, int8_t *xq,
                                            int64_t ldq, float *x_scale, const void *w_packed,
                                            const float *w_scale, const uint16_t *bias, int64_t M,
                                            int64_t N, int64_t K, int mode, void *out,
                                            int64_t ldo, void *stream)
{
    return int8_quant_scaled_mm_tile(x, ldx, xq, ldq, x_scale, w_packed, w_scale, bias, M, N, K,
                                     mode, out, ldo, stream, -1);
}

W8A8_API w8a8_status_t int8_quant_scaled_mm_ws(const uint16_t *x, int64_t ldx, int8_t *xq,
                                               int64_t ldq, float *x_scale, const void *w_packed,
                                               const float *w_scale, const uint16_t *bias,
                                               int64_t M, int64_t N, int64_t K, int mode,
                                               void *out, int64_t ldo, void *workspace,
                                               size_t workspace_bytes, void *stream)
{
    return quant_mm_common(x, w8a8::kElemBF16, ldx, xq, ldq, x_scale, w_packed, w_scale, bias, M,
                           N, K, mode, out, ldo, stream, -1, "int8_quant_scaled_mm_ws", workspace,
                           workspace_bytes);
}

W8A8_API w8a8_status_t int8_quant_scaled_mm_noalloc(const uint16_t *x, int64_t ldx, int8_t *xq,
                                                    int64_t ldq, float *x_scale,
                                                    const void *w_packed, const float *w_scale,
                                                    const uint16_t *bias, int64_t M, int64_t N,
                                                    int64_t K, int mode, void *out, int64_t ldo,
                                                    void *stream)
{
    const char *what = "int8_quant_scaled_mm_noalloc";
    const size_t need = int8_scaled_mm_workspace_bytes(M, N, K);
    if (need > w8a8::kScratchBytes)
        return fail(W8A8_ERR_SHAPE,
                    "%s: this shape's split needs %zu bytes of workspace, more than the %zu "
                    "the library holds",
                    what, need, w8a8::kScratchBytes);
    void *scratch = nullptr;
    if (need > 0 && M > 0) {
        // Argument errors are reported before any HIP call.
        w8a8::MmArgs a;
        int t;
        w8a8_status_t st = mm_args(xq, ldq, x_scale, w_packed, w_scale, bias, M, N, K, mode, out,
                                   ldo, -1, true, what, a, t);
        if (st != W8A8_OK)
            return st;
        st = check_device();
        if (st != W8A8_OK)
            return st;
        hipError_t err = w8a8::scratch_address(&scratch);
        if (err != hipSuccess)
            return fail(W8A8_ERR_HIP, "%s: the library's workspace has no device address: %s", what,
                        hipGetErrorString(err));
    }
    return quant_mm_common(x, w8a8::kElemBF16, ldx, xq, ldq, x_scale, w_packed, w_scale, bias, M,
                           N, K, mode, out, ldo, stream, -1, what, scratch, w8a8::kScratchBytes);
}

W8A8_API w8a8_status_t int8_scaled_mm(const int8_t *xq, int64_t ldq, const float *x_scale,
                                      const void *w_packed, const float *w_scale,
                                      const uint16_t *bias, int64_t M, int64_t N, int64_t K,
                                      int mode, void *out, int64_t ldo, void *stream)
{
    return int8_scaled_mm_tile(xq, ldq, x_scale, w_packed, w_scale, bias, M, N, K, mode, out, ldo,
                               stream, -1);
}

// ---- the FP8 (e4m3) twin ----------------------------------------------

W8A8_API w8a8_status_t fp8_quant_per_token(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                                           uint8_t *xq, int64_t ldq, float *x_scale, void *stream)
{
    return quant_common(x, w8a8::kElemBF16, M, K, ldx, reinterpret_cast<int8_t *>(xq), ldq, x_scale,
                        stream, "fp8_quant_per_token", true);
}

W8A8_API w8a8_status_t fp8_quant_per_channel(const float *w, int64_t N, int64_t K, int64_t ldw,
                                             uint8_t *wq, int64_t ldq, float *w_scale,
                                             void *stream)
{
    return quant_common(w, w8a8::kElemF32, N, K, ldw, reinterpret_cast<int8_t *>(wq), ldq, w_scale,
                        stream, "fp8_quant_per_channel", true);
}

W8A8_API w8a8_status_t fp8_quant_prepack_weight(const void *w, int w_dtype, int64_t N, int64_t K,
                                                int64_t ldw, void *w_packed, float *w_scale,
                                                void *stream)
{
    const char *what = "fp8_quant_prepack_weight";
    if (w_dtype != W8A8_W_F32 && w_dtype != W8A8_W_BF16)
        return fail(W8A8_ERR_MODE, "%s: unknown weight dtype %d", what, w_dtype);
    const bool f32 = w_dtype == W8A8_W_F32;
    w8a8_status_t st = pack_common(N, K, ldw, w, w_packed, w_packed, what, false);
    if (st != W8A8_OK)
        return st;
    if (!w_scale)
        return fail(W8A8_ERR_NULL, "%s: NULL tensor pointer", what);
    if (!aligned(w, 16) || ldw % (f32 ? 4 : 8) != 0 || !aligned(w_scale, 4))
        return fail(W8A8_ERR_ALIGN, "%s: w must be 16-byte aligned with ldw a multiple of %d, "
                    "w_scale 4-byte aligned", what, f32 ? 4 : 8);
    st = check_device();
    if (st != W8A8_OK)
        return st;
    return launched(w8a8::launch_quant_prepack(w, f32, N, K, ldw, w_packed, w_scale,
                                               reinterpret_cast<hipStream_t>(stream), true),
                    what);
}

W8A8_API w8a8_status_t fp8_scaled_mm_tile(const uint8_t *xq, int64_t ldq, const float *x_scale,
                                          const void *w_packed, const float *w_scale,
                                          const uint16_t *bias, int64_t M, int64_t N, int64_t K,
                                          int mode, void *out, int64_t ldo, void *stream, int tile)
{
    const char *what = "fp8_scaled_mm";
    w8a8::MmArgs a;
    int t;
    w8a8_status_t st = mm_args(reinterpret_cast<const int8_t *>(xq), ldq, x_scale, w_packed,
                               w_scale, bias, M, N, K, mode, out, ldo, tile, false, what, a, t,
                               true);
    if (st != W8A8_OK || M == 0)
        return st;
    st = check_device();
    if (st != W8A8_OK)
        return st;
    return launched(w8a8::launch_scaled_mm_fp8(a, mode, t, reinterpret_cast<hipStream_t>(stream)),
                    what);
}

W8A8_API w8a8_status_t fp8_scaled_mm(const uint8_t *xq, int64_t ldq, const float *x_scale,
                                     const void *w_packed, const float *w_scale,
                                     const uint16_t *bias, int64_t M, int64_t N, int64_t K,
                                     int mode, void *out, int64_t ldo, void *stream)
{
    return fp8_scaled_mm_tile(xq, ldq, x_scale, w_packed, w_scale, bias, M, N, K, mode, out, ldo,
                              stream, -1);
}

W8A8_API w8a8_status_t fp8_quant_scaled_mm_tile(const uint16_t *x, int64_t ldx, uint8_t *xq,
                                                int64_t ldq, float *x_scale, const void *w_packed,
                                                const float *w_scale, const uint16_t *bias,
                                                int64_t M, int64_t N, int64_t K, int mode,
                                                void *out, int64_t ldo, void *stream, int tile)
{
    const char *what = "fp8_quant_scaled_mm";
    w8a8::MmArgs a;
    int t;
    w8a8_status_t st = mm_args(reinterpret_cast<const int8_t *>(xq), ldq, x_scale, w_packed,
                               w_scale, bias, M, N, K, mode, out, ldo, tile, true, what, a, t,
                               true);
    if (st != W8A8_OK)
        return st;
    if (ldx < K)
        return fail(W8A8_ERR_SHAPE, "%s: ldx smaller than K", what);
    if (M == 0)
        return ok();
    if (!x)
        return fail(W8A8_ERR_NULL, "%s: NULL tensor pointer", what);
    if (!aligned(x, 16) || ldx % 8 != 0)
        return fail(W8A8_ERR_ALIGN, "%s: x must be 16-byte aligned with ldx a multiple of 8", what);
    st = check_device();
    if (st != W8A8_OK)
        return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // One launch where the int8 path would take one (the fused kernels read
    // bf16 x for bf16 and raw output), else the two steps.
    if (mode != W8A8_OUT_F16) {
        a.x = x;
        a.ldx = ldx;
        hipError_t err = w8a8::launch_quant_scaled_mm_fp8(a, mode, t, s);
        if (err != hipErrorNotSupported)
            return launched(err, what);
        (void)hipGetLastError();
        a.x = nullptr;
    }
    hipError_t err = w8a8::launch_quant_rows(x, w8a8::kElemBF16, M, K, ldx,
                                             reinterpret_cast<int8_t *>(xq), ldq, x_scale, s, true,
                                             true);
    if (err != hipSuccess)
        return launched(err, what);
    return launched(w8a8::launch_scaled_mm_fp8(a, mode, t, s), what);
}

W8A8_API w8a8_status_t fp8_quant_scaled_mm(const uint16_t *x, int64_t ldx, uint8_t *xq,
                                           int64_t ldq, float *x_scale, const void *w_packed,
                                           const float *w_scale, const uint16_t *bias, int64_t M,
                                           int64_t N, int64_t K, int mode, void *out, int64_t ldo,
                                           void *stream)
{
    return fp8_quant_scaled_mm_tile(x, ldx, xq, ldq, x_scale, w_packed, w_scale, bias, M, N, K,
                                    mode, out, ldo, stream, -1);
}

W8A8_API int w8a8_fp8_tile_count(void) { return w8a8::fp8_tile_count(); }

W8A8_API int w8a8_fp8_tile_auto(int64_t M, int64_t N, int64_t K)
{
    return w8a8::mm_tile_auto(M, N, K);
}

W8A8_API int w8a8_mm_tile_count(void) { return w8a8::mm_tile_count(); }

W8A8_API const char *w8a8_mm_tile_name(int tile) { return w8a8::mm_tile_name(tile); }

W8A8_API int w8a8_mm_tile_auto(int64_t M, int64_t N, int64_t K)
{
    return w8a8::mm_tile_auto(M, N, K);
}

W8A8_API int w8a8_fused_wait_limit(int polls)
{
    return polls >= 0 ? (int)w8a8::set_fused_wait_limit((unsigned)polls)
                      : (int)w8a8::fused_wait_limit();
}

W8A8_API int w8a8_device_supported(int device) { return query_supported(device); }

W8A8_API const char *w8a8_status_string(int status)
{
    switch (status) {
    case W8A8_OK: return "success";
    case W8A8_ERR_NULL: return "a required pointer is NULL";
    case W8A8_ERR_SHAPE: return "a size or leading dimension is out of range";
    case W8A8_ERR_ALIGN: return "a pointer or leading dimension breaks an alignment rule";
    case W8A8_ERR_DEVICE: return "no usable current device, or it is not gfx950";
    case W8A8_ERR_MODE: return "unknown output mode or tile id";
    case W8A8_ERR_HIP: return "the HIP runtime reported an error when launching";
    default: return "unknown status";
    }
}

W8A8_API const char *w8a8_last_error(void) { return g_last_error.c_str(); }
