/*
 * w8a8.h - C ABI of libw8a8, W8A8 int8-dynamic linear layers on MI355X (gfx950).
 *
 * The layer computed here is the one the page "Issue 5 probe: int8 quantized
 * DiT serve paths on the RTX 3090 (24 GB)" serves in its "Round two" section:
 * int8 weights quantized per output channel with fp32 scales, activations
 * quantized per token at run time (dynamic, symmetric), an int8 x int8 ->
 * int32 matmul, and a scale epilogue back to bf16. The same page's kernel-path
 * paragraph names the two run-time ops (a per-token quant, then a scaled
 * matmul) and the load-time transpose-repack of the weight; this header
 * exposes those three steps, the offline weight quantization that produces
 * the int8 weights and a debug unpack of the repacked weight. Beyond them:
 * the quant and the matmul in one call (int8_quant_scaled_mm), fp16
 * activations and outputs, the online weight quant straight into the
 * repacked layout, and an FP8 (e4m3) twin of the whole path.
 *
 * Conventions for every entry point:
 *   - Pointers to tensors are DEVICE pointers on the current HIP device.
 *     bf16 values are passed as their raw 16-bit patterns (uint16_t).
 *   - Shapes are row-major with an explicit leading dimension (elements
 *     between consecutive rows). A matrix [R, C] with leading dimension ld
 *     occupies (R-1)*ld + C elements.
 *   - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued
 *     and the call returns without synchronizing; inputs must stay alive and
 *     unmodified until the stream reaches the work.
 *   - The library never allocates, frees or synchronizes device memory. The
 *     caller owns every buffer. Outputs must not alias inputs.
 *   - All argument checks run on the host before any HIP call, so a bad
 *     argument returns an error without touching the device. There is no
 *     fallback path: an unsupported device or argument is an error.
 *   - Calls are thread-safe. Shared host state is atomic: per-device caches
 *     (the "is this a gfx950" answer, the fused kernels' resident-workgroup
 *     capacity) and a per-device launch counter for the fused kernels'
 *     flags; the error message is thread-local. The library-owned device
 *     memory is static: those flags (see int8_quant_scaled_mm) and the
 *     workspace of int8_quant_scaled_mm_noalloc.
 */
#ifndef W8A8_H
#define W8A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum w8a8_status {
    W8A8_OK = 0,
    W8A8_ERR_NULL = 1,   /* a required pointer is NULL */
    W8A8_ERR_SHAPE = 2,  /* a size or leading dimension is out of range */
    W8A8_ERR_ALIGN = 3,  /* a pointer or leading dimension breaks an alignment rule */
    W8A8_ERR_DEVICE = 4, /* no usable current device, or it is not gfx950 */
    W8A8_ERR_MODE = 5,   /* unknown output mode or tile id */
    W8A8_ERR_HIP = 6     /* the HIP runtime reported an error when launching */
} w8a8_status_t;

/* Output of int8_scaled_mm: the layer output in bf16 or fp16, or the raw
 * int32 accumulators (debug mode; the scales and bias are then ignored).
 * The bias, when given, has the output's type (bf16 or fp16 bits). */
typedef enum w8a8_mm_out {
    W8A8_OUT_BF16 = 0,
    W8A8_OUT_I32 = 1,
    W8A8_OUT_F16 = 2
} w8a8_mm_out_t;

/* Largest K accepted by int8_scaled_mm: the largest multiple of 16 with
 * 128 * 128 * K < 2^31, so no int32 partial sum can overflow for any int8
 * codes (the quantizers only emit -127..127). */
#define W8A8_MAX_K 131056

/* Largest row pitch ldq (bytes) of the int8 (or e4m3) activation codes that
 * the matmuls accept: the main kernel addresses a tile's 256 token rows with
 * 32-bit offsets from the tile's first row. */
#define W8A8_MAX_LDQ 4194304

/*
 * int8_quant_per_token - dynamic per-token symmetric activation quantization.
 * (Page "Issue 5 probe ...", section "Round two": dynamic per-token symmetric
 * int8 activations; page "Online Quantization", Parameters table: the
 * "dynamic" activation scheme computes activation scales at run time.)
 *
 * For each row m of x [M, ldx] (bf16), over its first K elements:
 *   a = max_k |x[m,k]|
 *   if a < 2^-100:  x_scale[m] = 0, xq[m,:] = 0
 *   else:           x_scale[m] = fl32(a / 127), inv = fl32(127 / a),
 *                   xq[m,k] = clamp(round_half_even(fl32(x[m,k] * inv)), -127, 127)
 * Outputs: xq int8 [M, ldq], x_scale fp32 [M].
 * Requirements: M >= 0 (M == 0 is a no-op), K >= 1, ldx >= K, ldq >= K;
 * x 16-byte aligned and ldx a multiple of 8; xq 8-byte aligned and ldq a
 * multiple of 8; x_scale 4-byte aligned. Any K is allowed (ragged tails are
 * handled element by element). NaN/Inf inputs give unspecified codes.
 */
w8a8_status_t int8_quant_per_token(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                                   int8_t *xq, int64_t ldq, float *x_scale, void *stream);

/*
 * int8_quant_per_token_f16 - int8_quant_per_token for fp16 activations (the
 * pages run the layer with bf16 and with fp16 activations: page "Issue 5
 * probe ...", the isolation table's two activation columns). Each element
 * is widened to fp32 exactly; the rule, outputs and requirements are those
 * of int8_quant_per_token (x holds fp16 bit patterns).
 */
w8a8_status_t int8_quant_per_token_f16(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                                       int8_t *xq, int64_t ldq, float *x_scale, void *stream);

/*
 * int8_quant_per_channel - per-output-channel symmetric weight quantization.
 * (Page "Issue 5 probe ...", "Round one" setup paragraph: int8 weights,
 * per-output-channel symmetric; "Round two" artifacts paragraph: int8 weights
 * with fp32 per-channel scales. Page "Online Quantization", Overview: online
 * quantization computes weights and scales while loading.)
 *
 * The same rule as int8_quant_per_token applied to each row of an fp32
 * weight w [N, ldw] (out x in). Outputs: wq int8 [N, ldq], w_scale fp32 [N].
 * Requirements: N >= 0, K >= 1, ldw >= K, ldq >= K; w 16-byte aligned and
 * ldw a multiple of 4; wq 8-byte aligned, ldq a multiple of 8.
 */
w8a8_status_t int8_quant_per_channel(const float *w, int64_t N, int64_t K, int64_t ldw,
                                     int8_t *wq, int64_t ldq, float *w_scale, void *stream);

/*
 * int8_prepack_weight_bytes - size in bytes of the prepacked form of an
 * int8 weight [N, K]: round_up(N, 16) * round_up(K, 64). Returns 0 when
 * N < 1, K < 1 or the size does not fit in size_t.
 */
size_t int8_prepack_weight_bytes(int64_t N, int64_t K);

/*
 * int8_prepack_weight - load-time repack of an int8 weight into the layout
 * int8_scaled_mm reads (page "Issue 5 probe ...", "Round two" kernel-path
 * paragraph: load, then transpose-repack, then apply).
 *
 * A pure byte permutation with zero padding: the packed buffer is a sequence
 * of 1024-byte fragments F[nb][kb] (nb < round_up(N,16)/16, kb <
 * round_up(K,64)/64, kb fastest). Byte 16*l + j of F[nb][kb] holds
 * wq[16*nb + l % 16][64*kb + 16*(l / 16) + j] for l < 64, j < 16, or 0 when
 * that row or column lies outside [N, K].
 * Requirements: N >= 1, K >= 1, ldw >= K; w_packed 16-byte aligned with
 * int8_prepack_weight_bytes(N, K) bytes. wq has no alignment rule.
 */
w8a8_status_t int8_prepack_weight(const int8_t *wq, int64_t N, int64_t K, int64_t ldw,
                                  void *w_packed, void *stream);

/* Element type of a weight handed to int8_quant_prepack_weight. */
typedef enum {
    W8A8_W_F32 = 0,
    W8A8_W_BF16 = 1
} w8a8_w_dtype_t;

/*
 * int8_quant_prepack_weight - online (load-time) weight quantization: the
 * per-output-channel rule of int8_quant_per_channel applied to a bf16 or
 * fp32 weight w [N, ldw] (out x in), written straight into the layout of
 * int8_prepack_weight, with the scales w_scale fp32 [N]. (Page "Online
 * Quantization", Overview: weights and scales are computed while the model
 * loads, from a BF16 checkpoint, with no separately prepared quantized
 * checkpoint.)
 *
 * The packed bytes and scales are identical to int8_quant_per_channel of
 * the weight (as fp32; bf16 converts exactly) followed by
 * int8_prepack_weight; the int8 weight is never stored unpacked.
 * w_dtype: W8A8_W_F32 or W8A8_W_BF16.
 * Requirements: N >= 1, K >= 1, ldw >= K; w 16-byte aligned with ldw a
 * multiple of 4 (fp32) or 8 (bf16); w_packed 16-byte aligned with
 * int8_prepack_weight_bytes(N, K) bytes; w_scale 4-byte aligned.
 */
w8a8_status_t int8_quant_prepack_weight(const void *w, int w_dtype, int64_t N, int64_t K,
                                        int64_t ldw, void *w_packed, float *w_scale,
                                        void *stream);

/*
 * int8_unpack_weight - inverse of int8_prepack_weight (debug/verification):
 * writes wq[n, k] for n < N, k < K; other bytes of wq are not touched.
 */
w8a8_status_t int8_unpack_weight(const void *w_packed, int64_t N, int64_t K, int8_t *wq,
                                 int64_t ldw, void *stream);

/*
 * int8_scaled_mm - int8 x int8 -> int32 matmul with the scale epilogue
 * (page "Issue 5 probe ...", "Round two" kernel-path paragraph: the scaled
 * matmul after the per-token quant, whose reference must include the
 * act_scale factor; page "INT8 Quant for Dual-Max Recipe": W8A8 runs
 * int8 x int8 with no dequantization).
 *
 *   acc[m,n] = sum_{k<K} xq[m,k] * wq[n,k]                (exact, int32)
 *   W8A8_OUT_BF16: out[m,n] = bf16_rne( fl32(fl32(fl32(acc) * x_scale[m]) * w_scale[n])
 *                                        [+ bias[n], rounded to fp32] )
 *   W8A8_OUT_F16:  the same fp32 value (with an fp16 bias) rounded to fp16,
 *                  nearest-even (overflow gives infinity)
 *   W8A8_OUT_I32:  out[m,n] = acc[m,n]
 * Inputs: xq int8 [M, ldq]; x_scale fp32 [M]; w_packed from
 * int8_prepack_weight(N, K); w_scale fp32 [N]; bias [N] in the output's
 * type (bf16 or fp16 bits) or NULL.
 * Output: bf16, fp16 or int32 [M, ldo].
 * Requirements: M >= 0 (M == 0 is a no-op), N >= 1, 16 <= K <= W8A8_MAX_K
 * with K a multiple of 16, K <= ldq <= W8A8_MAX_LDQ, ldo >= N; xq and
 * w_packed 16-byte aligned, ldq a multiple of 16; out aligned to its element
 * size. In I32
 * mode x_scale, w_scale and bias may be NULL and are ignored.
 * Errors: W8A8_ERR_SHAPE also when the tile's workgroups over M x N, times
 * its threads, do not fit in 32 bits (one launch's grid). That takes more
 * than about 2^36 outputs on the smallest main tile, or more than about 2^27
 * channels on a small-M tile.
 */
w8a8_status_t int8_scaled_mm(const int8_t *xq, int64_t ldq, const float *x_scale,
                             const void *w_packed, const float *w_scale, const uint16_t *bias,
                             int64_t M, int64_t N, int64_t K, int mode, void *out, int64_t ldo,
                             void *stream);

/*
 * int8_scaled_mm_tile - int8_scaled_mm with an explicit tile configuration
 * (0 <= tile < w8a8_mm_tile_count()), or -1 for the automatic choice that
 * int8_scaled_mm makes. Every tile computes bit-identical results; this
 * exists for tuning and for testing each configuration.
 */
w8a8_status_t int8_scaled_mm_tile(const int8_t *xq, int64_t ldq, const float *x_scale,
                                  const void *w_packed, const float *w_scale,
                                  const uint16_t *bias, int64_t M, int64_t N, int64_t K, int mode,
                                  void *out, int64_t ldo, void *stream, int tile);

/*
 * int8_quant_scaled_mm - the layer's two run-time steps in one call:
 * int8_quant_per_token of x, then int8_scaled_mm of the result (page "Issue 5
 * probe ...", "Round two" kernel-path paragraph: a per-token quant followed
 * by the scaled matmul). Results are bit-identical to calling the two entry
 * points in sequence.
 *
 * Inputs: x bf16 [M, ldx]; w_packed, w_scale, bias as for int8_scaled_mm.
 * Outputs: the codes xq int8 [M, ldq] and scales x_scale fp32 [M] (written,
 * as int8_quant_per_token writes them) and out ([M, ldo] in the mode's type).
 * The single-launch paths below serve modes W8A8_OUT_BF16 and W8A8_OUT_I32;
 * W8A8_OUT_F16 from bf16 activations runs as two launches.
 * Requirements: those of int8_scaled_mm, plus ldx >= K, x 16-byte aligned
 * and ldx a multiple of 8; x_scale is required in both output modes.
 *
 * When the chosen tile is one of the main kernel's, every workgroup of the
 * matmul can be resident at once (true for the fused-QKV layer at M 512
 * and smaller) and xq and x_scale both start on 256-byte boundaries (so
 * that no cache line holds rows of two row tiles; buffers from the usual
 * allocators are), one launch does both steps: each workgroup quantizes a slice
 * of rows, raises its flag (a word in the library's device memory, set to a
 * number unique to the launch), and waits, bounded, only for the flags of
 * its own tile's rows; should a wait ever run out, that workgroup quantizes
 * its tile's rows itself, so the result never depends on scheduling. Calls
 * that overlap on one device therefore stay correct (each sees only its own
 * launch's flags) but may take that slower path. The launch number is
 * fixed when the launch is made, so a call made while `stream` is being
 * captured into a graph takes the two launches instead (a replayed graph
 * would otherwise reuse one number).
 *
 * With a small-M tile and at most two token rows (K up to 4096 for two
 * rows, 8192 for one), one launch also does both steps, with no flags: each
 * workgroup quantizes the rows into its own LDS and the workgroups of the
 * first column block also write xq and x_scale. This form is safe under
 * graph capture.
 *
 * Otherwise (a grid too large to be resident, xq or x_scale not 256-byte
 * aligned, or more rows on a small-M tile) the two steps run as two
 * launches on `stream`.
 */
w8a8_status_t int8_quant_scaled_mm(const uint16_t *x, int64_t ldx, int8_t *xq, int64_t ldq,
                                   float *x_scale, const void *w_packed, const float *w_scale,
                                   const uint16_t *bias, int64_t M, int64_t N, int64_t K, int mode,
                                   void *out, int64_t ldo, void *stream);

/*
 * int8_scaled_mm_workspace_bytes - bytes of workspace that int8_scaled_mm_ws
 * and int8_quant_scaled_mm_ws use for an M x N x K product (automatic tile),
 * or 0 when that shape runs without one.
 *
 * A workspace serves the small-M (decode-shaped) kernel when the weight has
 * too few 16-channel column blocks to keep every CU streaming it (page
 * "INT8 Quant for Dual-Max Recipe", controlled-run takeaways: decode is
 * bound by moving the weight): K is then split over 2 to 8 workgroups per
 * tile. Each takes a ticket from a per-tile arrival word; all but the last
 * leave their int32 partial sums in the workspace and count themselves in a
 * second per-tile word; the last waits for that count, adds the partial
 * sums up (exact in int32, so the output is bit-identical to the unsplit
 * one), applies the epilogue and sets both words back to 0. Layout: the
 * per-tile words (8 bytes per tile, rounded up to 256 bytes), then 1 KB of
 * partial sums per 16 x 16 fragment pair of each split. Arguments out of
 * range give 0.
 */
size_t int8_scaled_mm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * int8_scaled_mm_ws - int8_scaled_mm (automatic tile) with a workspace
 * (device memory, 256-byte aligned, workspace_bytes long) that the split of
 * K described at int8_scaled_mm_workspace_bytes uses when the shape calls
 * for one and workspace_bytes is at least that many bytes; otherwise the
 * call runs as int8_scaled_mm. Results are bit-identical either way.
 *
 * The workspace's per-tile words must be zero before its first use (zero it
 * once when allocating it); every call leaves them zero. The caller owns it
 * and keeps it alive until the stream has run the call. Calls that overlap
 * on one workspace (two streams, or graph replays that run concurrently)
 * race: give each concurrent caller its own. workspace may be NULL (no
 * split). Errors: those of int8_scaled_mm, plus W8A8_ERR_ALIGN for a
 * workspace that is used but not 256-byte aligned.
 */
w8a8_status_t int8_scaled_mm_ws(const int8_t *xq, int64_t ldq, const float *x_scale,
                                const void *w_packed, const float *w_scale, const uint16_t *bias,
                                int64_t M, int64_t N, int64_t K, int mode, void *out, int64_t ldo,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * int8_quant_scaled_mm_ws - int8_quant_scaled_mm (bf16 activations,
 * automatic tile) with a workspace for the split of K, on the terms of
 * int8_scaled_mm_ws. The split applies to the small-M kernel (its fused
 * quant included; the workgroups of the first column block and first split
 * write xq and x_scale).
 */
w8a8_status_t int8_quant_scaled_mm_ws(const uint16_t *x, int64_t ldx, int8_t *xq, int64_t ldq,
                                      float *x_scale, const void *w_packed, const float *w_scale,
                                      const uint16_t *bias, int64_t M, int64_t N, int64_t K,
                                      int mode, void *out, int64_t ldo, void *workspace,
                                      size_t workspace_bytes, void *stream);

/*
 * int8_quant_scaled_mm_noalloc - int8_quant_scaled_mm_ws for callers that
 * cannot allocate device memory (code under graph capture, tight serving
 * loops, harnesses that forbid allocation): the workspace is the library's
 * own, a static device array of 4 MiB that each GPU holds from the
 * library's first use until the process ends. The call allocates nothing
 * (no hipMalloc, no allocating library routine); the caller still passes
 * inputs and outputs.
 *
 * Shapes whose split needs more than 4 MiB of workspace
 * (int8_scaled_mm_workspace_bytes) are W8A8_ERR_SHAPE. All calls on one GPU
 * share that GPU's array: its per-tile words start at zero and every call
 * leaves them zero, but calls that overlap on one GPU (two streams, or
 * concurrent graph replays) race and must be serialized by the caller.
 * Other requirements and errors: those of int8_quant_scaled_mm.
 */
w8a8_status_t int8_quant_scaled_mm_noalloc(const uint16_t *x, int64_t ldx, int8_t *xq,
                                           int64_t ldq, float *x_scale, const void *w_packed,
                                           const float *w_scale, const uint16_t *bias, int64_t M,
                                           int64_t N, int64_t K, int mode, void *out, int64_t ldo,
                                           void *stream);

/*
 * int8_quant_scaled_mm_f16 - int8_quant_scaled_mm for fp16 activations x
 * (fp16 bits, [M, ldx]): int8_quant_per_token_f16 of x, then int8_scaled_mm
 * of the result, bit-identical to those two calls. With mode W8A8_OUT_F16
 * (fp16 out, fp16 bias) the single-launch paths of int8_quant_scaled_mm
 * apply; the other modes run the two steps as two launches.
 */
w8a8_status_t int8_quant_scaled_mm_f16(const uint16_t *x, int64_t ldx, int8_t *xq, int64_t ldq,
                                       float *x_scale, const void *w_packed,
                                       const float *w_scale, const uint16_t *bias, int64_t M,
                                       int64_t N, int64_t K, int mode, void *out, int64_t ldo,
                                       void *stream);

/* int8_quant_scaled_mm_f16 with an explicit tile configuration (or -1). */
w8a8_status_t int8_quant_scaled_mm_f16_tile(const uint16_t *x, int64_t ldx, int8_t *xq,
                                            int64_t ldq, float *x_scale, const void *w_packed,
                                            const float *w_scale, const uint16_t *bias,
                                            int64_t M, int64_t N, int64_t K, int mode, void *out,
                                            int64_t ldo, void *stream, int tile);

/* int8_quant_scaled_mm with an explicit tile configuration (or -1). */
w8a8_status_t int8_quant_scaled_mm_tile(const uint16_t *x, int64_t ldx, int8_t *xq, int64_t ldq,
                                        float *x_scale, const void *w_packed,
                                        const float *w_scale, const uint16_t *bias, int64_t M,
                                        int64_t N, int64_t K, int mode, void *out, int64_t ldo,
                                        void *stream, int tile);

/*
 * ---- The FP8 (e4m3) W8A8 twin ----
 * (Page "Online Quantization": FP8 W8A8 is the sibling method of Int8 W8A8
 * in its method and hardware tables, with the "dynamic" activation scheme
 * of its Parameters table.) The pages give no formula for it; this library
 * reads it the way of the int8 path, with OCP e4m3 codes (largest finite
 * value 448, the format the gfx950 fp8 MFMA takes):
 *   per row (token, or output channel) a = max |x|;  a < 2^-100 -> scale 0,
 *   codes 0; else scale = fl32(a/448), inv = fl32(448/a),
 *   code = e4m3(clamp(fl32(x*inv), -448, 448)), nearest-even, sign kept
 *   (zeros too; code 0x80 is -0).
 *   acc[m,n] = sum_k e4m3(xq[m,k]) * e4m3(wq[n,k]) on the fp8 MFMA with fp32
 *   accumulation: unlike the int8 path, the sums depend on the hardware's
 *   summation order (each partial fp32 sum rounded).
 *   out: the epilogue of int8_scaled_mm on acc (same order and modes;
 *   W8A8_OUT_I32 stores the raw fp32 accumulators as 4-byte floats).
 * Codes are uint8 bit patterns. The packed weight uses the layout of
 * int8_prepack_weight (a byte permutation; int8_prepack_weight packs e4m3
 * codes as well). Requirements are those of the int8 counterparts.
 */
w8a8_status_t fp8_quant_per_token(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                                  uint8_t *xq, int64_t ldq, float *x_scale, void *stream);
w8a8_status_t fp8_quant_per_channel(const float *w, int64_t N, int64_t K, int64_t ldw,
                                    uint8_t *wq, int64_t ldq, float *w_scale, void *stream);
/* Online weight quant from bf16 or fp32 straight into the packed layout, as
 * int8_quant_prepack_weight with e4m3 codes. */
w8a8_status_t fp8_quant_prepack_weight(const void *w, int w_dtype, int64_t N, int64_t K,
                                       int64_t ldw, void *w_packed, float *w_scale,
                                       void *stream);
w8a8_status_t fp8_scaled_mm(const uint8_t *xq, int64_t ldq, const float *x_scale,
                            const void *w_packed, const float *w_scale, const uint16_t *bias,
                            int64_t M, int64_t N, int64_t K, int mode, void *out, int64_t ldo,
                            void *stream);
/* fp8_scaled_mm with an explicit tile (0 <= tile < w8a8_fp8_tile_count(): the
 * int8 configurations, same numbers and names, main and small-M) or -1. */
w8a8_status_t fp8_scaled_mm_tile(const uint8_t *xq, int64_t ldq, const float *x_scale,
                                 const void *w_packed, const float *w_scale, const uint16_t *bias,
                                 int64_t M, int64_t N, int64_t K, int mode, void *out, int64_t ldo,
                                 void *stream, int tile);
/* fp8_quant_per_token of bf16 x, then fp8_scaled_mm, writing xq and x_scale
 * too; in one launch where int8_quant_scaled_mm would use one (modes
 * W8A8_OUT_BF16 and W8A8_OUT_I32), else two. */
w8a8_status_t fp8_quant_scaled_mm(const uint16_t *x, int64_t ldx, uint8_t *xq, int64_t ldq,
                                  float *x_scale, const void *w_packed, const float *w_scale,
                                  const uint16_t *bias, int64_t M, int64_t N, int64_t K, int mode,
                                  void *out, int64_t ldo, void *stream);
/* fp8_quant_scaled_mm with an explicit tile (or -1). */
w8a8_status_t fp8_quant_scaled_mm_tile(const uint16_t *x, int64_t ldx, uint8_t *xq, int64_t ldq,
                                       float *x_scale, const void *w_packed,
                                       const float *w_scale, const uint16_t *bias, int64_t M,
                                       int64_t N, int64_t K, int mode, void *out, int64_t ldo,
                                       void *stream, int tile);
int w8a8_fp8_tile_count(void);
int w8a8_fp8_tile_auto(int64_t M, int64_t N, int64_t K);

/* Number of tile configurations, a short name of one, and the tile the
 * automatic choice picks for a shape. Main kernel: "128x192/m1n2k2/l33" is
 * tile rows x columns / wave row groups, column groups and k-groups / token
 * and weight fetch leads in stages. Small-M kernel (for a few token rows; the
 * automatic choice considers it up to 32 rows): "s16x32/k8/u4" is token rows
 * x channels per workgroup / wavefronts splitting K / k-blocks per load
 * group. */
int w8a8_mm_tile_count(void);
const char *w8a8_mm_tile_name(int tile);
int w8a8_mm_tile_auto(int64_t M, int64_t N, int64_t K);

/* Bound on the polls (about 1 us each; default 4096) that a workgroup of the
 * one-launch path of int8_quant_scaled_mm / fp8_quant_scaled_mm makes for
 * the producers of its tile's rows before it quantizes those rows itself.
 * For tests and diagnosis: 0 sends every workgroup down that path at once,
 * with results unchanged. polls >= 0 sets the bound for launches made after
 * the call (process wide, every device) and returns the previous bound; a
 * negative value only returns the current one. */
int w8a8_fused_wait_limit(int polls);

/* 1 when `device` is a gfx950 GPU this library can run on, else 0. */
int w8a8_device_supported(int device);

/* Static description of a status code. */
const char *w8a8_status_string(int status);

/* Thread-local detail of the most recent error returned on this thread
 * (argument name, HIP error string); "" when there is none. */
const char *w8a8_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */
