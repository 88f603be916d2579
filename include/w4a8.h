/*
 * w4a8.h -- C ABI of the MI355X (gfx950) W4A8 linear-layer library, libw4a8.so.
 *
 * The method (page keys as in the design notes):
 *   [p1] "Kimi 2.7 MoE: from 4-bit storage to INT8 compute" (hotelren.com/news/5173946)
 *   [p2] "Kimi 2.7 MoE, 4-bit storage to INT8, dissected"   (pptc.cn/news/121597)
 *   [p3] "LLM quantization primer"                            (hotelren.com/news/5982361)
 *   [p4] "MoE deployment: active parameters are not the storage bill" (feinterview.poetries.top)
 *
 * Weights W[N][K] (row n = output feature n, the nn.Linear out x in layout) are
 * quantized in groups of 128 consecutive K entries per output feature, each
 * group with an fp16 scale and an fp16 zero point ([p2 §2.1, §2.2, §2.3]):
 *     scale = (max - min) / 15, zp = round(-min / scale),
 *     q = clamp(round(w / scale) + zp, 0, 15),   w ~ (q - zp) * scale,
 * where [min, max] is the group's range widened to contain 0, rounding is to
 * nearest-even, and q is computed with the fp16-rounded scale.  Two codes share
 * a byte, the first (lower k) in the low nibble ([p2 §2.2]).
 *
 * Activations x[M][K] are quantized per token to symmetric INT8 at run time
 * ([p1 §3.1, §5.3]; [p3 §2.1]): s_m = max_k |x[m][k]| / 127,
 * qa = clamp(rint(x / s_m), -127, 127); a row with s_m == 0 gets codes 0.
 *
 * The product is an INT8 x INT8 matmul with int32 accumulation per group,
 * followed by a floating-point epilogue ([p2 §3.2, §5.4]; [p1 §4.3]):
 *     isum[g][m][n] = sum_{k in g} qa[m][k] * (q[n][k] - zp[g][n])
 *     out[m][n]     = s_m * sum_g scale[g][n] * isum[g][m][n]      (fp32)
 *
 * Layouts (all row-major, C-contiguous):
 *     W        fp32  [N][K]
 *     packed   u8    [N][K/2]      byte (n, j) = q[n][2j] | q[n][2j+1] << 4
 *     scale    u16   [K/128][N]    fp16 bit patterns
 *     zp       u16   [K/128][N]    fp16 bit patterns of integers 0..15
 *     qa       i8    [M][K],  a_scale fp32 [M]
 *     out      fp32  [M][N]
 * MoE weights stack E experts: packed [E][N][K/2], scale/zp [E][K/128][N].
 *
 * Conventions for every entry point:
 *   - Return codes only; nothing throws or aborts across the ABI.  Arguments
 *     are validated on the host before anything is launched; a rejected call
 *     launches nothing and writes nothing.  w4a8_last_error() then describes
 *     the problem (thread-local text, valid until the next call on the thread).
 *   - group is 128 unless an entry point says otherwise (the packers, the GEMM
 *     and expert-grouped GEMM entry points and their debug forms also take 64
 *     and 256; the tile-major layout and the MoE layer take 128 only);
 *     any other value is W4A8_EUNSUPPORTED, with no fallback.  K must be a
 *     multiple of 128 (W4A8_EINVAL; pad K at conversion time).
 *   - Device pointers (marked "device") must be device memory owned by the
 *     caller; the library allocates nothing and keeps no pointer after the
 *     call returns.  Device calls are asynchronous on `stream` (NULL = the
 *     default stream); a fault inside a kernel surfaces at the caller's next
 *     synchronisation.  A failed launch returns W4A8_EHIP.
 *   - Packed weights, qa and out must be 16-byte aligned (W4A8_EINVAL).
 *   - Results are deterministic: identical inputs give identical output bytes
 *     (no floating-point atomics anywhere).
 *   - Non-finite activations give unspecified codes (no error is raised on the
 *     device); the host packer rejects non-finite weights.
 */
#ifndef W4A8_H
#define W4A8_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W4A8_OK = 0,
    W4A8_EINVAL = 1,        /* bad pointer, size, alignment or value */
    W4A8_EUNSUPPORTED = 2,  /* valid request this library does not implement (e.g. group != 128) */
    W4A8_EHIP = 3,          /* a HIP runtime call or kernel launch failed */
    W4A8_EWORKSPACE = 4     /* the caller's workspace is smaller than the call needs */
} w4a8_status;

#define W4A8_ABI_VERSION 6
#define W4A8_GROUP 128

int w4a8_abi_version(void);
const char *w4a8_status_str(int status);
const char *w4a8_last_error(void);

/* ------------------------------------------------------------------ packing */

/* Host, synchronous.  Quantizes W[N][K] (host fp32) into packed codes and fp16
 * scale/zero point per group, exactly as stated at the top of this file
 * ([p2 §2.1, §2.2]).  All pointers are host memory owned by the caller.
 * A group whose scale rounds to 0 in fp16 stores scale 1.0 and zp 0.
 * group is 128, 64 or 256 ([p2 §4.3] weighs the three); scale/zp are then
 * [K/group][N].
 * Errors: W4A8_EINVAL for null pointers, N <= 0, K <= 0, K % 128 != 0,
 * K % group != 0, non-finite weights, or a group scale above the largest finite
 * fp16; W4A8_EUNSUPPORTED for another group size. */
w4a8_status w4a8_pack_weights(const float *W, int64_t N, int64_t K, int32_t group,
                              uint8_t *packed, uint16_t *scale, uint16_t *zp);

/* Host, synchronous.  Packer variants in the same stored format, so every GEMM entry
 * point takes their output unchanged:
 *   mode W4A8_PACK_ASYMMETRIC: the packer above.
 *   mode W4A8_PACK_SYMMETRIC: zero point fixed at 0 ([p2 §2.1] names it as the
 *     simpler choice; [p3 §2.1] gives the b-bit form scale = max|w| / (2^(b-1) - 1)):
 *     scale = fp16(max|w| / 7) per group, q = clamp(round(w / scale), -7, 7), stored as
 *     code q + 8 with zp 8, so that (code - zp) = q.
 *   clip_percent p in [50, 100] ([p2 §2.2, §5.1]: the range comes from percentiles, not
 *     the extremes, and weights past them are cut back): each output column's K
 *     weights are clamped to their own [100 - p, p] percentiles (linear interpolation
 *     between order statistics at position (K - 1) * pct / 100, in double, rounded to
 *     fp32) before the group quantizer.  p = 100 leaves the weights as they are.
 * Host memory owned by the caller.  Errors as w4a8_pack_weights, plus W4A8_EINVAL for an
 * unknown mode or p outside [50, 100]. */
#define W4A8_PACK_ASYMMETRIC 0
#define W4A8_PACK_SYMMETRIC 1
w4a8_status w4a8_pack_weights_ex(const float *W, int64_t N, int64_t K, int32_t group, int32_t mode,
                                 double clip_percent, uint8_t *packed, uint16_t *scale, uint16_t *zp);

/* Device, asynchronous.  The same quantization as w4a8_pack_weights, run on the
 * GPU for W (device fp32 [N][K]) -- for weight sets too large to convert on the
 * host.  Bit-identical to the host packer.  Device memory only.  Errors as the
 * host packer for sizes; non-finite weights or fp16 scale overflow cannot be
 * reported from the device: such groups get scale 0x7C00 (inf) and must be
 * checked by the caller if the input is untrusted.  W 8-byte aligned (16-byte
 * for group 256), packed 2-byte aligned. */
w4a8_status w4a8_pack_weights_device(const float *W, int64_t N, int64_t K, int32_t group,
                                     uint8_t *packed, uint16_t *scale, uint16_t *zp,
                                     hipStream_t stream);

/* Host, synchronous.  Inverse view of a packed weight: q_out[N][K] receives the
 * 4-bit codes (may be NULL) and w_hat[N][K] the dequantized fp32 values
 * (q - zp) * scale (may be NULL) [p2 §2.1].  Host memory. */
w4a8_status w4a8_unpack_weights(const uint8_t *packed, const uint16_t *scale, const uint16_t *zp,
                                int64_t N, int64_t K, int32_t group, uint8_t *q_out, float *w_hat);

/* -------------------------------------------------------- activation quant */

/* Device.  Per-token symmetric INT8 quantization of x (rows of length K, row
 * stride ldx >= K floats) into qa[M][K] and a_scale[M] ([p1 §5.3]: the scale is
 * computed in the kernel at forward time; [p3 §2.1]: symmetric INT8 form).
 * Division and rounding are IEEE fp32 (correctly rounded divide, ties-to-even).
 * Errors: W4A8_EINVAL for null pointers, M < 0, K <= 0, ldx < K, or qa not
 * 16-byte aligned, or K % 16 != 0.  M == 0 is a no-op. */
w4a8_status w4a8_quantize_act(const float *x, int64_t M, int64_t K, int64_t ldx,
                              int8_t *qa, float *a_scale, hipStream_t stream);

/* ------------------------------------------------- per-channel smoothing
 * [p3 §3.4] (quantization-friendly transforms): a positive factor s_k per input
 * channel moves part of the activations' outlier range into the weights; the
 * layer's product is unchanged because x_k * W[n][k] = (x_k / s_k) * (W[n][k] * s_k).
 * The page names the idea without a formula; this library reads it as
 *   ax_k = max over calibration rows of |x[r][k]|,  aw_k = max over n of |W[n][k]|,
 *   s_k  = ax_k^alpha / aw_k^(1 - alpha)  (double, rounded to fp32; 1 where
 *          ax_k or aw_k is 0),  inv_s_k = fp32(1 / s_k),
 * weights quantized as fp32(W[n][k] * s_k) and activations as fp32(x[m][k] * inv_s_k).
 * The GEMM entry points take the results unchanged. */

/* Device, asynchronous.  out[k] = max over r < rows of |A[r][k]| for a row-major
 * A (row stride lda >= K floats); rows == 0 gives 0 (A may then be NULL).  Exact
 * (a maximum has no rounding) and deterministic.  Device memory.  Errors:
 * W4A8_EINVAL for null pointers, rows < 0, K <= 0 or lda < K. */
w4a8_status w4a8_channel_absmax(const float *A, int64_t rows, int64_t K, int64_t lda, float *out,
                                hipStream_t stream);

/* Host, synchronous.  s[K] and inv_s[K] from the channel maxima ax[K] (activations)
 * and aw[K] (weights) with migration strength alpha in [0, 1], as stated above.
 * Host memory owned by the caller.  Errors: W4A8_EINVAL for null pointers, K <= 0,
 * alpha outside [0, 1], a negative or non-finite maximum, or a factor that is not
 * a positive finite fp32 (extreme ratios of the two maxima). */
w4a8_status w4a8_smooth_factors(const float *ax, const float *aw, int64_t K, double alpha,
                                float *s, float *inv_s);

/* Device, asynchronous.  w4a8_pack_weights_device of the smoothed weights
 * fp32(W[n][k] * s[k]) (s: device fp32 [K]); the smoothed matrix is not stored.
 * W and s 8-byte aligned (16-byte for group 256).  Errors as
 * w4a8_pack_weights_device. */
w4a8_status w4a8_pack_weights_device_smooth(const float *W, int64_t N, int64_t K, int32_t group,
                                            const float *s, uint8_t *packed, uint16_t *scale,
                                            uint16_t *zp, hipStream_t stream);

/* Device, asynchronous.  w4a8_quantize_act of the smoothed rows fp32(x[m][k] *
 * inv_s[k]) (inv_s: device fp32 [K]); the row maximum and the codes are taken of
 * those products and the scaled rows are never written out.  Errors as
 * w4a8_quantize_act, plus a null inv_s. */
w4a8_status w4a8_quantize_act_smooth(const float *x, int64_t M, int64_t K, int64_t ldx,
                                     const float *inv_s, int8_t *qa, float *a_scale,
                                     hipStream_t stream);

/* --------------------------------------------------------------------- GEMM */

/* Device.  out[M][N] = W4A8 linear layer of the quantized activations with the
 * packed weights (formula at the top; [p2 §3.2]: INT8 matmul with int32
 * accumulation, then multiply by the scales; [p1 §4.3 step 2]: the 4-bit codes
 * are widened to INT8 inside the kernel, never in memory).  Small M takes an
 * HBM-streaming path, large M an LDS-tiled MFMA path; both give the same
 * per-group int32 sums.  The fp32 epilogue adds groups in increasing g.
 * Group sizes 64 and 256 take the decode loop for 1 <= M <= 16 when K % 256 == 0
 * (and its size limits hold) and the tiled loop otherwise: 256 keeps one int32
 * sum over its two 128-k halves, 64 takes two sums per half.
 * Errors: W4A8_EINVAL (null, M < 0, N <= 0, K <= 0, K % 128, K % group,
 * N % 16 != 0, misalignment), W4A8_EUNSUPPORTED (group not 64, 128 or 256; 64
 * or 256 with path 1 forced outside the decode loop's range).  M == 0 is a
 * no-op. */
w4a8_status w4a8_gemm(const int8_t *qa, const float *a_scale, int64_t M, int64_t K,
                      const uint8_t *packed, const uint16_t *scale, const uint16_t *zp,
                      int64_t N, int32_t group, float *out, hipStream_t stream);

/* Device, test/debug aid.  Same main loop as w4a8_gemm, but instead of the fp32
 * epilogue it stores every per-group int32 sum: isums[K/group][M][N] ([p2 §5.4]).
 * `path` selects the main loop: 0 = the one w4a8_gemm would pick for M,
 * 1 = the small-M streaming loop (M <= 64; for group 64 or 256, the decode loop,
 * M <= 16), 2 = the large-M tiled loop with the tile w4a8_gemm would pick,
 * 3 = tiled with 128x128 workgroup tiles, 4 = tiled with 256x128 workgroup tiles,
 * 5 = tiled with 256x256 workgroup tiles (group 128; 256x128 for 64 and 256). */
w4a8_status w4a8_gemm_debug_isums(const int8_t *qa, int64_t M, int64_t K,
                                  const uint8_t *packed, const uint16_t *zp, int64_t N,
                                  int32_t group, int32_t path, int32_t *isums, hipStream_t stream);

/* Same as w4a8_gemm with a forced main loop (`path` as above); for tests and
 * benchmarks that compare the two loops on one shape. */
w4a8_status w4a8_gemm_path(const int8_t *qa, const float *a_scale, int64_t M, int64_t K,
                           const uint8_t *packed, const uint16_t *scale, const uint16_t *zp,
                           int64_t N, int32_t group, int32_t path, float *out, hipStream_t stream);

/* --------------------------------------------- tile-major weights (decode) */

/* The same codes, scales and zero points as the standard layout, reordered
 * offline so that the decode GEMM (M <= 16, where the weights are the whole cost:
 * [p1 §4.3] on decode being bound by the weight stream) reads each weight byte in
 * one contiguous stream per wave.  This is only a storage order; the arithmetic
 * is that of w4a8_gemm.  For N % 16 == 0 and K % 256 == 0, with G = K/128:
 *     tm  u8  [N/16][G/2][2176]   block (t, w) for columns 16t..16t+15 and groups
 *                                 2w, 2w+1:
 *       bytes [1024h, 1024h + 1024), h = 0, 1: group 2w+h; the 16 bytes at 16l
 *           (l = 0..63) hold the codes k = 32*(l >> 4) + [0, 32) of that group for
 *           column 16t + (l & 15), each run of 8 codes c0..c7 (in k order) as the
 *           4 bytes c_b | c_(b+4) << 4, b = 0..3
 *       bytes [2048, 2176): 8 bytes per column c = 0..15 at 2048 + 8c: the fp16
 *           scale[2w][16t + c] and scale[2w + 1][16t + c], then the bytes -zp
 *           (two's complement int8) of groups 2w and 2w + 1, then two zero bytes
 * Total size: N*K/2 + 4*N*(K/128) bytes, the same as packed + scale + zp. */

/* Bytes of the tile-major array for an N x K weight (0 if N % 16 or K % 256). */
size_t w4a8_tm_bytes(int64_t N, int64_t K);

/* Device, asynchronous.  Writes the tile-major array `tm` (device, 16-byte
 * aligned, w4a8_tm_bytes(N, K) bytes) from standard-layout device weights.
 * Errors: W4A8_EINVAL (null, N % 16 != 0, K % 256 != 0, misalignment),
 * W4A8_EUNSUPPORTED (group != 128). */
w4a8_status w4a8_weights_to_tm(const uint8_t *packed, const uint16_t *scale, const uint16_t *zp,
                               int64_t N, int64_t K, int32_t group, uint8_t *tm,
                               hipStream_t stream);

/* Device.  out[M][N] as w4a8_gemm, with the weights in the tile-major array.
 * M <= 16 runs the decode loop: output bytes identical to w4a8_gemm's for the same
 * weights.  M > 16 runs the 256x256 tiled loop, where the tile-major nibble order
 * spares the unpack its byte permutes: output bytes identical to w4a8_gemm_path's
 * path 5 (the same loop over the standard layout).  Besides w4a8_gemm's conditions
 * it needs K % 256 == 0, a tile-major array below 4 GiB, and M * (K + 16) <= 143360
 * (the staged activation rows) for M <= 16 or M * K < 2^32 above; anything else
 * is W4A8_EINVAL.  M == 0 is a no-op. */
w4a8_status w4a8_gemm_tm(const int8_t *qa, const float *a_scale, int64_t M, int64_t K,
                         const uint8_t *tm, int64_t N, int32_t group, float *out,
                         hipStream_t stream);

/* ---------------------------------------------------------------------- MoE */

/* Device.  Router for T tokens over E experts ([p1 §5.2]: the router stays in
 * high precision and sends each token to its experts; [p4]: toy top-1 model).
 *   topk_ids[T][k]  the k largest logits per token, descending, ties -> lower id
 *   topk_w[T][k]    softmax over the k selected logits (fp32)
 *   expert_offsets[E+1+with_shared]  exclusive scan of the per-expert pair
 *                   counts; with with_shared = 1 a shared expert (index E) that
 *                   every token visits follows: expert_offsets[E+1] = T*k + T
 *   perm[T*k]       pair indices p = t*k + j grouped by ascending expert and,
 *                   within an expert, ascending p ("slot" s holds pair perm[s])
 *   slot_row[T*k + with_shared*T]  (may be NULL) the activation row of each
 *                   slot: perm[s] / k for routed slots, s - T*k for the shared
 *                   expert's slots -- the row_index of w4a8_moe_grouped_gemm
 *   slot_of_pair[T*k]  the inverse of perm
 * logits: device fp32 [T][E].  Requires 1 <= k <= min(E, 8), E <= 1024,
 * with_shared in {0, 1} and T*k + T < 2^31.  With T == 0 only expert_offsets is
 * written (all zeros) and the other pointers may be NULL.  The bucketing runs in
 * one workgroup, in chunks of pairs taken in increasing p, which is what makes
 * the order within an expert stable.
 * Errors: W4A8_EINVAL (null, T < 0, bad E/k/with_shared). */
w4a8_status w4a8_moe_route(const float *logits, int64_t T, int32_t E, int32_t topk,
                           int32_t with_shared, int32_t *topk_ids, float *topk_w,
                           int32_t *expert_offsets, int32_t *perm, int32_t *slot_row,
                           int32_t *slot_of_pair, hipStream_t stream);

/* Device.  Expert-grouped W4A8 GEMM.  Slots s in [expert_offsets[e],
 * expert_offsets[e+1]) belong to expert e; slot s multiplies activation row
 * row_index[s] (qa/a_scale row; row_index NULL means row s) with expert e's
 * packed weights, and writes out[s][0..N).  The per-expert slot counts stay on
 * the device: the kernel reads expert_offsets itself, so no host round trip
 * is needed between routing and the GEMM.  Each expert takes the loop for its
 * slot count: a streaming loop over 16-row chunks (up to 16 slots), one weight
 * pass per 64 rows (17 to 128), or the tiled loop (more); a loop is launched only
 * when max_slots allows an expert of its size.  (When K/128 is not a multiple of
 * 4, or below 8, the streaming loop takes up to 64 slots and the tiled loop the
 * rest.)  Group sizes 64 and 256: the 16-row loop up to 16 slots (when K/128 is
 * a multiple of 4), the tiled loop above.
 *   qa [R][K] i8 and a_scale [R] (R = rows of the activation matrix),
 *   packed [E][N][K/2], scale/zp [E][K/group][N], out [max_slots][N].
 * The caller guarantees expert_offsets[E] <= max_slots and row_index[s] < R
 * (the kernel clamps slots to max_slots and skips slots whose row_index is
 * outside [0, R)).  Errors as w4a8_gemm, plus E <= 0. */
w4a8_status w4a8_moe_grouped_gemm(const int8_t *qa, const float *a_scale, int64_t R,
                                  const int32_t *row_index, const int32_t *expert_offsets,
                                  int32_t E, int64_t K, const uint8_t *packed,
                                  const uint16_t *scale, const uint16_t *zp, int64_t N,
                                  int32_t group, int64_t max_slots, float *out,
                                  hipStream_t stream);

/* Device, test/debug aid.  The main loops of w4a8_moe_grouped_gemm (each expert
 * takes the loop its slot count selects, as above), but instead of the fp32
 * epilogue every per-group int32 sum is stored ([p2 §3.2, §5.4]: INT8 products
 * accumulated in int32 per group):
 *     isums[g][s][n] = sum_{k in group g} qa[row_index[s]][k] * (q_e[n][k] - zp_e[g][n])
 * for g < K/group, slots s < max_slots of expert e, n < N; isums is device int32
 * [K/group][max_slots][N], caller-owned.  Slots past expert_offsets[E] are not
 * written; slots whose row_index is outside [0, R) get unspecified values.  No
 * scale array is read.  Errors as w4a8_moe_grouped_gemm. */
w4a8_status w4a8_moe_grouped_gemm_debug_isums(const int8_t *qa, int64_t R, const int32_t *row_index,
                                              const int32_t *expert_offsets, int32_t E, int64_t K,
                                              const uint8_t *packed, const uint16_t *zp, int64_t N,
                                              int32_t group, int64_t max_slots, int32_t *isums,
                                              hipStream_t stream);

/* Device.  MoE expert activation then per-row re-quantization to INT8:
 * h = silu(gate) * up with gate = gu[p][0..I), up = gu[p][I..2I),
 * silu(v) * u = v * (1 / (1 + 2^(-v log2 e))) * u in fp32 with the hardware
 * base-2 exponential and reciprocal (about 1 ulp each, relative error a few 1e-7;
 * the pages fix no precision for the activation); then the per-token quantizer
 * above on each row of h: qh[P][I], h_scale[P].  h_out[P][I] (optional, may be
 * NULL) receives the fp32 h that was quantized.  Errors: W4A8_EINVAL (null,
 * P < 0, I <= 0, I % 16). */
w4a8_status w4a8_silu_mul_quantize(const float *gu, int64_t P, int64_t I, int8_t *qh,
                                   float *h_scale, float *h_out, hipStream_t stream);

/* Device.  Weighted combine of expert outputs back to tokens:
 * out[t][c] = sum_{j<k} topk_w[t][j] * y[slot_of_pair[t*k+j]][c] + y_shared[t][c]
 * (y_shared may be NULL), summed in fp32 in the order j = 0..k-1, then shared.
 * y [S][H], out [T][H] fp32.  Errors: W4A8_EINVAL (null, T < 0, H <= 0, k <= 0). */
w4a8_status w4a8_moe_combine(const float *y, const int32_t *slot_of_pair, const float *topk_w,
                             const float *y_shared, int64_t T, int32_t topk, int64_t H,
                             float *out, hipStream_t stream);

/* ------------------------------------------------------------ MoE FFN layer */

/* The whole expert FFN of one MoE layer in one call (the composition the
 * entry points above provide, [p1 §5.1-§5.3]: route in high precision, quantize
 * the tokens once, group them by expert, run the experts' W4A8 products):
 *   1. w4a8_moe_route (with_shared = 1)          logits [T][E]
 *   2. w4a8_quantize_act                         x [T][H] -> qa, a_scale
 *   3. w4a8_moe_grouped_gemm, E+1 experts        gate/up weights [E+1][2I][H/2]
 *   4. w4a8_silu_mul_quantize                    gu [S][2I] -> qh [S][I], h_scale
 *   5. w4a8_moe_grouped_gemm, E+1 experts        down weights [E+1][H][I/2]
 *   6. w4a8_moe_combine (y_shared = the shared expert's rows)  -> out [T][H]
 * with S = T*k + T slots (routed pairs, then one shared slot per token).
 * Expert E of each weight stack is the shared expert.  Steps 3-4 and 5-6 are partly
 * fused ([p1 §4.3]: the dequant/requant around the INT8 product stays in registers):
 *   - an expert with more than 128 slots runs its gate/up product on the tiled loop
 *     with SiLU(gate) * up in the epilogue.  Its gu lines then hold h [I] and, after
 *     it, the largest |h| of each 16 columns [I/16] instead of gate | up (h is
 *     bit-identical to step 4's own h of those gate/up rows), and the requant takes
 *     the row maximum from those maxima.  Other experts' lines hold gate | up.
 *   - with T > 128 the shared expert's down product runs after the routed experts'
 *     with the combine in its epilogue.  The layer output is the same bits as step 6,
 *     and the shared expert's rows are still written to y.
 * The intermediates live in
 * the caller's workspace (device memory, at least w4a8_moe_ffn_workspace_size
 * bytes, 256-byte aligned); w4a8_moe_ffn_workspace_layout gives each part's byte
 * offset in it (enum w4a8_moe_ws_part order), so a caller can read any stage.
 * Errors: as the steps, W4A8_EINVAL for H or I not multiples of 128 and for a
 * misaligned workspace, W4A8_EWORKSPACE when ws_bytes is too small. */
enum w4a8_moe_ws_part {
    W4A8_WS_TOPK_IDS = 0, W4A8_WS_TOPK_W, W4A8_WS_OFFSETS, W4A8_WS_PERM, W4A8_WS_SLOT_ROW,
    W4A8_WS_SLOT_OF_PAIR, W4A8_WS_QA, W4A8_WS_A_SCALE, W4A8_WS_GU, W4A8_WS_QH, W4A8_WS_H_SCALE,
    W4A8_WS_Y, W4A8_WS_PARTS
};
size_t      w4a8_moe_ffn_workspace_size(int64_t T, int64_t H, int64_t I, int32_t E, int32_t topk);
w4a8_status w4a8_moe_ffn_workspace_layout(int64_t T, int64_t H, int64_t I, int32_t E, int32_t topk,
                                          int64_t *offsets /* [W4A8_WS_PARTS + 1], host */);
w4a8_status w4a8_moe_ffn(const float *x, const float *logits, int64_t T, int64_t H, int64_t I,
                         int32_t E, int32_t topk,
                         const uint8_t *gu_packed, const uint16_t *gu_scale, const uint16_t *gu_zp,
                         const uint8_t *dn_packed, const uint16_t *dn_scale, const uint16_t *dn_zp,
                         float *out, void *workspace, size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): w4a8_moe_ffn with its
 * intermediates in a fixed scratch array inside the library instead of a caller
 * workspace.  The array holds w4a8_moe_ffn_noalloc_max_bytes() bytes (64 MiB) on
 * each GPU the library runs on, from the library's load until the process ends;
 * layers whose w4a8_moe_ffn_workspace_size exceeds it are rejected with
 * W4A8_EWORKSPACE (at H=7168, I=2048, E=384, top-8 that is T above 155 tokens).
 * Arguments, results and errors otherwise as w4a8_moe_ffn; `stream` must belong to
 * the current device.  The call allocates nothing.  Every call on one GPU uses the
 * same array, which keeps the last call's contents: calls that overlap on one GPU
 * (other streams, other host threads) race, and the caller must order them. */
size_t      w4a8_moe_ffn_noalloc_max_bytes(void);
w4a8_status w4a8_moe_ffn_noalloc(const float *x, const float *logits, int64_t T, int64_t H, int64_t I,
                                 int32_t E, int32_t topk,
                                 const uint8_t *gu_packed, const uint16_t *gu_scale, const uint16_t *gu_zp,
                                 const uint8_t *dn_packed, const uint16_t *dn_scale, const uint16_t *dn_zp,
                                 float *out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A8_H */
