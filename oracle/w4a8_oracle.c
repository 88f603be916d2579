/*
 * w4a8_oracle.c -- plain, slow CPU oracle for the W4A8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or the library built from it; only the test suite, the
 * smoke check and the benchmark's cpu_baseline leg do.  It shares no code,
 * header, table or helper with the HIP library.
 *
 * Every function restates, as directly as possible, what the source pages
 * say the method computes.  Page keys used in the citations:
 *   [p1] "Kimi 2.7 MoE: from 4-bit storage to INT8 compute" (hotelren.com/news/5173946)
 *   [p2] "Kimi 2.7 MoE, 4-bit storage to INT8, dissected"   (pptc.cn/news/121597)
 *   [p3] "LLM quantization primer"                            (hotelren.com/news/5982361)
 *   [p4] "MoE deployment: active parameters are not the storage bill"
 *        (feinterview.poetries.top, Kimi K3.1 Pro article)
 *
 * Floating point: fp32 steps are single IEEE-754 binary32 operations
 * (compiled with -ffp-contract=off, no fast-math), so the quantizer's integer
 * decisions are taken in fp32 exactly as written.  Reference outputs of the
 * epilogue are evaluated in double.
 *
 * Readings of points the pages leave open (each is listed in the design notes):
 *   - "round" is round-half-to-even (rint in the default rounding mode).
 *   - The weight range [lo, hi] always contains 0, so zp lands in [0, 15] and
 *     (q - zp) lies in [-15, 15].
 *   - The weight codes are computed with the fp16-rounded scale that is stored,
 *     so quantization and dequantization use one and the same scale.
 *   - A group whose scale rounds to 0 in fp16 stores scale 1.0, zp 0.
 *   - An activation row whose scale is 0 (all-zero row, or max|x|/127 underflows
 *     in fp32) has codes 0.
 *   - A group whose scale exceeds the largest finite fp16 is an error.
 *   - Symmetric weights (O9) keep the stored format: code q + 8 with zp 8.
 *   - Percentile clipping (O10) is per output column over its K weights,
 *     linear interpolation between order statistics, both tails.
 *   - Smoothing (O8): s_k = ax_k^alpha / aw_k^(1-alpha) from the channel maxima
 *     of calibration activations and of the weights (1 where either is 0),
 *     rounded to fp32; inv_s_k = fp32(1 / s_k); weights multiplied by s and
 *     activations by inv_s, one fp32 product each, before the quantizers.
 *
 * Parity pins: see tests/test_oracle_pins.py.  Every function here is pinned
 * by at least one test against values the pages print, closed forms, brute
 * force on tiny inputs, or an independent library route.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

/* ------------------------------------------------------------------------ */
/* IEEE-754 binary16 <-> binary32, written from the format's definition:    */
/* 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; subnormals have */
/* value frac * 2^-24; conversion rounds to nearest, ties to even.          */
/* [p2 §2.3] stores one fp16 scale and one fp16 zero point per group.       */
/* ------------------------------------------------------------------------ */
uint16_t orc_f32_to_f16(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, 4);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    if (isnan(f))
        return (uint16_t)(sign | 0x7E00u);
    double a = fabs((double)f);
    if (isinf(f) || a >= 65520.0) /* 65520 is the halfway point above 65504 */
        return (uint16_t)(sign | 0x7C00u);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: value = n * 2^-24, n in [0, 1024]; n = 1024 is the
           smallest normal number and gets the right encoding automatically */
        double n = rint(ldexp(a, 24)); /* exact scaling, then ties-to-even */
        return (uint16_t)(sign | (uint16_t)n);
    }
    int e;
    double m = frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
    m *= 2.0;
    e -= 1; /* a = m * 2^e, m in [1, 2) */
    double frac = rint((m - 1.0) * 1024.0); /* exact product, ties-to-even */
    if (frac == 1024.0) {
        frac = 0.0;
        e += 1;
    }
    if (e + 15 >= 31)
        return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)frac);
}

float orc_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1F;
    int fr = h & 0x3FF;
    double v;
    if (ex == 0)
        v = ldexp((double)fr, -24);
    else if (ex == 31)
        v = fr ? NAN : INFINITY;
    else
        v = ldexp(1.0 + fr / 1024.0, ex - 15);
    return (float)(sign ? -v : v);
}

/* ------------------------------------------------------------------------ */
/* O1: asymmetric 4-bit weight quantization, one (scale, zero point) per    */
/* group of `group` consecutive K entries of one output column.             */
/* [p2 §2.1] group quantization with a scale and a zero point per group of  */
/* 128; [p2 §2.2] scale = (max-min)/(2^4-1), zero_point = round(-min/scale),*/
/* index = round(w/scale) + zero_point clamped to 0..15.                    */
/*                                                                          */
/* W: [N][K] fp32 (row n = output column n).  q: [N][K] codes (one per     */
/* byte).  scale16/zp16: [K/group][N] fp16 bit patterns.                    */
/* Returns 0, or -1 for bad sizes / non-finite input / fp16 scale overflow. */
/* ------------------------------------------------------------------------ */
int orc_quantize_weights(const float *W, int64_t N, int64_t K, int64_t group,
                         uint8_t *q, uint16_t *scale16, uint16_t *zp16)
{
    if (N <= 0 || K <= 0 || group <= 0 || K % group != 0)
        return -1;
    int64_t G = K / group;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            const float *w = W + n * K + g * group;
            float lo = 0.0f, hi = 0.0f; /* the range always contains 0 */
            for (int64_t i = 0; i < group; ++i) {
                if (!isfinite(w[i]))
                    return -1;
                if (w[i] < lo)
                    lo = w[i];
                if (w[i] > hi)
                    hi = w[i];
            }
            float s32 = (hi - lo) / 15.0f;
            uint16_t sh = orc_f32_to_f16(s32);
            if ((sh & 0x7FFFu) == 0x7C00u)
                return -1; /* scale not representable in fp16 */
            float s = orc_f16_to_f32(sh);
            if (s == 0.0f) {
                sh = 0x3C00u; /* 1.0 */
                s = 1.0f;
            }
            float zf = rintf(-lo / s);
            if (zf < 0.0f)
                zf = 0.0f;
            if (zf > 15.0f)
                zf = 15.0f;
            int zp = (int)zf;
            scale16[g * N + n] = sh;
            zp16[g * N + n] = orc_f32_to_f16((float)zp);
            for (int64_t i = 0; i < group; ++i) {
                int v = (int)rintf(w[i] / s) + zp;
                if (v < 0)
                    v = 0;
                if (v > 15)
                    v = 15;
                q[n * K + g * group + i] = (uint8_t)v;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O9: symmetric 4-bit weights [p3 §2.1] (zero point fixed at 0; scale =    */
/* max|w| / (2^(b-1) - 1) = max|w| / 7; q = round(w / scale) in [-7, 7]),   */
/* [p2 §2.1] names it as the simpler alternative.  Stored in the same       */
/* format as O1 so that every GEMM serves it: code = q + 8, zp = 8, so that  */
/* code - zp = q.  fp16 scale rules as O1 (codes use the stored scale; a     */
/* scale that rounds to 0 stores 1.0; an fp16 overflow is an error).         */
/* ------------------------------------------------------------------------ */
int orc_quantize_weights_sym(const float *W, int64_t N, int64_t K, int64_t group,
                             uint8_t *q, uint16_t *scale16, uint16_t *zp16)
{
    if (N <= 0 || K <= 0 || group <= 0 || K % group != 0)
        return -1;
    int64_t G = K / group;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            const float *w = W + n * K + g * group;
            float amax = 0.0f;
            for (int64_t i = 0; i < group; ++i) {
                if (!isfinite(w[i]))
                    return -1;
                if (fabsf(w[i]) > amax)
                    amax = fabsf(w[i]);
            }
            uint16_t sh = orc_f32_to_f16(amax / 7.0f);
            if ((sh & 0x7FFFu) == 0x7C00u)
                return -1;
            float s = orc_f16_to_f32(sh);
            if (s == 0.0f) {
                sh = 0x3C00u;
                s = 1.0f;
            }
            scale16[n + g * N] = sh;
            zp16[n + g * N] = orc_f32_to_f16(8.0f);
            for (int64_t i = 0; i < group; ++i) {
                float r = rintf(w[i] / s);
                if (r < -7.0f)
                    r = -7.0f;
                if (r > 7.0f)
                    r = 7.0f;
                q[n * K + g * group + i] = (uint8_t)((int)r + 8);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O10: percentile range clipping [p2 §2.2, §5.1]: the range is taken from   */
/* percentiles instead of the minimum and maximum, and weights beyond the    */
/* percentile are cut back to it.  Reading: per output column n, over its K  */
/* weights, the p-th and (100-p)-th percentiles with linear interpolation    */
/* between order statistics (position h = (K-1) * pct / 100,                 */
/* v[floor h] + (h - floor h) * (v[floor h + 1] - v[floor h]), in double),   */
/* rounded to fp32; every weight is clamped to [lo, hi] before O1 or O9.     */
/* p = 100 gives [min, max]: no change.                                      */
/* ------------------------------------------------------------------------ */
static int orc_cmp_float(const void *a, const void *b)
{
    float x = *(const float *)a, y = *(const float *)b;
    return (x > y) - (x < y);
}

double orc_percentile(const float *v, int64_t n, double pct)
{
    float *t = (float *)malloc((size_t)n * sizeof(float));
    memcpy(t, v, (size_t)n * sizeof(float));
    qsort(t, (size_t)n, sizeof(float), orc_cmp_float);
    double h = (double)(n - 1) * pct / 100.0;
    int64_t i = (int64_t)floor(h);
    double r = (double)t[i];
    if (i + 1 < n)
        r += (h - (double)i) * ((double)t[i + 1] - (double)t[i]);
    free(t);
    return r;
}

void orc_clip_rows(const float *W, int64_t N, int64_t K, double pct, float *out)
{
    for (int64_t n = 0; n < N; ++n) {
        float lo = (float)orc_percentile(W + n * K, K, 100.0 - pct);
        float hi = (float)orc_percentile(W + n * K, K, pct);
        for (int64_t k = 0; k < K; ++k) {
            float w = W[n * K + k];
            out[n * K + k] = w < lo ? lo : (w > hi ? hi : w);
        }
    }
}

/* Dequantized weight w_hat = (q - zp) * scale  [p2 §2.1, §2.2]. */
void orc_dequantize_weights(const uint8_t *q, const uint16_t *scale16, const uint16_t *zp16,
                            int64_t N, int64_t K, int64_t group, double *w_hat)
{
    int64_t G = K / group;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t g = k / group;
            double s = orc_f16_to_f32(scale16[g * N + n]);
            double z = orc_f16_to_f32(zp16[g * N + n]);
            w_hat[n * K + k] = ((double)q[n * K + k] - z) * s;
        }
}

/* ------------------------------------------------------------------------ */
/* Nibble packing [p2 §2.2]: two 4-bit codes per byte, the first code of    */
/* the pair in the low 4 bits, the second in the high 4 bits; codes are     */
/* packed along K (a group of even size then starts on a byte boundary).    */
/* ------------------------------------------------------------------------ */
int orc_pack_nibbles(const uint8_t *q, int64_t N, int64_t K, uint8_t *packed)
{
    if (N <= 0 || K <= 0 || K % 2 != 0)
        return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K / 2; ++j) {
            uint8_t first = q[n * K + 2 * j];
            uint8_t second = q[n * K + 2 * j + 1];
            if (first > 15 || second > 15)
                return -1;
            packed[n * (K / 2) + j] = (uint8_t)(first | (second << 4));
        }
    return 0;
}

void orc_unpack_nibbles(const uint8_t *packed, int64_t N, int64_t K, uint8_t *q)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K / 2; ++j) {
            uint8_t b = packed[n * (K / 2) + j];
            q[n * K + 2 * j] = (uint8_t)(b & 0x0F);
            q[n * K + 2 * j + 1] = (uint8_t)(b >> 4);
        }
}

/* ------------------------------------------------------------------------ */
/* O2: per-token dynamic symmetric INT8 activation quantization.            */
/* [p1 §5.3] per-token scale computed at forward time; [p3 §2.1] symmetric  */
/* form q = round(x/scale), scale = max|x| / (2^(b-1)-1) = max|x|/127.       */
/* x: [M][K] fp32 with row stride ldx.  qa: [M][K] int8.  a_scale: [M].     */
/* ------------------------------------------------------------------------ */
void orc_quantize_act(const float *x, int64_t M, int64_t K, int64_t ldx, int8_t *qa, float *a_scale)
{
    for (int64_t m = 0; m < M; ++m) {
        const float *row = x + m * ldx;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(row[k]);
            if (a > amax)
                amax = a;
        }
        float s = amax / 127.0f;
        a_scale[m] = s;
        for (int64_t k = 0; k < K; ++k) {
            int v = 0;
            if (s != 0.0f) { /* s is 0 for an all-zero row, or when amax/127 underflows */
                float r = rintf(row[k] / s);
                if (r > 127.0f)
                    r = 127.0f;
                if (r < -127.0f)
                    r = -127.0f;
                v = (int)r;
            }
            qa[m * K + k] = (int8_t)v;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* O8: per-channel activation smoothing [p3 §3.4]: a factor per input        */
/* channel moves part of the activations' outlier range into the weights,    */
/* so that both fall in a range the quantizers handle.  The page gives the   */
/* idea, not a formula; the reading used here (listed in the design notes):  */
/*   ax_k = max_m |x_cal[m][k]| over calibration rows,                        */
/*   aw_k = max_n |W[n][k]|,                                                  */
/*   s_k  = ax_k^alpha / aw_k^(1 - alpha)   (double, then fp32),              */
/*          1 where ax_k or aw_k is 0,                                        */
/*   inv_s_k = 1 / s_k                      (double, then fp32),              */
/* the weights become W[n][k] * s_k (one fp32 product) before the group      */
/* quantization, and at run time every activation is multiplied by inv_s_k  */
/* (one fp32 product) before the per-token quantizer O2.                     */
/* ------------------------------------------------------------------------ */
void orc_channel_absmax(const float *A, int64_t rows, int64_t K, float *out)
{
    for (int64_t k = 0; k < K; ++k) {
        float m = 0.0f;
        for (int64_t r = 0; r < rows; ++r) {
            float a = fabsf(A[r * K + k]);
            if (a > m)
                m = a;
        }
        out[k] = m;
    }
}

void orc_smooth_factors(const float *ax, const float *aw, int64_t K, double alpha, float *s, float *inv_s)
{
    for (int64_t k = 0; k < K; ++k) {
        double f = 1.0;
        if (ax[k] > 0.0f && aw[k] > 0.0f)
            f = pow((double)ax[k], alpha) / pow((double)aw[k], 1.0 - alpha);
        s[k] = (float)f;
        inv_s[k] = (float)(1.0 / (double)s[k]);
    }
}

void orc_smooth_weights(const float *W, int64_t N, int64_t K, const float *s, float *out)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            out[n * K + k] = W[n * K + k] * s[k];
}

/* O2 applied to the smoothed activations x[m][k] * inv_s[k] (fp32 products). */
void orc_quantize_act_smooth(const float *x, int64_t M, int64_t K, int64_t ldx, const float *inv_s, int8_t *qa,
                             float *a_scale)
{
    float *y = (float *)malloc((size_t)(M * K) * sizeof(float));
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k)
            y[m * K + k] = x[m * ldx + k] * inv_s[k];
    orc_quantize_act(y, M, K, K, qa, a_scale);
    free(y);
}

/* ------------------------------------------------------------------------ */
/* O3: per-group integer product with int32 accumulation [p2 §3.2, §5.4]:   */
/*   isum[g][m][n] = sum_{k in group g} qa[m][k] * (q[n][k] - zp[g][n]).    */
/* isums: [G][M][N] int32.                                                  */
/* ------------------------------------------------------------------------ */
void orc_group_isums(const int8_t *qa, const uint8_t *q, const uint16_t *zp16,
                     int64_t M, int64_t N, int64_t K, int64_t group, int32_t *isums)
{
    int64_t G = K / group;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t g = 0; g < G; ++g) {
            int32_t z = (int32_t)orc_f16_to_f32(zp16[g * N + n]);
            for (int64_t m = 0; m < M; ++m) {
                int32_t acc = 0;
                for (int64_t k = g * group; k < (g + 1) * group; ++k)
                    acc += (int32_t)qa[m * K + k] * ((int32_t)q[n * K + k] - z);
                isums[(g * M + m) * N + n] = acc;
            }
        }
}

/* ------------------------------------------------------------------------ */
/* O4: the epilogue, in double [p1 §4.3 step 4; p2 §3.2 "multiply by the    */
/* scales"]:  out[m][n] = sum_g a_scale[m] * scale[g][n] * isum[g][m][n].   */
/* Also returns sum_g |a_scale * scale * isum|, the magnitude that sets the */
/* fp32 tolerance.  Computed for the listed (m, n) pairs only; rows m of qa */
/* and columns n of q are read in full.                                     */
/* ------------------------------------------------------------------------ */
void orc_gemm_at(const int8_t *qa, const float *a_scale, const uint8_t *q,
                 const uint16_t *scale16, const uint16_t *zp16,
                 int64_t M, int64_t N, int64_t K, int64_t group,
                 const int64_t *ms, const int64_t *ns, int64_t count,
                 double *out, double *mag)
{
    int64_t G = K / group;
    (void)M;
    #pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = ms[i], n = ns[i];
        double total = 0.0, total_abs = 0.0;
        for (int64_t g = 0; g < G; ++g) {
            int32_t z = (int32_t)orc_f16_to_f32(zp16[g * N + n]);
            int32_t isum = 0;
            for (int64_t k = g * group; k < (g + 1) * group; ++k)
                isum += (int32_t)qa[m * K + k] * ((int32_t)q[n * K + k] - z);
            double term = (double)a_scale[m] * (double)orc_f16_to_f32(scale16[g * N + n]) * (double)isum;
            total += term;
            total_abs += fabs(term);
        }
        out[i] = total;
        mag[i] = total_abs;
    }
}

/* Full dense version of the same definition: out, mag are [M][N]. */
void orc_gemm(const int8_t *qa, const float *a_scale, const uint8_t *q,
              const uint16_t *scale16, const uint16_t *zp16,
              int64_t M, int64_t N, int64_t K, int64_t group, double *out, double *mag)
{
    int64_t G = K / group;
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t m = 0; m < M; ++m) {
            double total = 0.0, total_abs = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                int32_t z = (int32_t)orc_f16_to_f32(zp16[g * N + n]);
                int32_t isum = 0;
                for (int64_t k = g * group; k < (g + 1) * group; ++k)
                    isum += (int32_t)qa[m * K + k] * ((int32_t)q[n * K + k] - z);
                double term = (double)a_scale[m] * (double)orc_f16_to_f32(scale16[g * N + n]) * (double)isum;
                total += term;
                total_abs += fabs(term);
            }
            out[m * N + n] = total;
            mag[m * N + n] = total_abs;
        }
}

/* ------------------------------------------------------------------------ */
/* O5: router.  [p1 §5.2] the router stays in high precision and picks the  */
/* experts each token goes to; [p4] a token picks its expert(s) from E.     */
/* Per token: the k largest logits in descending order, ties broken toward */
/* the lower expert id; weights = softmax over the k selected logits        */
/* (evaluated in double, stored as fp32).                                   */
/* ------------------------------------------------------------------------ */
int orc_route_topk(const float *logits, int64_t T, int32_t E, int32_t k, int32_t *ids, float *w)
{
    if (T < 0 || E <= 0 || k <= 0 || k > E)
        return -1;
    for (int64_t t = 0; t < T; ++t) {
        const float *z = logits + t * E;
        for (int32_t j = 0; j < k; ++j) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e) {
                int taken = 0;
                for (int32_t i = 0; i < j; ++i)
                    if (ids[t * k + i] == e)
                        taken = 1;
                if (taken)
                    continue;
                if (best < 0 || z[e] > z[best])
                    best = e; /* strict '>' keeps the lower id on ties */
            }
            ids[t * k + j] = best;
        }
        double zmax = z[ids[t * k]];
        double denom = 0.0;
        for (int32_t j = 0; j < k; ++j)
            denom += exp((double)z[ids[t * k + j]] - zmax);
        for (int32_t j = 0; j < k; ++j)
            w[t * k + j] = (float)(exp((double)z[ids[t * k + j]] - zmax) / denom);
    }
    return 0;
}

/* Expert buckets: count[e] pairs per expert, offsets = exclusive scan of the
 * counts (E+1 entries), perm = pair indices p = t*k + j listed by ascending
 * expert and, within an expert, ascending p. */
int orc_bucket(const int32_t *ids, int64_t P, int32_t E, int32_t *offsets, int32_t *perm)
{
    for (int32_t e = 0; e <= E; ++e)
        offsets[e] = 0;
    for (int64_t p = 0; p < P; ++p) {
        if (ids[p] < 0 || ids[p] >= E)
            return -1;
        offsets[ids[p] + 1] += 1;
    }
    for (int32_t e = 0; e < E; ++e)
        offsets[e + 1] += offsets[e];
    int64_t slot = 0;
    for (int32_t e = 0; e < E; ++e)
        for (int64_t p = 0; p < P; ++p)
            if (ids[p] == e)
                perm[slot++] = (int32_t)p;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* MoE FFN pieces (the expert block around the grouped GEMM):               */
/*   h = silu(gate) * up with silu(v) = v / (1 + exp(-v)), in double;       */
/*   out[t] = sum_j w[t][j] * y[slot of (t, j)] + y_shared[t], in double.   */
/* gu: [P][2I] (gate = columns [0, I), up = columns [I, 2I)).               */
/* ------------------------------------------------------------------------ */
void orc_silu_mul(const float *gu, int64_t P, int64_t I, double *h)
{
    for (int64_t p = 0; p < P; ++p)
        for (int64_t i = 0; i < I; ++i) {
            double g = gu[p * 2 * I + i];
            double u = gu[p * 2 * I + I + i];
            h[p * I + i] = g / (1.0 + exp(-g)) * u;
        }
}

/* y: [S][H] rows in slot order; slot_of_pair: [T*k]; y_shared: [T][H] or NULL. */
void orc_combine(const float *y, const int32_t *slot_of_pair, const float *w, const float *y_shared,
                 int64_t T, int32_t k, int64_t H, double *out)
{
    for (int64_t t = 0; t < T; ++t)
        for (int64_t c = 0; c < H; ++c) {
            double acc = 0.0;
            for (int32_t j = 0; j < k; ++j)
                acc += (double)w[t * k + j] * (double)y[(int64_t)slot_of_pair[t * k + j] * H + c];
            if (y_shared)
                acc += (double)y_shared[t * H + c];
            out[t * H + c] = acc;
        }
}

/* Number of host threads the parallel loops above use (OpenMP's team size). */
int orc_num_threads(void) { return omp_get_max_threads(); }
