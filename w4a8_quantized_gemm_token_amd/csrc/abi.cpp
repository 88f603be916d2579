// abi.cpp -- the extern "C" entry points of libw4a8.so: argument validation,
// error reporting, the host-side weight packer, and dispatch to the kernels.
//
// The host packer restates the group quantization of [p2 §2.1, §2.2]
// (pptc.cn/news/121597, "Kimi 2.7 MoE, 4-bit storage to INT8, dissected"):
// scale = (max - min)/15 over the group's range widened to contain 0, stored as
// fp16; zp = round(-min/scale); q = clamp(round(w/scale) + zp, 0, 15) with the
// stored fp16 scale; two codes per byte, first code in the low nibble.  fp16
// conversion uses the compiler's _Float16 (IEEE binary16, round to nearest even).
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

#include "w4a8_internal.hpp"

namespace w4a8 {

static thread_local char g_err[512] = "";

void set_error(const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

void clear_error() { g_err[0] = '\0'; }

w4a8_status hip_status(hipError_t err, const char *what) {
    if (err == hipSuccess) return W4A8_OK;
    set_error("%s: %s", what, hipGetErrorString(err));
    return W4A8_EHIP;
}

}  // namespace w4a8

using namespace w4a8;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

#define W4A8_REQUIRE(cond, code, ...) \
    do {                              \
        if (!(cond)) {                \
            set_error(__VA_ARGS__);   \
            return code;              \
        }                             \
    } while (0)

w4a8_status check_group(int32_t group, int64_t K) {
    W4A8_REQUIRE(group == W4A8_GROUP, W4A8_EUNSUPPORTED, "group size %d is not supported (only 128)", (int)group);
    W4A8_REQUIRE(K > 0 && K % W4A8_GROUP == 0, W4A8_EINVAL, "K=%lld must be a positive multiple of 128",
                 (long long)K);
    return W4A8_OK;
}

// Group sizes of the host packer and the tiled GEMM loop: 64, 128 or 256 along K.
w4a8_status check_group_any(int32_t group, int64_t K) {
    W4A8_REQUIRE(group == 64 || group == 128 || group == 256, W4A8_EUNSUPPORTED,
                 "group size %d is not supported (64, 128 or 256)", (int)group);
    W4A8_REQUIRE(K > 0 && K % 128 == 0 && K % group == 0, W4A8_EINVAL,
                 "K=%lld must be a positive multiple of 128 and of the group size", (long long)K);
    return W4A8_OK;
}

uint16_t f32_to_f16_bits(float f) {
    const _Float16 h = (_Float16)f;
    uint16_t b;
    std::memcpy(&b, &h, 2);
    return b;
}

float f16_bits_to_f32(uint16_t b) {
    _Float16 h;
    std::memcpy(&h, &b, 2);
    return (float)h;
}

// Quantize columns [n0, n1); returns false on non-finite input or fp16 overflow.
// One output column n (its K weights w): group-wise asymmetric 4-bit codes, or with
// sym the symmetric form stored in the same format (code q + 8, zp 8).
bool pack_row(const float *w0, int64_t n, int64_t N, int64_t K, int64_t group, bool sym, uint8_t *packed,
              uint16_t *scale, uint16_t *zp) {
    const int64_t G = K / group;
    uint8_t codes[256];
    for (int64_t g = 0; g < G; ++g) {
        const float *w = w0 + g * group;
        float lo = 0.0f, hi = 0.0f;
        for (int i = 0; i < group; ++i) {
            if (!std::isfinite(w[i])) return false;
            lo = std::fmin(lo, w[i]);
            hi = std::fmax(hi, w[i]);
        }
        // asymmetric: (max - min) / (2^4 - 1); symmetric: max|w| / (2^3 - 1)
        uint16_t sh = f32_to_f16_bits(sym ? std::fmax(-lo, hi) / 7.0f : (hi - lo) / 15.0f);
        if ((sh & 0x7C00u) == 0x7C00u) return false;
        float s = f16_bits_to_f32(sh);
        if (s == 0.0f) {
            sh = 0x3C00u;
            s = 1.0f;
        }
        const int z = sym ? 8 : (int)std::fmin(std::fmax(std::nearbyint(-lo / s), 0.0f), 15.0f);
        for (int i = 0; i < group; ++i) {
            int v;
            if (sym) v = (int)std::fmin(std::fmax(std::nearbyint(w[i] / s), -7.0f), 7.0f) + 8;
            else v = (int)std::nearbyint(w[i] / s) + z;
            codes[i] = (uint8_t)(v < 0 ? 0 : (v > 15 ? 15 : v));
        }
        uint8_t *dst = packed + n * (K / 2) + g * (group / 2);
        for (int j = 0; j < group / 2; ++j) dst[j] = (uint8_t)(codes[2 * j] | (codes[2 * j + 1] << 4));
        scale[g * N + n] = sh;
        zp[g * N + n] = f32_to_f16_bits((float)z);
    }
    return true;
}

// pct-th percentile of v (linear interpolation between order statistics, position
// (K - 1) * pct / 100, in double); v is reordered.
double row_percentile(std::vector<float> &v, double pct) {
    const int64_t n = (int64_t)v.size();
    const double h = (double)(n - 1) * pct / 100.0;
    const int64_t i = (int64_t)std::floor(h);
    std::nth_element(v.begin(), v.begin() + i, v.end());
    double r = (double)v[(size_t)i];
    if (i + 1 < n) {
        const float next = *std::min_element(v.begin() + i + 1, v.end());
        r += (h - (double)i) * ((double)next - (double)v[(size_t)i]);
    }
    return r;
}

// Columns [n0, n1).  clip < 100: each column's weights are first clamped to its own
// [100 - clip, clip] percentiles (rounded to fp32).
bool pack_columns(const float *W, int64_t N, int64_t K, int64_t group, int64_t n0, int64_t n1, bool sym, double clip,
                  uint8_t *packed, uint16_t *scale, uint16_t *zp) {
    std::vector<float> row, work;
    if (clip < 100.0) {
        row.resize((size_t)K);
        work.resize((size_t)K);
    }
    for (int64_t n = n0; n < n1; ++n) {
        const float *w = W + n * K;
        if (clip < 100.0) {
            for (int64_t k = 0; k < K; ++k)
                if (!std::isfinite(w[k])) return false;
            work.assign(w, w + K);
            const float lo = (float)row_percentile(work, 100.0 - clip);
            const float hi = (float)row_percentile(work, clip);
            for (int64_t k = 0; k < K; ++k) row[(size_t)k] = w[k] < lo ? lo : (w[k] > hi ? hi : w[k]);
            w = row.data();
        }
        if (!pack_row(w, n, N, K, group, sym, packed, scale, zp)) return false;
    }
    return true;
}

}  // namespace

extern "C" {

int w4a8_abi_version(void) { return W4A8_ABI_VERSION; }

const char *w4a8_status_str(int status) {
    switch (status) {
    case W4A8_OK: return "ok";
    case W4A8_EINVAL: return "invalid argument";
    case W4A8_EUNSUPPORTED: return "unsupported";
    case W4A8_EHIP: return "HIP error";
    case W4A8_EWORKSPACE: return "workspace too small";
    default: return "unknown status";
    }
}

const char *w4a8_last_error(void) { return g_err; }

w4a8_status w4a8_pack_weights(const float *W, int64_t N, int64_t K, int32_t group, uint8_t *packed, uint16_t *scale,
                              uint16_t *zp) {
    return w4a8_pack_weights_ex(W, N, K, group, W4A8_PACK_ASYMMETRIC, 100.0, packed, scale, zp);
}

w4a8_status w4a8_pack_weights_ex(const float *W, int64_t N, int64_t K, int32_t group, int32_t mode,
                                 double clip_percent, uint8_t *packed, uint16_t *scale, uint16_t *zp) {
    clear_error();
    W4A8_REQUIRE(W && packed && scale && zp, W4A8_EINVAL, "null pointer");
    W4A8_REQUIRE(N > 0, W4A8_EINVAL, "N=%lld must be positive", (long long)N);
    if (w4a8_status st = check_group_any(group, K)) return st;
    W4A8_REQUIRE(mode == W4A8_PACK_ASYMMETRIC || mode == W4A8_PACK_SYMMETRIC, W4A8_EINVAL, "mode=%d is not a packer mode",
                 (int)mode);
    W4A8_REQUIRE(clip_percent >= 50.0 && clip_percent <= 100.0, W4A8_EINVAL, "clip_percent=%g must lie in [50, 100]",
                 clip_percent);
    const bool sym = mode == W4A8_PACK_SYMMETRIC;
    unsigned hw = std::thread::hardware_concurrency();
    int64_t nthreads = hw ? hw : 1;
    if (nthreads > N) nthreads = N;
    if ((N * K) < (1 << 20)) nthreads = 1;
    std::vector<char> ok((size_t)nthreads, 1);
    std::vector<std::thread> pool;
    const int64_t per = (N + nthreads - 1) / nthreads;
    for (int64_t t = 0; t < nthreads; ++t) {
        const int64_t n0 = t * per, n1 = std::min(N, n0 + per);
        if (n0 >= n1) continue;
        pool.emplace_back(
            [=, &ok] { ok[t] = pack_columns(W, N, K, group, n0, n1, sym, clip_percent, packed, scale, zp); });
    }
    for (auto &th : pool) th.join();
    for (char c : ok)
        W4A8_REQUIRE(c, W4A8_EINVAL, "weights contain non-finite values or a group range too large for an fp16 scale");
    return W4A8_OK;
}

w4a8_status w4a8_unpack_weights(const uint8_t *packed, const uint16_t *scale, const uint16_t *zp, int64_t N, int64_t K,
                                int32_t group, uint8_t *q_out, float *w_hat) {
    clear_error();
    W4A8_REQUIRE(packed && scale && zp, W4A8_EINVAL, "null pointer");
    W4A8_REQUIRE(N > 0, W4A8_EINVAL, "N=%lld must be positive", (long long)N);
    if (w4a8_status st = check_group_any(group, K)) return st;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            const uint8_t b = packed[n * (K / 2) + k / 2];
            const uint8_t q = (k & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 0x0F);
            if (q_out) q_out[n * K + k] = q;
            if (w_hat) {
                const int64_t g = k / group;
                const float s = f16_bits_to_f32(scale[g * N + n]);
                const float z = f16_bits_to_f32(zp[g * N + n]);
                w_hat[n * K + k] = ((float)q - z) * s;
            }
        }
    return W4A8_OK;
}

w4a8_status w4a8_pack_weights_device(const float *W, int64_t N, int64_t K, int32_t group, uint8_t *packed,
                                     uint16_t *scale, uint16_t *zp, hipStream_t stream) {
    clear_error();
    W4A8_REQUIRE(W && packed && scale && zp, W4A8_EINVAL, "null pointer");
    W4A8_REQUIRE(N > 0, W4A8_EINVAL, "N=%lld must be positive", (long long)N);
    if (w4a8_status st = check_group_any(group, K)) return st;
    W4A8_REQUIRE(((uintptr_t)W & (group == 256 ? 15u : 7u)) == 0 && ((uintptr_t)packed & 1u) == 0, W4A8_EINVAL,
                 "W must be 8-byte aligned (16 for group 256) and packed 2-byte aligned");
    return hip_status(launch_pack_weights(W, N, K, group, nullptr, packed, scale, zp, stream),
                      "pack_weights_device launch");
}

w4a8_status w4a8_pack_weights_device_smooth(const float *W, int64_t N, int64_t K, int32_t group, const float *s,
                                            uint8_t *packed, uint16_t *scale, uint16_t *zp, hipStream_t stream) {
    clear_error();
    W4A8_REQUIRE(W && s && packed && scale && zp, W4A8_EINVAL, "null pointer");
    W4A8_REQUIRE(N > 0, W4A8_EINVAL, "N=%lld must be positive", (long long)N);
    if (w4a8_status st = check_group_any(group, K)) return st;
    const uintptr_t am = group == 256 ? 15u : 7u;
    W4A8_REQUIRE(((uintptr_t)W & am) == 0 && ((uintptr_t)s & am) == 0 && ((uintptr_t)packed & 1u) == 0, W4A8_EINVAL,
                 "W and s must be 8-byte aligned (16 for group 256) and packed 2-byte aligned");
    return hip_status(launch_pack_weights(W, N, K, group, s, packed, scale, zp, stream),
                      "pack_weights_device_smooth launch");
}

w4a8_status w4a8_channel_absmax(const float *A, int64_t rows, int64_t K, int64_t lda, float *out, hipStream_t stream) {
    clear_error();
    W4A8_REQUIRE((A || rows == 0) && out, W4A8_EINVAL, "null pointer");
    W4A8_REQUIRE(rows >= 0 && K > 0 && lda >= K, W4A8_EINVAL, "bad sizes rows=%lld K=%lld lda=%lld", (long long)rows,
                 (long long)K, (long long)lda);
    W4A8_REQUIRE((K + 63) / 64 < (1ll << 31), W4A8_EINVAL, "K too large");
    return hip_status(launch_channel_absmax(A, rows, K, lda, out, stream), "channel_absmax launch");
}

w4a8_status w4a8_smooth_factors(const float *ax, const float *aw, int64_t K, double alpha, float *s, float *inv_s) {
    clear_error();
    W4A8_REQUIRE(ax && aw && s && inv_s, W4A8_EINVAL, "null pointer");
    W4A8_REQUIRE(K > 0, W4A8_EINVAL, "K=%lld must be positive", (long long)K);
    W4A8_REQUIRE(alpha >= 0.0 && alpha <= 1.0, W4A8_EINVAL, "alpha=%g must lie in [0, 1]", alpha);
    for (int64_t k = 0; k < K; ++k)
        W4A8_REQUIRE(std::isfinite(ax[k]) && ax[k] >= 0.0f && std::isfinite(aw[k]) && aw[k] >= 0.0f, W4A8_EINVAL,
                     "channel maxima must be finite and non-negative (channel %lld)", (long long)k);
    for (int64_t k = 0; k < K; ++k) {
        // migration strength alpha: activation range ax^alpha over weight range aw^(1-alpha)
        const double f = (ax[k] > 0.0f && aw[k] > 0.0f) ? std::pow((double)ax[k], alpha) /
                                                                std::pow((double)aw[k], 1.0 - alpha)
                                                          : 1.0;
        const float sf = (float)f;
        W4A8_REQUIRE(std::isfinite(sf) && sf > 0.0f, W4A8_EINVAL,
                     "smoothing factor of channel %lld is not a positive finite fp32", (long long)k);
        s[k] = sf;
        inv_s[k] = (float)(1.0 / (double)sf);
    }
    return W4A8_OK;
}

w4a8_status w4a8_quantize_act(const float *x, int64_t M, int64_t K, int64_t ldx, int8_t *qa, float *a_scale,
                              hipStream_t stream) {
    clear_error();
    W4A8_REQUIRE(x && qa && a_scale, W4A8_EINVAL, "null pointer");
    W4A8_REQUIRE(M >= 0 && K > 0 && ldx >= K, W4A8_EINVAL, "bad sizes M=%lld K=%lld ldx=%lld", (long long)M,
                 (long long)K, (long long)ldx);
    W4A8_REQUIRE(K % 16 == 0, W4A8_EINVAL, "K=%lld must be a multiple of 16", (long long)K);
    W4A8_REQUIRE(aligned16(qa), W4A8_EINVAL, "qa must be 16-byte aligned");
    W4A8_REQUIRE(M < (1ll << 31), W4A8_EINVAL, "M too large");
    if (M == 0) return W4A8_OK;
    return hip_status(launch_quantize_act(x, M, K, ldx, nullptr, qa, a_scale, stream), "quantize_act launch");
}

w4a8_status w4a8_quantize_act_smooth(const float *x, int64_t M, int64_t K, int64_t ldx, const float *inv_s, int8_t *qa,
                                     float *a_scale, hipStream_t stream) {
    clear_error();
    W4A8_REQUIRE(x && inv_s && qa && a_scale, W4A8_EINVAL, "null pointer");
    W4A8_REQUIRE(M >= 0 && K > 0 && ldx >= K, W4A8_EINVAL, "bad sizes M=%lld K=%lld ldx=%lld", (long long)M,
                 (long long)K, (long long)ldx);
    W4A8_REQUIRE(K % 16 == 0, W4A8_EINVAL, "K=%lld must be a multiple of 16", (long long)K);
    W4A8_REQUIRE(aligned16(qa), W4A8_EINVAL, "qa must be 16-byte aligned");
    W4A8_REQUIRE(M < (1ll << 31), W4A8_EINVAL, "M too large");
    if (M == 0) return W4A8_OK;
    return hip_status(launch_quantize_act(x, M, K, ldx, inv_s, qa, a_scale, stream), "quantize_act_smooth launch");
}

static w4a8_status check_gemm(const int8_t *qa, int64_t M, int64_t K, const uint8_t *packed, const uint16_t *scale,
                              const uint16_t *zp, int64_t N, int32_t group, const void *out) {
    W4A8_REQUIRE(qa && packed && zp && out, W4A8_EINVAL, "null pointer");
    (void)scale;
    W4A8_REQUIRE(M >= 0, W4A8_EINVAL, "M=%lld must be >= 0", (long long)M);
    W4A8_REQUIRE(N > 0 && N % 16 == 0, W4A8_EINVAL, "N=%lld must be a positive multiple of 16", (long long)N);
    if (w4a8_status st = check_group_any(group, K)) return st;
    W4A8_REQUIRE(aligned16(qa) && aligned16(packed) && aligned16(out), W4A8_EINVAL,
                 "qa, packed and out must be 16-byte aligned");
    return W4A8_OK;
}

static w4a8_status gemm_common(const int8_t *qa, const float *a_scale, int64_t M, int64_t K, const uint8_t *packed,
                               const uint16_t *scale, const uint16_t *zp, int64_t N, int32_t group, int32_t path,
                               float *out, int32_t *isums, hipStream_t stream) {
    W4A8_REQUIRE(path >= 0 && path <= 5, W4A8_EINVAL, "path=%d must be in [0, 5]", (int)path);
    if (group != W4A8_GROUP) {
        // group sizes 64 and 256: the decode loop for M <= 16 (K a multiple of 256), the
        // tiled loop otherwise
        if (path == 0) path = decode_group_fits(M, K, N) ? 1 : 2;
        W4A8_REQUIRE(path != 1 || M == 0 || decode_group_fits(M, K, N), W4A8_EUNSUPPORTED,
                     "group size %d takes the decode loop (path 1) only for 1 <= M <= 16 and K %% 256 == 0",
                     (int)group);
        if (M == 0) return W4A8_OK;
        return hip_status(launch_gemm_tiled_group(qa, a_scale, M, K, packed, scale, zp, N, group, path, out, isums,
                                                  stream),
                          "gemm launch");
    }
    if (path == 0) path = (M <= kStreamMaxM) ? 1 : 2;
    W4A8_REQUIRE(!(path == 1 && M > kStreamMaxM), W4A8_EINVAL, "the streaming loop takes M <= %lld",
                 (long long)kStreamMaxM);
    if (M == 0) return W4A8_OK;
    return hip_status(launch_gemm(qa, a_scale, M, K, packed, scale, zp, N, path, out, isums, stream), "gemm launch");
}

w4a8_status w4a8_gemm(const int8_t *qa, const float *a_scale, int64_t M, int64_t K, const uint8_t *packed,
                      const uint16_t *scale, const uint16_t *zp, int64_t N, int32_t group, float *out,
                      hipStream_t stream) {
    return w4a8_gemm_path(qa, a_scale, M, K, packed, scale, zp, N, group, 0, out, stream);
}

w4a8_status w4a8_gemm_path(const int8_t *qa, const float *a_scale, int64_t M, int64_t K, const uint8_t *packed,
                           const uint16_t *scale, const uint16_t *zp, int64_t N, int32_t group, int32_t path,
                           float *out, hipStream_t stream) {
    clear_error();
    if (w4a8_status st = check_gemm(qa, M, K, packed, scale, zp, N, group, out)) return st;
    W4A8_REQUIRE(a_scale && scale, W4A8_EINVAL, "null pointer");
    return gemm_common(qa, a_scale, M, K, packed, scale, zp, N, group, path, out, nullptr, stream);
}

w4a8_status w4a8_gemm_debug_isums(const int8_t *qa, int64_t M, int64_t K, const uint8_t *packed, const uint16_t *zp,
                                  int64_t N, int32_t group, int32_t path, int32_t *isums, hipStream_t stream) {
    clear_error();
    if (w4a8_status st = check_gemm(qa, M, K, packed, nullptr, zp, N, group, isums)) return st;
    return gemm_common(qa, nullptr, M, K, packed, nullptr, zp, N, group, path, nullptr, isums, stream);
}

size_t w4a8_tm_bytes(int64_t N, int64_t K) {
    if (N <= 0 || K <= 0 || N % 16 != 0 || K % (2 * W4A8_GROUP) != 0) return 0;
    return (size_t)tm_bytes(N, K);
}

w4a8_status w4a8_weights_to_tm(const uint8_t *packed, const uint16_t *scale, const uint16_t *zp, int64_t N, int64_t K,
                               int32_t group, uint8_t *tm, hipStream_t stream) {
    clear_error();
    W4A8_REQUIRE(packed && scale && zp && tm, W4A8_EINVAL, "null pointer");
    W4A8_REQUIRE(N > 0 && N % 16 == 0, W4A8_EINVAL, "N=%lld must be a positive multiple of 16", (long long)N);
    if (w4a8_status st = check_group(group, K)) return st;
    W4A8_REQUIRE(K % (2 * W4A8_GROUP) == 0, W4A8_EINVAL, "K=%lld must be a multiple of 256", (long long)K);
    W4A8_REQUIRE(aligned16(packed) && aligned16(tm), W4A8_EINVAL, "packed and tm must be 16-byte aligned");
    W4A8_REQUIRE((N / 16) * (K / 256) < (1ll << 31), W4A8_EINVAL, "weight too large");
    return hip_status(launch_weights_to_tm(packed, scale, zp, N, K, tm, stream), "weights_to_tm launch");
}

w4a8_status w4a8_gemm_tm(const int8_t *qa, const float *a_scale, int64_t M, int64_t K, const uint8_t *tm, int64_t N,
                         int32_t group, float *out, hipStream_t stream) {
    clear_error();
    W4A8_REQUIRE(qa && a_scale && tm && out, W4A8_EINVAL, "null pointer");
    W4A8_REQUIRE(M >= 0, W4A8_EINVAL, "M=%lld must be >= 0", (long long)M);
    W4A8_REQUIRE(N > 0 && N % 16 == 0, W4A8_EINVAL, "N=%lld must be a positive multiple of 16", (long long)N);
    if (w4a8_status st = check_group(group, K)) return st;
    W4A8_REQUIRE(aligned16(qa) && aligned16(tm) && aligned16(out), W4A8_EINVAL,
                 "qa, tm and out must be 16-byte aligned");
    if (M == 0) return W4A8_OK;
    W4A8_REQUIRE(gemm_tm_supported(M, K, N), W4A8_EINVAL,
                 "the tile-major GEMM takes K %% 256 == 0, a tile-major array below 4 GiB, and "
                 "M*(K+16) <= 143360 for M <= 16 or M*K < 2^32 above (M=%lld K=%lld N=%lld)",
                 (long long)M, (long long)K, (long long)N);
    return hip_status(launch_gemm_tm(qa, a_scale, M, K, tm, N, out, stream), "gemm_tm launch");
}

w4a8_status w4a8_moe_route(const float *logits, int64_t T, int32_t E, int32_t topk, int32_t with_shared,
                           int32_t *topk_ids, float *topk_w, int32_t *expert_offsets, int32_t *perm,
                           int32_t *slot_row, int32_t *slot_of_pair, hipStream_t stream) {
    clear_error();
    W4A8_REQUIRE(expert_offsets && (T == 0 || (logits && topk_ids && topk_w && perm && slot_of_pair)), W4A8_EINVAL,
                 "null pointer");
    W4A8_REQUIRE(T >= 0, W4A8_EINVAL, "T=%lld must be >= 0", (long long)T);
    W4A8_REQUIRE(E > 0 && E <= 1024, W4A8_EINVAL, "E=%d must be in [1, 1024]", (int)E);
    W4A8_REQUIRE(topk >= 1 && topk <= 8 && topk <= E, W4A8_EINVAL, "topk=%d must be in [1, min(E, 8)]", (int)topk);
    W4A8_REQUIRE(with_shared == 0 || with_shared == 1, W4A8_EINVAL, "with_shared=%d must be 0 or 1", (int)with_shared);
    W4A8_REQUIRE(T * (topk + 1) < (1ll << 31), W4A8_EINVAL, "T*(topk+1) too large");
    return hip_status(launch_moe_route(logits, T, E, topk, with_shared, topk_ids, topk_w, expert_offsets, perm,
                                       slot_row, slot_of_pair, stream),
                      "moe_route launch");
}

w4a8_status w4a8_moe_grouped_gemm(const int8_t *qa, const float *a_scale, int64_t R, const int32_t *row_index,
                                  const int32_t *expert_offsets, int32_t E, int64_t K, const uint8_t *packed,
                                  const uint16_t *scale, const uint16_t *zp, int64_t N, int32_t group,
                                  int64_t max_slots, float *out, hipStream_t stream) {
    clear_error();
    if (w4a8_status st = check_gemm(qa, R, K, packed, scale, zp, N, group, out)) return st;
    W4A8_REQUIRE(a_scale && scale && expert_offsets, W4A8_EINVAL, "null pointer");
    W4A8_REQUIRE(E > 0 && E <= 1024, W4A8_EINVAL, "E=%d must be in [1, 1024]", (int)E);
    W4A8_REQUIRE(max_slots >= 0 && max_slots < (1ll << 31), W4A8_EINVAL, "bad max_slots");
    if (max_slots == 0 || R == 0) return W4A8_OK;
    return hip_status(launch_grouped_gemm(qa, a_scale, R, row_index, expert_offsets, E, K, packed, scale, zp, N,
                                          max_slots, max_slots, out, nullptr, group, stream),
                      "grouped_gemm launch");
}

w4a8_status w4a8_moe_grouped_gemm_debug_isums(const int8_t *qa, int64_t R, const int32_t *row_index,
                                              const int32_t *expert_offsets, int32_t E, int64_t K,
                                              const uint8_t *packed, const uint16_t *zp, int64_t N, int32_t group,
                                              int64_t max_slots, int32_t *isums, hipStream_t stream) {
    clear_error();
    if (w4a8_status st = check_gemm(qa, R, K, packed, nullptr, zp, N, group, isums)) return st;
    W4A8_REQUIRE(expert_offsets, W4A8_EINVAL, "null pointer");
    W4A8_REQUIRE(E > 0 && E <= 1024, W4A8_EINVAL, "E=%d must be in [1, 1024]", (int)E);
    W4A8_REQUIRE(max_slots >= 0 && max_slots < (1ll << 31), W4A8_EINVAL, "bad max_slots");
    if (max_slots == 0 || R == 0) return W4A8_OK;
    return hip_status(launch_grouped_gemm(qa, nullptr, R, row_index, expert_offsets, E, K, packed, nullptr, zp, N,
                                          max_slots, max_slots, nullptr, isums, group, stream),
                      "grouped_gemm_debug_isums launch");
}

w4a8_status w4a8_silu_mul_quantize(const float *gu, int64_t P, int64_t I, int8_t *qh, float *h_scale, float *h_out,
                                   hipStream_t stream) {
    clear_error();
    W4A8_REQUIRE(gu && qh && h_scale, W4A8_EINVAL, "null pointer");
    W4A8_REQUIRE(P >= 0 && I > 0 && I % 16 == 0, W4A8_EINVAL, "bad sizes P=%lld I=%lld (I must be a multiple of 16)",
                 (long long)P, (long long)I);
    W4A8_REQUIRE(aligned16(qh), W4A8_EINVAL, "qh must be 16-byte aligned");
    W4A8_REQUIRE(P < (1ll << 31), W4A8_EINVAL, "P too large");
    if (P == 0) return W4A8_OK;
    return hip_status(launch_silu_mul_quantize(gu, P, I, qh, h_scale, h_out, stream), "silu_mul_quantize launch");
}

w4a8_status w4a8_moe_combine(const float *y, const int32_t *slot_of_pair, const float *topk_w, const float *y_shared,
                             int64_t T, int32_t topk, int64_t H, float *out, hipStream_t stream) {
    clear_error();
    W4A8_REQUIRE(y && slot_of_pair && topk_w && out, W4A8_EINVAL, "null pointer");
    W4A8_REQUIRE(T >= 0 && topk > 0 && H > 0 && H % 4 == 0, W4A8_EINVAL,
                 "bad sizes T=%lld topk=%d H=%lld (H must be a multiple of 4)", (long long)T, (int)topk, (long long)H);
    W4A8_REQUIRE(aligned16(y) && aligned16(out) && (!y_shared || aligned16(y_shared)), W4A8_EINVAL,
                 "y, y_shared and out must be 16-byte aligned");
    W4A8_REQUIRE(T < (1ll << 31), W4A8_EINVAL, "T too large");
    return hip_status(launch_moe_combine(y, slot_of_pair, topk_w, y_shared, T, topk, H, out, stream),
                      "moe_combine launch");
}

// ------------------------------------------------------------------ MoE FFN layer
namespace {

constexpr int64_t kWsAlign = 256;

int64_t ws_round(int64_t b) { return (b + kWsAlign - 1) / kWsAlign * kWsAlign; }

// byte offsets of the workspace parts; off[W4A8_WS_PARTS] = total size
void ws_layout(int64_t T, int64_t H, int64_t I, int32_t E, int32_t topk, int64_t *off) {
    const int64_t P = T * topk, S = P + T;
    const int64_t bytes[W4A8_WS_PARTS] = {
        4 * P,            // topk ids
        4 * P,            // topk weights
        4 * (E + 2),      // offsets (E routed + shared)
        4 * P,            // perm
        4 * S,            // slot_row
        4 * P,            // slot_of_pair
        T * H,            // qa
        4 * T,            // a_scale
        4 * S * 2 * I,    // gate/up output
        S * I,            // qh
        4 * S,            // h_scale
        4 * S * H,        // down output
    };
    int64_t o = 0;
    for (int i = 0; i < W4A8_WS_PARTS; ++i) {
        off[i] = o;
        o += ws_round(bytes[i]);
    }
    off[W4A8_WS_PARTS] = o;
}

w4a8_status check_ffn_sizes(int64_t T, int64_t H, int64_t I, int32_t E, int32_t topk) {
    W4A8_REQUIRE(T >= 0 && H > 0 && I > 0 && H % W4A8_GROUP == 0 && I % W4A8_GROUP == 0, W4A8_EINVAL,
                 "bad sizes T=%lld H=%lld I=%lld (H and I must be positive multiples of 128)", (long long)T,
                 (long long)H, (long long)I);
    W4A8_REQUIRE(E > 0 && E + 1 <= 1024, W4A8_EINVAL, "E=%d must be in [1, 1023]", (int)E);
    W4A8_REQUIRE(topk >= 1 && topk <= 8 && topk <= E, W4A8_EINVAL, "topk=%d must be in [1, min(E, 8)]", (int)topk);
    W4A8_REQUIRE(T * (topk + 1) < (1ll << 31) && T * (topk + 1) * 2 * I < (1ll << 40), W4A8_EINVAL,
                 "T=%lld too large", (long long)T);
    return W4A8_OK;
}

}  // namespace

}  // extern "C"

namespace w4a8 {

int64_t moe_ffn_ws_bytes(int64_t T, int64_t H, int64_t I, int32_t E, int32_t topk) {
    if (check_ffn_sizes(T, H, I, E, topk) != W4A8_OK) return -1;
    int64_t off[W4A8_WS_PARTS + 1];
    ws_layout(T, H, I, E, topk, off);
    return off[W4A8_WS_PARTS];
}

w4a8_status moe_ffn_run(const float *x, const float *logits, int64_t T, int64_t H, int64_t I, int32_t E,
                        int32_t topk, const uint8_t *gu_packed, const uint16_t *gu_scale, const uint16_t *gu_zp,
                        const uint8_t *dn_packed, const uint16_t *dn_scale, const uint16_t *dn_zp, float *out,
                        void *workspace, size_t ws_bytes, hipStream_t stream) {
    if (w4a8_status st = check_ffn_sizes(T, H, I, E, topk)) return st;
    W4A8_REQUIRE(workspace && (T == 0 || (x && logits && out)), W4A8_EINVAL, "null pointer");
    W4A8_REQUIRE(gu_packed && gu_scale && gu_zp && dn_packed && dn_scale && dn_zp, W4A8_EINVAL, "null weight pointer");
    W4A8_REQUIRE(aligned16(gu_packed) && aligned16(dn_packed) && (T == 0 || (aligned16(x) && aligned16(out))),
                 W4A8_EINVAL, "x, out and packed weights must be 16-byte aligned");
    int64_t off[W4A8_WS_PARTS + 1];
    ws_layout(T, H, I, E, topk, off);
    W4A8_REQUIRE((int64_t)ws_bytes >= off[W4A8_WS_PARTS], W4A8_EWORKSPACE, "workspace of %zu bytes, %lld needed",
                 ws_bytes, (long long)off[W4A8_WS_PARTS]);
    char *ws = (char *)workspace;
    int32_t *ids = (int32_t *)(ws + off[W4A8_WS_TOPK_IDS]);
    float *w = (float *)(ws + off[W4A8_WS_TOPK_W]);
    int32_t *offsets = (int32_t *)(ws + off[W4A8_WS_OFFSETS]);
    int32_t *perm = (int32_t *)(ws + off[W4A8_WS_PERM]);
    int32_t *slot_row = (int32_t *)(ws + off[W4A8_WS_SLOT_ROW]);
    int32_t *sop = (int32_t *)(ws + off[W4A8_WS_SLOT_OF_PAIR]);
    int8_t *qa = (int8_t *)(ws + off[W4A8_WS_QA]);
    float *a_scale = (float *)(ws + off[W4A8_WS_A_SCALE]);
    float *gu = (float *)(ws + off[W4A8_WS_GU]);
    int8_t *qh = (int8_t *)(ws + off[W4A8_WS_QH]);
    float *h_scale = (float *)(ws + off[W4A8_WS_H_SCALE]);
    float *y = (float *)(ws + off[W4A8_WS_Y]);
    const int64_t P = T * topk, S = P + T;
    hipError_t err = launch_moe_route(logits, T, E, topk, 1, ids, w, offsets, perm, slot_row, sop, stream);
    if (err != hipSuccess) return hip_status(err, "moe_ffn: route");
    if (T == 0) return W4A8_OK;
    if ((err = launch_quantize_act(x, T, H, H, nullptr, qa, a_scale, stream)) != hipSuccess)
        return hip_status(err, "moe_ffn: quantize");
    // top-k picks distinct experts per token, so no expert (the shared one included) gets more than T slots.
    // Experts on the three-stage tiled loop fold SiLU * up into the gate/up epilogue (their gu
    // lines then hold h and its per-16-column maxima); the requant reads either form.
    T3Epi silu;
    silu.half = I;
    int64_t fused_min = INT64_MAX;
    const bool fuse_silu = I <= 4096;
    if ((err = launch_grouped_gemm(qa, a_scale, T, slot_row, offsets, E + 1, H, gu_packed, gu_scale, gu_zp, 2 * I, S, T,
                                   gu, nullptr, W4A8_GROUP, stream, fuse_silu ? &silu : nullptr, &fused_min)) !=
        hipSuccess)
        return hip_status(err, "moe_ffn: gate/up grouped GEMM");
    if ((err = launch_moe_requant(gu, S, I, offsets, E + 1, fused_min, qh, h_scale, stream)) != hipSuccess)
        return hip_status(err, "moe_ffn: silu*up requant");
    if (shared_combine_fits(T, I, H, topk)) {
        // routed experts, then the shared one (slots P .. S, token order) with the combine folded in
        if ((err = launch_grouped_gemm(qh, h_scale, S, nullptr, offsets, E, I, dn_packed, dn_scale, dn_zp, H, S, T, y,
                                       nullptr, W4A8_GROUP, stream)) != hipSuccess)
            return hip_status(err, "moe_ffn: down grouped GEMM");
        const int64_t eb = (int64_t)E;
        if ((err = launch_shared_combine(qh + P * I, h_scale + P, T, I, dn_packed + eb * H * (I / 2),
                                         dn_scale + eb * (I / W4A8_GROUP) * H, dn_zp + eb * (I / W4A8_GROUP) * H, H,
                                         y + P * H, y, sop, w, topk, out, stream)) != hipSuccess)
            return hip_status(err, "moe_ffn: shared expert down GEMM + combine");
        return W4A8_OK;
    }
    if ((err = launch_grouped_gemm(qh, h_scale, S, nullptr, offsets, E + 1, I, dn_packed, dn_scale, dn_zp, H, S, T, y,
                                   nullptr, W4A8_GROUP, stream)) != hipSuccess)
        return hip_status(err, "moe_ffn: down grouped GEMM");
    if ((err = launch_moe_combine(y, sop, w, y + P * H, T, topk, H, out, stream)) != hipSuccess)
        return hip_status(err, "moe_ffn: combine");
    return W4A8_OK;
}

}  // namespace w4a8

extern "C" {

size_t w4a8_moe_ffn_workspace_size(int64_t T, int64_t H, int64_t I, int32_t E, int32_t topk) {
    if (check_ffn_sizes(T, H, I, E, topk) != W4A8_OK) return 0;
    int64_t off[W4A8_WS_PARTS + 1];
    ws_layout(T, H, I, E, topk, off);
    return (size_t)off[W4A8_WS_PARTS];
}

w4a8_status w4a8_moe_ffn_workspace_layout(int64_t T, int64_t H, int64_t I, int32_t E, int32_t topk, int64_t *offsets) {
    clear_error();
    W4A8_REQUIRE(offsets, W4A8_EINVAL, "null pointer");
    if (w4a8_status st = check_ffn_sizes(T, H, I, E, topk)) return st;
    ws_layout(T, H, I, E, topk, offsets);
    return W4A8_OK;
}

w4a8_status w4a8_moe_ffn(const float *x, const float *logits, int64_t T, int64_t H, int64_t I, int32_t E,
                         int32_t topk, const uint8_t *gu_packed, const uint16_t *gu_scale, const uint16_t *gu_zp,
                         const uint8_t *dn_packed, const uint16_t *dn_scale, const uint16_t *dn_zp, float *out,
                         void *workspace, size_t ws_bytes, hipStream_t stream) {
    clear_error();
    W4A8_REQUIRE(workspace, W4A8_EINVAL, "null pointer");
    W4A8_REQUIRE(((uintptr_t)workspace % kWsAlign) == 0, W4A8_EINVAL, "workspace must be 256-byte aligned");
    return w4a8::moe_ffn_run(x, logits, T, H, I, E, topk, gu_packed, gu_scale, gu_zp, dn_packed, dn_scale, dn_zp,
                             out, workspace, ws_bytes, stream);
}

}  // extern "C"
