// quant_kernels.hip -- the quantizers of the W4A8 layer on gfx950.
//
//  * quantize_act: per-token dynamic symmetric INT8 ([p1 §5.3]: the scale is
//    computed in the kernel at forward time; [p3 §2.1]: q = round(x/s),
//    s = max|x| / 127).  One workgroup per row; the row maximum is a wave64
//    shuffle reduction followed by a cross-wave LDS step.
//    With a per-channel factor inv_s (smoothing, [p3 §3.4]) each entry is first
//    multiplied by inv_s[k] in fp32; the maximum and the codes are taken of that
//    product, so the scaled row is never written out.
//  * silu_mul_quantize: the MoE expert activation silu(gate) * up followed by the
//    same per-row quantizer (the INT8 input of the down projection).
//  * pack_weights: group-wise asymmetric 4-bit weight quantization and nibble
//    packing ([p2 §2.1, §2.2]), one wave per (output feature, group of 128),
//    optionally of the smoothed weights W[n][k] * s[k].
//  * channel_absmax: per-channel maxima of |A| over rows, the statistic the
//    smoothing factors are computed from.
//
// Page keys: [p1] hotelren.com/news/5173946 "Kimi 2.7 MoE: from 4-bit storage to
// INT8 compute"; [p2] pptc.cn/news/121597 "Kimi 2.7 MoE, 4-bit storage to INT8,
// dissected"; [p3] hotelren.com/news/5982361 "LLM quantization primer".
//
// All three are HBM-bound streaming kernels: they read fp32 and write int8.
#include "w4a8_internal.hpp"

using namespace w4a8dev;

namespace {

constexpr int kActThreads = 256;
constexpr int kActWaves = kActThreads / kWave;

// Block-wide max of a non-negative float over kActThreads threads.
__device__ __forceinline__ float block_max(float v, float *red) {
    v = wave_max(v);
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int i = 1; i < kActWaves; ++i) m = fmaxf(m, red[i]);
    return m;
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) |
           ((uint32_t)(d & 0xFF) << 24);
}

// Four consecutive columns of a row, times the smoothing factors when SMOOTH
// (one fp32 product per entry).  VEC: row and inv_s are 16-byte aligned.
template <bool VEC, bool SMOOTH>
__device__ __forceinline__ float4 load4(const float *row, const float *inv_s, int64_t c) {
    float4 v;
    if (VEC) v = reinterpret_cast<const float4 *>(row)[c];
    else v = make_float4(row[4 * c], row[4 * c + 1], row[4 * c + 2], row[4 * c + 3]);
    if (SMOOTH) {
        float4 f;
        if (VEC) f = reinterpret_cast<const float4 *>(inv_s)[c];
        else f = make_float4(inv_s[4 * c], inv_s[4 * c + 1], inv_s[4 * c + 2], inv_s[4 * c + 3]);
        v = make_float4(v.x * f.x, v.y * f.y, v.z * f.z, v.w * f.w);
    }
    return v;
}

// x rows of K floats (stride ldx); each thread owns groups of 4 consecutive
// columns.  VEC: x rows (and inv_s) are 16-byte aligned, so float4 loads are used.
template <bool VEC, bool SMOOTH>
__global__ __launch_bounds__(kActThreads) void quantize_act_kernel(const float *__restrict__ x, int64_t K,
                                                                   int64_t ldx, const float *__restrict__ inv_s,
                                                                   int8_t *__restrict__ qa,
                                                                   float *__restrict__ a_scale) {
    __shared__ float red[kActWaves];
    const int64_t m = blockIdx.x;
    const float *row = x + m * ldx;
    const int64_t K4 = K / 4;
    float amax = 0.0f;
    for (int64_t c = threadIdx.x; c < K4; c += kActThreads) {
        const float4 v = load4<VEC, SMOOTH>(row, inv_s, c);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    amax = block_max(amax, red);
    const float s = amax / 127.0f;
    if (threadIdx.x == 0) a_scale[m] = s;
    uint32_t *out = reinterpret_cast<uint32_t *>(qa + m * K);
    for (int64_t c = threadIdx.x; c < K4; c += kActThreads) {
        const float4 v = load4<VEC, SMOOTH>(row, inv_s, c);
        out[c] = pack4_i8(quantize_i8(v.x, s), quantize_i8(v.y, s), quantize_i8(v.z, s), quantize_i8(v.w, s));
    }
}

// Single-pass form for rows of K <= 4 * VPT4 * 1024 floats: one 1024-thread workgroup
// per row keeps the row in registers between the maximum and the quantization, so
// the row is read from memory once (this is the latency-critical small-M case).
constexpr int kRowThreads = 1024;
template <int VPT4, bool SMOOTH>
__global__ __launch_bounds__(kRowThreads) void quantize_act_row_kernel(const float *__restrict__ x, int64_t K,
                                                                       int64_t ldx, const float *__restrict__ inv_s,
                                                                       int8_t *__restrict__ qa,
                                                                       float *__restrict__ a_scale) {
    __shared__ float red[kRowThreads / kWave];
    const int64_t m = blockIdx.x;
    const float *row = x + m * ldx;
    const int64_t K4 = K / 4;
    float4 v[VPT4];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < VPT4; ++i) {
        const int64_t c = threadIdx.x + (int64_t)i * kRowThreads;
        v[i] = c < K4 ? load4<true, SMOOTH>(row, inv_s, c) : make_float4(0.f, 0.f, 0.f, 0.f);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
    }
    amax = wave_max(amax);
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = red[0];
#pragma unroll
    for (int i = 1; i < kRowThreads / kWave; ++i) amax = fmaxf(amax, red[i]);
    const float s = amax / 127.0f;
    if (threadIdx.x == 0) a_scale[m] = s;
    uint32_t *out = reinterpret_cast<uint32_t *>(qa + m * K);
#pragma unroll
    for (int i = 0; i < VPT4; ++i) {
        const int64_t c = threadIdx.x + (int64_t)i * kRowThreads;
        if (c < K4)
            out[c] = pack4_i8(quantize_i8(v[i].x, s), quantize_i8(v[i].y, s), quantize_i8(v[i].z, s),
                              quantize_i8(v[i].w, s));
    }
}

// One workgroup per row p of gu [P][2I]; h lives in registers between the max
// and the quantization (VPT4 float4 per thread covers I <= 4 * VPT4 * 256).
template <int VPT4>
__global__ __launch_bounds__(kActThreads) void silu_mul_quantize_kernel(const float *__restrict__ gu, int64_t I,
                                                                        int8_t *__restrict__ qh,
                                                                        float *__restrict__ h_scale,
                                                                        float *__restrict__ h_out) {
    __shared__ float red[kActWaves];
    const int64_t p = blockIdx.x;
    const float4 *gate = reinterpret_cast<const float4 *>(gu + p * 2 * I);
    const float4 *up = reinterpret_cast<const float4 *>(gu + p * 2 * I + I);
    const int64_t I4 = I / 4;
    float4 h[VPT4];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < VPT4; ++i) {
        const int64_t c = threadIdx.x + (int64_t)i * kActThreads;
        if (c < I4) {
            const float4 g = gate[c], u = up[c];
            h[i] = make_float4(silu_mul(g.x, u.x), silu_mul(g.y, u.y), silu_mul(g.z, u.z), silu_mul(g.w, u.w));
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(h[i].x), fabsf(h[i].y)), fmaxf(fabsf(h[i].z), fabsf(h[i].w))));
            if (h_out) reinterpret_cast<float4 *>(h_out + p * I)[c] = h[i];
        }
    }
    amax = block_max(amax, red);
    const float s = amax / 127.0f;
    if (threadIdx.x == 0) h_scale[p] = s;
    uint32_t *out = reinterpret_cast<uint32_t *>(qh + p * I);
#pragma unroll
    for (int i = 0; i < VPT4; ++i) {
        const int64_t c = threadIdx.x + (int64_t)i * kActThreads;
        if (c < I4)
            out[c] = pack4_i8(quantize_i8(h[i].x, s), quantize_i8(h[i].y, s), quantize_i8(h[i].z, s),
                              quantize_i8(h[i].w, s));
    }
}

// Fallback for long rows: h recomputed in the second pass.
__global__ __launch_bounds__(kActThreads) void silu_mul_quantize_long_kernel(const float *__restrict__ gu, int64_t I,
                                                                             int8_t *__restrict__ qh,
                                                                             float *__restrict__ h_scale,
                                                                             float *__restrict__ h_out) {
    __shared__ float red[kActWaves];
    const int64_t p = blockIdx.x;
    const float *gate = gu + p * 2 * I;
    const float *up = gate + I;
    float amax = 0.0f;
    for (int64_t c = threadIdx.x; c < I; c += kActThreads) {
        const float h = silu_mul(gate[c], up[c]);
        amax = fmaxf(amax, fabsf(h));
        if (h_out) h_out[p * I + c] = h;
    }
    amax = block_max(amax, red);
    const float s = amax / 127.0f;
    if (threadIdx.x == 0) h_scale[p] = s;
    for (int64_t c = threadIdx.x; c < I; c += kActThreads) qh[p * I + c] = (int8_t)quantize_i8(silu_mul(gate[c], up[c]), s);
}

// The MoE requant after the gate/up product, kRequantRows slots per workgroup.  A slot of an
// expert with more than fused_min slots holds h [I] and the maxima of |h| over each 16
// columns [I / 16] (the fused gate/up epilogue), the others gate [I] | up [I].  The row
// maximum of |h| is the same number either way (a maximum of maxima), so the codes and
// scales are those of silu_mul_quantize_kernel for the same h.
constexpr int kRequantRows = 8;
constexpr int kMaxOffsets = 1025;
template <int VPT4>
__global__ __launch_bounds__(kActThreads) void moe_requant_kernel(const float *__restrict__ gu, int64_t S, int64_t I,
                                                                  const int32_t *__restrict__ offsets, int32_t E1,
                                                                  int64_t fused_min, int8_t *__restrict__ qh,
                                                                  float *__restrict__ h_scale) {
    __shared__ float red[kActWaves];
    __shared__ int32_t off[kMaxOffsets];
    for (int e = threadIdx.x; e <= E1; e += kActThreads) off[e] = offsets[e];
    __syncthreads();
    const int64_t I4 = I / 4;
    const int64_t p1 = ((int64_t)blockIdx.x + 1) * kRequantRows < S ? ((int64_t)blockIdx.x + 1) * kRequantRows : S;
    for (int64_t p = (int64_t)blockIdx.x * kRequantRows; p < p1; ++p) {
        // the expert of slot p: the last e with off[e] <= p
        int lo = 0, hi = E1;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (off[mid] <= p) lo = mid;
            else hi = mid;
        }
        const bool fused = (int64_t)(off[lo + 1] - off[lo]) > fused_min;
        const float4 *line = reinterpret_cast<const float4 *>(gu + p * 2 * I);
        float4 h[VPT4];
        float amax = 0.0f;
        if (fused) {
#pragma unroll
            for (int i = 0; i < VPT4; ++i) {
                const int64_t c = threadIdx.x + (int64_t)i * kActThreads;
                if (c < I4) h[i] = line[c];
            }
            for (int64_t c = threadIdx.x; c < I / 16; c += kActThreads) amax = fmaxf(amax, gu[p * 2 * I + I + c]);
        } else {
#pragma unroll
            for (int i = 0; i < VPT4; ++i) {
                const int64_t c = threadIdx.x + (int64_t)i * kActThreads;
                if (c < I4) {
                    const float4 g = line[c], u = line[I4 + c];
                    h[i] = make_float4(silu_mul(g.x, u.x), silu_mul(g.y, u.y), silu_mul(g.z, u.z),
                                       silu_mul(g.w, u.w));
                    amax = fmaxf(amax,
                                 fmaxf(fmaxf(fabsf(h[i].x), fabsf(h[i].y)), fmaxf(fabsf(h[i].z), fabsf(h[i].w))));
                }
            }
        }
        amax = block_max(amax, red);
        const float s = amax / 127.0f;
        if (threadIdx.x == 0) h_scale[p] = s;
        uint32_t *out = reinterpret_cast<uint32_t *>(qh + p * I);
#pragma unroll
        for (int i = 0; i < VPT4; ++i) {
            const int64_t c = threadIdx.x + (int64_t)i * kActThreads;
            if (c < I4)
                out[c] = pack4_i8(quantize_i8(h[i].x, s), quantize_i8(h[i].y, s), quantize_i8(h[i].z, s),
                                  quantize_i8(h[i].w, s));
        }
        __syncthreads();  // red is reused by the next row
    }
}

// One wave per unit of one output feature n and SPAN consecutive k (128, or 256 for GS 256):
//  GS 128: one group per wave; lane l owns weights 2l and 2l+1, i.e. packed byte l.
//  GS 64:  two groups per wave (lanes 0-31 and 32-63), lane l again weights 2l, 2l+1 of the
//          wave's 128 k; the range is reduced over each half-wave.
//  GS 256: one group per wave; lane l owns weights 4l .. 4l+3, i.e. packed bytes 2l, 2l+1.
// SMOOTH: each weight is first multiplied by its channel's smoothing factor
// s[k] (one fp32 product), so the smoothed matrix is never written out.
constexpr int kPackThreads = 256;

template <int GS>
__device__ __forceinline__ float unit_min(float v) {
    if constexpr (GS == 64) {
#pragma unroll
        for (int off = 16; off > 0; off >>= 1) v = fminf(v, __shfl_xor(v, off, kWave));
        return v;
    } else {
        return wave_min(v);
    }
}
template <int GS>
__device__ __forceinline__ float unit_max(float v) {
    if constexpr (GS == 64) {
#pragma unroll
        for (int off = 16; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
        return v;
    } else {
        return wave_max(v);
    }
}

template <bool SMOOTH, int GS>
__global__ __launch_bounds__(kPackThreads) void pack_weights_kernel(const float *__restrict__ W, int64_t N,
                                                                    int64_t K, const float *__restrict__ sf,
                                                                    uint8_t *__restrict__ packed,
                                                                    uint16_t *__restrict__ scale,
                                                                    uint16_t *__restrict__ zp) {
    constexpr int SPAN = GS == 256 ? 256 : 128;  // k covered by one wave
    constexpr int PER = SPAN / kWave;            // weights per lane: 2 or 4
    const int64_t U = K / SPAN;
    const int64_t unit = (int64_t)blockIdx.x * (kPackThreads / kWave) + threadIdx.x / kWave;
    if (unit >= N * U) return;
    const int64_t n = unit / U, u = unit % U;
    const int lane = threadIdx.x % kWave;
    float w[PER];
    if constexpr (PER == 2) {
        const float2 v = reinterpret_cast<const float2 *>(W + n * K + u * SPAN)[lane];
        w[0] = v.x;
        w[1] = v.y;
        if (SMOOTH) {
            const float2 f = reinterpret_cast<const float2 *>(sf + u * SPAN)[lane];
            w[0] = w[0] * f.x;
            w[1] = w[1] * f.y;
        }
    } else {
        const float4 v = reinterpret_cast<const float4 *>(W + n * K + u * SPAN)[lane];
        w[0] = v.x;
        w[1] = v.y;
        w[2] = v.z;
        w[3] = v.w;
        if (SMOOTH) {
            const float4 f = reinterpret_cast<const float4 *>(sf + u * SPAN)[lane];
            w[0] = w[0] * f.x;
            w[1] = w[1] * f.y;
            w[2] = w[2] * f.z;
            w[3] = w[3] * f.w;
        }
    }
    // the range always contains 0: zp in [0, 15], (q - zp) in [-15, 15]
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        lo = fminf(lo, w[i]);
        hi = fmaxf(hi, w[i]);
    }
    lo = unit_min<GS>(lo);
    hi = unit_max<GS>(hi);
    uint16_t sh = float_to_half_bits((hi - lo) / 15.0f);
    float s = half_bits_to_float(sh);
    if (s == 0.0f) {
        sh = 0x3C00;  // 1.0
        s = 1.0f;
    }
    const int z = (int)fminf(fmaxf(__builtin_rintf(-lo / s), 0.0f), 15.0f);
    int q[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) q[i] = min(max((int)__builtin_rintf(w[i] / s) + z, 0), 15);
    if constexpr (PER == 2) {
        packed[n * (K / 2) + u * (SPAN / 2) + lane] = (uint8_t)(q[0] | (q[1] << 4));
    } else {
        const uint16_t two = (uint16_t)((q[0] | (q[1] << 4)) | ((q[2] | (q[3] << 4)) << 8));
        reinterpret_cast<uint16_t *>(packed + n * (K / 2) + u * (SPAN / 2))[lane] = two;
    }
    // the group's first lane writes its scale and zero point ([K / GS][N])
    const bool first = GS == 64 ? (lane & 31) == 0 : lane == 0;
    if (first) {
        const int64_t g = GS == 64 ? 2 * u + (lane >> 5) : u;
        scale[g * N + n] = sh;
        zp[g * N + n] = float_to_half_bits((float)z);
    }
}

// Channel maxima out[k] = max_r |A[r][k]| (calibration for smoothing): a workgroup
// owns 64 columns, each of its 16 waves a residue class of rows, read one coalesced
// 256-byte row slice at a time; the 16 partial maxima meet in LDS.  The maximum
// does not depend on the order, so the result is exact and deterministic.
constexpr int kAbsThreads = 1024;
__global__ __launch_bounds__(kAbsThreads) void channel_absmax_kernel(const float *__restrict__ A, int64_t rows,
                                                                     int64_t K, int64_t lda, float *__restrict__ out) {
    __shared__ float part[kAbsThreads / kWave][kWave];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int64_t k = (int64_t)blockIdx.x * kWave + lane;
    float m = 0.0f;
    if (k < K)
        for (int64_t r = wave; r < rows; r += kAbsThreads / kWave) m = fmaxf(m, fabsf(A[r * lda + k]));
    part[wave][lane] = m;
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int i = 1; i < kAbsThreads / kWave; ++i) m = fmaxf(m, part[i][lane]);
        if (k < K) out[k] = m;
    }
}

}  // namespace

namespace w4a8 {

hipError_t launch_channel_absmax(const float *A, int64_t rows, int64_t K, int64_t lda, float *out,
                                 hipStream_t stream) {
    hipLaunchKernelGGL(channel_absmax_kernel, dim3((uint32_t)((K + kWave - 1) / kWave)), dim3(kAbsThreads), 0, stream,
                       A, rows, K, lda, out);
    return hipGetLastError();
}

template <bool SMOOTH>
static hipError_t quantize_act_forms(const float *x, int64_t M, int64_t K, int64_t ldx, const float *inv_s,
                                     int8_t *qa, float *a_scale, hipStream_t stream) {
    const bool vec = ((uintptr_t)x % 16 == 0) && (ldx % 4 == 0) && (!SMOOTH || (uintptr_t)inv_s % 16 == 0);
    const dim3 grid((uint32_t)M);
    if (vec && K <= 4 * 2 * kRowThreads)
        hipLaunchKernelGGL((quantize_act_row_kernel<2, SMOOTH>), grid, dim3(kRowThreads), 0, stream, x, K, ldx, inv_s,
                           qa, a_scale);
    else if (vec && K <= 4 * 4 * kRowThreads)
        hipLaunchKernelGGL((quantize_act_row_kernel<4, SMOOTH>), grid, dim3(kRowThreads), 0, stream, x, K, ldx, inv_s,
                           qa, a_scale);
    else if (vec)
        hipLaunchKernelGGL((quantize_act_kernel<true, SMOOTH>), grid, dim3(kActThreads), 0, stream, x, K, ldx, inv_s,
                           qa, a_scale);
    else
        hipLaunchKernelGGL((quantize_act_kernel<false, SMOOTH>), grid, dim3(kActThreads), 0, stream, x, K, ldx, inv_s,
                           qa, a_scale);
    return hipGetLastError();
}

hipError_t launch_quantize_act(const float *x, int64_t M, int64_t K, int64_t ldx, const float *inv_s, int8_t *qa,
                               float *a_scale, hipStream_t stream) {
    return inv_s ? quantize_act_forms<true>(x, M, K, ldx, inv_s, qa, a_scale, stream)
                 : quantize_act_forms<false>(x, M, K, ldx, nullptr, qa, a_scale, stream);
}

hipError_t launch_silu_mul_quantize(const float *gu, int64_t P, int64_t I, int8_t *qh, float *h_scale, float *h_out,
                                    hipStream_t stream) {
    const int64_t I4 = I / 4;
    const bool vec = ((uintptr_t)gu % 16 == 0) && (h_out == nullptr || (uintptr_t)h_out % 16 == 0);
    if (vec && I4 <= kActThreads * 2)
        hipLaunchKernelGGL(silu_mul_quantize_kernel<2>, dim3((uint32_t)P), dim3(kActThreads), 0, stream, gu, I, qh,
                           h_scale, h_out);
    else if (vec && I4 <= kActThreads * 4)
        hipLaunchKernelGGL(silu_mul_quantize_kernel<4>, dim3((uint32_t)P), dim3(kActThreads), 0, stream, gu, I, qh,
                           h_scale, h_out);
    else
        hipLaunchKernelGGL(silu_mul_quantize_long_kernel, dim3((uint32_t)P), dim3(kActThreads), 0, stream, gu, I, qh,
                           h_scale, h_out);
    return hipGetLastError();
}

hipError_t launch_moe_requant(const float *gu, int64_t S, int64_t I, const int32_t *offsets, int32_t E1,
                              int64_t fused_min, int8_t *qh, float *h_scale, hipStream_t stream) {
    const int64_t I4 = I / 4;
    // no fused rows, or rows the fused kernel does not take: the plain kernel
    if (fused_min == INT64_MAX || E1 + 1 > kMaxOffsets || I % 128 != 0 || I4 > kActThreads * 4 ||
        (uintptr_t)gu % 16 != 0)
        return fused_min == INT64_MAX ? launch_silu_mul_quantize(gu, S, I, qh, h_scale, nullptr, stream)
                                      : hipErrorInvalidValue;
    const dim3 grid((uint32_t)((S + kRequantRows - 1) / kRequantRows));
    if (I4 <= kActThreads * 2)
        hipLaunchKernelGGL(moe_requant_kernel<2>, grid, dim3(kActThreads), 0, stream, gu, S, I, offsets, E1,
                           fused_min, qh, h_scale);
    else
        hipLaunchKernelGGL(moe_requant_kernel<4>, grid, dim3(kActThreads), 0, stream, gu, S, I, offsets, E1,
                           fused_min, qh, h_scale);
    return hipGetLastError();
}

hipError_t launch_pack_weights(const float *W, int64_t N, int64_t K, int group, const float *s, uint8_t *packed,
                               uint16_t *scale, uint16_t *zp, hipStream_t stream) {
    const int64_t span = group == 256 ? 256 : 128;
    const int64_t units = N * (K / span);
    const int64_t per_block = kPackThreads / kWave;
    const dim3 grid((uint32_t)((units + per_block - 1) / per_block));
#define W4A8_PACK(SM, GG)                                                                                           \
    hipLaunchKernelGGL((pack_weights_kernel<SM, GG>), grid, dim3(kPackThreads), 0, stream, W, N, K, s, packed,      \
                       scale, zp)
    if (group == 64) {
        if (s) W4A8_PACK(true, 64);
        else W4A8_PACK(false, 64);
    } else if (group == 256) {
        if (s) W4A8_PACK(true, 256);
        else W4A8_PACK(false, 256);
    } else {
        if (s) W4A8_PACK(true, 128);
        else W4A8_PACK(false, 128);
    }
#undef W4A8_PACK
    return hipGetLastError();
}

}  // namespace w4a8
