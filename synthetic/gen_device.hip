// gen_device.hip -- GPU filler for the seeded synthetic inputs (test and
// benchmark infrastructure; holds none of the W4A8 method's arithmetic).
//
// Produces exactly the bytes of the numpy generator in synthetic/__init__.py:
//   bits(key, i) = mix64(key + (i + 1) * GOLDEN)   (SplitMix64 output function)
//   normal       = fp32(sum of the four 16-bit fields - 131070) * fp32(sqrt(3)/65536)
//   weight       = normal * fp32(std)
// with fp32 multiplies and adds rounded one at a time (no contraction).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t bits(uint64_t key, uint64_t idx) { return mix64(key + (idx + 1) * kGolden); }

__device__ __forceinline__ float normal(uint64_t key, uint64_t idx, float unit) {
    const uint64_t b = bits(key, idx);
    const int64_t s = (int64_t)(b & 0xFFFF) + (int64_t)((b >> 16) & 0xFFFF) + (int64_t)((b >> 32) & 0xFFFF) +
                      (int64_t)(b >> 48);
    return __fmul_rn((float)(s - 131070), unit);
}

// mode 0: plain weights; 1: + outliers (x factor where bits(key_o) >> 11 < p_bits);
// 2: + per-row mean offset mu_r = fp32(u24 - 2^23) * mu_unit with u24 = bits(key_o, r) >> 40
__global__ void fill_weights_kernel(float *__restrict__ out, uint64_t key, uint64_t key_o, int64_t row0, int64_t rows,
                                    int64_t K, float unit, float stdv, int mode, uint64_t p_bits, float factor,
                                    float mu_unit) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= rows * K) return;
    const int64_t r = i / K, k = i % K;
    const uint64_t idx = (uint64_t)((row0 + r) * K + k);
    float w = __fmul_rn(normal(key, idx, unit), stdv);
    if (mode == 1) {
        if ((bits(key_o, idx) >> 11) < p_bits) w = __fmul_rn(w, factor);
    } else if (mode == 2) {
        const int64_t u = (int64_t)(bits(key_o, (uint64_t)(row0 + r)) >> 40);
        w = __fadd_rn(__fmul_rn((float)(u - (1ll << 23)), mu_unit), w);
    }
    out[i] = w;
}

}  // namespace

extern "C" int synth_fill_weights(float *out, uint64_t key, uint64_t key_o, int64_t row0, int64_t rows, int64_t K,
                                  float unit, float stdv, int mode, uint64_t p_bits, float factor, float mu_unit,
                                  hipStream_t stream) {
    const int64_t n = rows * K;
    if (n <= 0) return 0;
    const int threads = 256;
    hipLaunchKernelGGL(fill_weights_kernel, dim3((uint32_t)((n + threads - 1) / threads)), dim3(threads), 0, stream,
                       out, key, key_o, row0, rows, K, unit, stdv, mode, p_bits, factor, mu_unit);
    return (int)hipGetLastError();
}
