/* gen_host.c -- host filler for the seeded synthetic inputs (test and benchmark
 * infrastructure; holds none of the W4A8 method's arithmetic).  Same bytes as
 * the numpy recipes in synthetic/__init__.py and the GPU filler gen_device.hip;
 * fp32 operations are rounded one at a time (built with -ffp-contract=off). */
#include <stdint.h>

static const uint64_t kGolden = 0x9E3779B97F4A7C15ull;

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline uint64_t bits(uint64_t key, uint64_t idx) { return mix64(key + (idx + 1) * kGolden); }

/* mode 0 plain, 1 outliers, 2 per-row mean offset (see gen_device.hip) */
void synth_fill_weights_host(float *out, uint64_t key, uint64_t key_o, int64_t row0, int64_t rows, int64_t K,
                             float unit, float stdv, int mode, uint64_t p_bits, float factor, float mu_unit)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float mu = 0.0f;
        if (mode == 2) {
            int64_t u = (int64_t)(bits(key_o, (uint64_t)(row0 + r)) >> 40);
            mu = (float)(u - (1ll << 23)) * mu_unit;
        }
        for (int64_t k = 0; k < K; ++k) {
            uint64_t idx = (uint64_t)((row0 + r) * K + k);
            uint64_t b = bits(key, idx);
            int64_t s = (int64_t)(b & 0xFFFF) + (int64_t)((b >> 16) & 0xFFFF) + (int64_t)((b >> 32) & 0xFFFF) +
                        (int64_t)(b >> 48);
            float w = ((float)(s - 131070) * unit) * stdv;
            if (mode == 1 && (bits(key_o, idx) >> 11) < p_bits)
                w = w * factor;
            if (mode == 2)
                w = mu + w;
            out[r * K + k] = w;
        }
    }
}
