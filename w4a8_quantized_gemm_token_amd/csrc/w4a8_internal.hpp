// w4a8_internal.hpp -- shared internals of libw4a8.so (gfx950 only).
//
// Error state for the C ABI, launch wrappers (one per kernel family) and small
// device helpers used by several kernels.  Nothing here is part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/w4a8.h"

namespace w4a8 {

// ---------------------------------------------------------------- error state
void set_error(const char *fmt, ...);
void clear_error();
w4a8_status hip_status(hipError_t err, const char *what);

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; arguments are already validated.
// inv_s: per-channel smoothing factors [K] (nullptr: none).
hipError_t launch_quantize_act(const float *x, int64_t M, int64_t K, int64_t ldx, const float *inv_s, int8_t *qa,
                               float *a_scale, hipStream_t stream);
hipError_t launch_silu_mul_quantize(const float *gu, int64_t P, int64_t I, int8_t *qh,
                                    float *h_scale, float *h_out, hipStream_t stream);
// s: per-channel smoothing factors [K] applied before quantization (nullptr: none).
hipError_t launch_pack_weights(const float *W, int64_t N, int64_t K, int group, const float *s, uint8_t *packed,
                               uint16_t *scale, uint16_t *zp, hipStream_t stream);
hipError_t launch_channel_absmax(const float *A, int64_t rows, int64_t K, int64_t lda, float *out,
                                 hipStream_t stream);

// Dense GEMM.  path: 1 = streaming (M <= 64), 2 = tiled.  isums != nullptr selects
// the debug epilogue that stores the per-group int32 sums instead of `out`.
hipError_t launch_gemm(const int8_t *qa, const float *a_scale, int64_t M, int64_t K,
                       const uint8_t *packed, const uint16_t *scale, const uint16_t *zp,
                       int64_t N, int path, float *out, int32_t *isums, hipStream_t stream);

// Group size 64 or 256 (K a multiple of 128 and of the group): path 1 = the decode loop
// (M <= 16, decode_group_fits), path 2 or 3 = the tiled loop (the 128-row tile unless path
// 2 has M > 128), 4 = tiled with 256-row tiles.
bool decode_group_fits(int64_t M, int64_t K, int64_t N);
hipError_t launch_gemm_tiled_group(const int8_t *qa, const float *a_scale, int64_t M, int64_t K, const uint8_t *packed,
                                   const uint16_t *scale, const uint16_t *zp, int64_t N, int group, int path, float *out,
                                   int32_t *isums, hipStream_t stream);

// Extra operands of the fused MoE epilogues of the three-stage tiled loop.
struct T3Epi {
    int64_t half = 0;               // gate/up with SiLU * up: I (gate rows [0, I), up rows [I, 2I))
    const float *y = nullptr;       // shared-expert combine: routed down rows [*][H]
    const int32_t *sop = nullptr;   //   slot of pair (t, j), [T][k]
    const float *tw = nullptr;      //   routing weights [T][k]
    int32_t k = 0;                  //   routed experts per token (<= 8)
    float *fin = nullptr;           //   layer output [T][H]
};

// max_per_expert: a bound on any one expert's slot count known to the caller (the
// MoE layer knows no expert gets more than T); loops for larger experts are not
// launched.  max_slots when nothing better is known.  isums != nullptr selects the
// debug form: per-group int32 sums isums[K/group][max_slots][N] instead of `out`.
// group: 64, 128 or 256 (scale/zp [E][K/group][N]).
// silu (group 128, MoE gate/up with N = 2 silu->half): experts that take the three-stage
// tiled loop (more than 128 slots) get SiLU(gate) * up in their epilogue: their out line
// holds h [half] and then the per-16-column maxima of |h| [half / 16] instead of gate | up;
// *fused_min is then set to 128 (left alone when no expert can take that loop).
hipError_t launch_grouped_gemm(const int8_t *qa, const float *a_scale, int64_t R,
                               const int32_t *row_index, const int32_t *expert_offsets, int32_t E,
                               int64_t K, const uint8_t *packed, const uint16_t *scale,
                               const uint16_t *zp, int64_t N, int64_t max_slots, int64_t max_per_expert,
                               float *out, int32_t *isums, int group, hipStream_t stream,
                               const T3Epi *silu = nullptr, int64_t *fused_min = nullptr);

// The MoE requant after the gate/up product: rows of experts (E1 of them, slots
// offsets[e] .. offsets[e+1]) with more than fused_min slots hold h and its per-16-column
// maxima (above), the others gate | up; qh and h_scale as launch_silu_mul_quantize.
hipError_t launch_moe_requant(const float *gu, int64_t S, int64_t I, const int32_t *offsets, int32_t E1,
                              int64_t fused_min, int8_t *qh, float *h_scale, hipStream_t stream);

// The MoE shared expert's down product over its T token rows (qh, h_scale of those rows)
// with the weighted combine folded in: y_shared [T][H] receives the product, out [T][H]
// the layer output sum_j w[t][j] y[slot(t, j)] + y_shared[t] (the combine kernel's order).
bool shared_combine_fits(int64_t T, int64_t I, int64_t H, int32_t topk);
hipError_t launch_shared_combine(const int8_t *qh, const float *h_scale, int64_t T, int64_t I, const uint8_t *packed,
                                 const uint16_t *scale, const uint16_t *zp, int64_t H, float *y_shared,
                                 const float *y, const int32_t *slot_of_pair, const float *topk_w, int32_t topk,
                                 float *out, hipStream_t stream);

// Tile-major weights for the decode loop (M <= 16): bytes of the array, whether a
// shape is served, the GEMM over it, and the conversion from the standard layout.
int64_t tm_bytes(int64_t N, int64_t K);
bool gemm_tm_supported(int64_t M, int64_t K, int64_t N);
hipError_t launch_gemm_tm(const int8_t *qa, const float *a_scale, int64_t M, int64_t K, const uint8_t *tm, int64_t N,
                          float *out, hipStream_t stream);
hipError_t launch_weights_to_tm(const uint8_t *packed, const uint16_t *scale, const uint16_t *zp, int64_t N, int64_t K,
                                uint8_t *tm, hipStream_t stream);

hipError_t launch_moe_route(const float *logits, int64_t T, int32_t E, int32_t topk, int32_t with_shared,
                            int32_t *ids, float *w, int32_t *offsets, int32_t *perm, int32_t *slot_row,
                            int32_t *slot_of_pair, hipStream_t stream);

hipError_t launch_moe_combine(const float *y, const int32_t *slot_of_pair, const float *topk_w,
                              const float *y_shared, int64_t T, int32_t topk, int64_t H, float *out,
                              hipStream_t stream);

// The MoE FFN layer over a caller-provided workspace (validated here, except the
// workspace's alignment); workspace bytes it needs, -1 for invalid sizes.
w4a8_status moe_ffn_run(const float *x, const float *logits, int64_t T, int64_t H, int64_t I, int32_t E,
                        int32_t topk, const uint8_t *gu_packed, const uint16_t *gu_scale, const uint16_t *gu_zp,
                        const uint8_t *dn_packed, const uint16_t *dn_scale, const uint16_t *dn_zp, float *out,
                        void *workspace, size_t ws_bytes, hipStream_t stream);
int64_t moe_ffn_ws_bytes(int64_t T, int64_t H, int64_t I, int32_t E, int32_t topk);

// Streaming-path threshold: the dense GEMM uses the streaming loop for M <= this.
constexpr int64_t kStreamMaxM = 64;

}  // namespace w4a8

// ---------------------------------------------------------------- device helpers
#ifdef __HIPCC__
namespace w4a8dev {

constexpr int kWave = 64;

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// Maximum over the wave, returned to every lane: DPP steps inside each 16-lane row
// (swap neighbours, swap pairs, rotate by 4 and by 8), then the four row results read
// as scalars -- no LDS round trips.
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
    const int o = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false);
    return fmaxf(v, __builtin_bit_cast(float, o));
}
__device__ __forceinline__ float wave_max(float v) {
    v = dpp_max<0xB1>(v);   // quad_perm [1,0,3,2]
    v = dpp_max<0x4E>(v);   // quad_perm [2,3,0,1]
    v = dpp_max<0x124>(v);  // row_ror:4
    v = dpp_max<0x128>(v);  // row_ror:8
    const int b = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fminf(v, __shfl_xor(v, off, kWave));
    return v;
}

// fp16 bit pattern <-> fp32 (hardware conversions, round to nearest even, subnormals kept)
__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// The MoE expert activation SiLU(g) * u = g / (1 + e^-g) * u, with e^-g = 2^(-g log2 e) from
// the hardware base-2 exponential and the quotient as g times the hardware reciprocal (about
// 1 ulp each; relative error a few 1e-7 for |g| < 20): a few instructions where the library
// exp and the correctly rounded divide take some twenty, which matters in the gate/up
// epilogue.  One definition for the unfused kernel and the fused epilogue, so both give the
// same bits.
__device__ __forceinline__ float silu_mul(float g, float u) {
    const float e = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// Per-token symmetric INT8 code of v for a row scale s (s == 0 -> 0).
// IEEE fp32 divide (the library is built with correctly rounded fp32 division),
// round half to even, clamp to [-127, 127].
__device__ __forceinline__ int quantize_i8(float v, float s) {
    if (s == 0.0f) return 0;
    float r = __builtin_rintf(v / s);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

}  // namespace w4a8dev
#endif
