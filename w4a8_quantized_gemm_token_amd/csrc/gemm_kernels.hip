// gemm_kernels.hip -- the W4A8 product on gfx950 (CDNA4) matrix cores.
//
// What is computed ([p2 §3.2, §5.4]: INT8 matmul with int32 accumulation, then
// multiply by the scales; [p1 §4.3]: 4-bit weights widened to INT8 inside the
// kernel, never through memory):
//     isum[g][m][n] = sum_{k in group g} qa[m][k] * (q[n][k] - zp[g][n])    (int32)
//     out[m][n]     = a_scale[m] * sum_g scale[g][n] * isum[g][m][n]       (fp32)
// Page keys: [p1] hotelren.com/news/5173946 "Kimi 2.7 MoE: from 4-bit storage to
// INT8 compute"; [p2] pptc.cn/news/121597 "Kimi 2.7 MoE, 4-bit storage to INT8,
// dissected" (§2.2 gives the nibble order: first code in the low nibble).
//
// Weight unpack (shared by both loops).  A packed dword d holds the codes of 8
// consecutive k: byte j = q[2j] | q[2j+1] << 4.  The low nibbles (even k) and
// high nibbles (odd k) are masked out, interleaved back into k order with two
// v_perm_b32, and turned into (q - zp) as int8 bytes by a carry-free SWAR step:
// each byte n in [0,15] plus (0x80 - zp) stays inside [0x71, 0x8F], and xor 0x80
// maps it to (n - zp) mod 256 -- the signed INT8 operand of the MFMA.
//
// The loops:
//  * decode (M <= 16, HBM-bound): one 1024-thread workgroup per CU stages the M
//    activation rows in LDS; its 16 waves stream whole 128-byte lines of their
//    columns' packed bytes through a ring in registers into
//    v_mfma_i32_16x16x64_i8, each 16-column tile split over two or four K parts.
//  * streaming (16 < M <= 64, or an odd group count): one wave owns 16 output
//    columns and all rows, activations read from memory.
//  * tiled (large M, MFMA-bound): a 512-thread workgroup computes a 256x128 tile
//    (or 256 threads a 128x128 one); each group of 128 k is staged in LDS
//    (double-buffered, padded rows), the weights are unpacked once per workgroup
//    into LDS as INT8, and each wave runs a 64x64 sub-tile with
//    v_mfma_i32_32x32x32_i8.
//  * expert-grouped forms of these, plus a weight-streaming loop on
//    v_mfma_i32_32x32x32_i8 for experts with 17..128 slots (see below).
// All keep the per-group int32 sum in the MFMA accumulator and fold it into an
// fp32 accumulator with one fma per element per group, groups in increasing g.
// Workgroups are ordered so that neighbouring column tiles run on the same XCD
// (their scale/zp rows share cache lines).
#include <algorithm>
#include <type_traits>

#include "w4a8_internal.hpp"

using namespace w4a8dev;
using w4a8::T3Epi;

namespace {

constexpr int G128 = W4A8_GROUP;

// ------------------------------------------------------------------ unpack
// zadd = 0x80808080 - zp * 0x01010101 (per-column, per-group constant)
__device__ __forceinline__ void unpack8(uint32_t d, uint32_t zadd, uint32_t &w0, uint32_t &w1) {
    const uint32_t lo = d & 0x0F0F0F0Fu;         // q0 q2 q4 q6
    const uint32_t hi = (d >> 4) & 0x0F0F0F0Fu;  // q1 q3 q5 q7
    const uint32_t n0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // q0 q1 q2 q3
    const uint32_t n1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // q4 q5 q6 q7
    w0 = (n0 + zadd) ^ 0x80808080u;
    w1 = (n1 + zadd) ^ 0x80808080u;
}

__device__ __forceinline__ uint32_t zp_add_const(uint16_t zp_bits) {
    const uint32_t z = (uint32_t)half_bits_to_float(zp_bits);
    return 0x80808080u - z * 0x01010101u;
}

// the same constant from the tile-major array's -zp byte (two's complement)
__device__ __forceinline__ uint32_t zp_add_const_neg(uint32_t neg_zp_byte) {
    const uint32_t z = (0u - neg_zp_byte) & 0xFFu;
    return 0x80808080u - __builtin_amdgcn_perm(0u, z, 0u);  // z in every byte
}

// Bijective XCD-aware order: workgroup b runs on XCD b % 8; give each XCD a
// contiguous range of tiles so that neighbouring tiles share that XCD's L2.
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t ntiles) {
    const int64_t q = ntiles / 8, r = ntiles % 8;
    const int64_t x = b % 8, i = b / 8;
    return x * q + (x < r ? x : r) + i;
}

// Tile (tm, tn) of linear position i in panel order: panels of up to PM m-tiles,
// inside a panel n fastest-varying over the panel's m-tiles.  Consecutive positions
// (the workgroups one XCD runs at a time) then cover a PM x (32 / PM) block of
// tiles, whose activation rows and weight columns its L2 serves to all of them.
template <int PM>
__device__ __forceinline__ void panel_tile(int64_t i, int64_t mt, int64_t nt, int64_t &tm, int64_t &tn) {
    const int64_t p = i / (PM * nt);
    const int64_t pm = (mt - PM * p) < PM ? (mt - PM * p) : PM;
    const int64_t ip = i - p * PM * nt;
    tm = PM * p + ip % pm;
    tn = ip / pm;
}

// Largest power of two <= umax that divides the group count G (prefetch ring depth).
__host__ __device__ inline int ring_depth(int64_t G, int umax) {
    int u = umax;
    while (u > 1 && G % u != 0) u >>= 1;
    return u;
}

// ------------------------------------------------------------------ streaming loop
constexpr int kStreamThreads = 64;

// Rows of one streaming unit: slot base, valid row count, and the activation row
// of each slot (identity for the dense layer, row_index for MoE).
struct StreamRows {
    int64_t slot0;
    int rows;
};

// One wave: 16 columns [n0, n0+16) x MT*16 rows, all K.  Lane l owns column
// n0 + (l & 15) and the k quarter kq = l >> 4 of each 64-k MFMA step: in group g
// it loads 16 packed bytes = codes g*128 + kq*32 + [0, 32), which feed MFMA step
// s = 0 (codes [0,16)) and s = 1 (codes [16,32)); the A fragment of lane l is
// row (l & 15) of the tile at the same 16 k.  16x16 accumulator: lane l holds
// rows 4*(l>>4) + r, r = 0..3, of column l & 15.
template <int MT, int U, bool ISUMS>
__device__ __forceinline__ void stream_unit(const int8_t *__restrict__ qa, const float *__restrict__ a_scale,
                                            const int32_t *__restrict__ row_index, int64_t R, StreamRows rows,
                                            int64_t K, const uint8_t *__restrict__ wpk,
                                            const uint16_t *__restrict__ wsc, const uint16_t *__restrict__ wzp,
                                            int64_t N, int64_t n0, float *__restrict__ out, int64_t ldo,
                                            int32_t *__restrict__ isums, int64_t M_isums) {
    // Every global load in the group loop is unconditional (rows outside the
    // unit read row 0 and are zeroed after the load), so the compiler can count
    // the U groups in flight exactly instead of draining the queue each group.
    const int lane = threadIdx.x & 63;
    const int kq = lane >> 4;
    const int64_t col = n0 + (lane & 15);
    const int64_t G = K / G128;  // a multiple of U (chosen by the launcher)

    const v4u *bptr = reinterpret_cast<const v4u *>(wpk + col * (K / 2) + kq * 16);
    const uint16_t *sptr = wsc + col;
    const uint16_t *zptr = wzp + col;

    const int8_t *aptr[MT];
    bool avalid[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int r = t * 16 + (lane & 15);
        int64_t row = -1;
        if (r < rows.rows) row = row_index ? (int64_t)row_index[rows.slot0 + r] : rows.slot0 + r;
        avalid[t] = row >= 0 && row < R;
        aptr[t] = qa + (avalid[t] ? row : 0) * K + kq * 32;
    }

    float acc[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][r] = 0.0f;

    v4u bq[U];
    v4u aq[U][MT][2];
    uint16_t zq[U], sq[U];

    auto load_group = [&](int u, int64_t g) {
        bq[u] = __builtin_nontemporal_load(bptr + g * (G128 / 2 / 16));
        zq[u] = zptr[g * N];
        if constexpr (!ISUMS) sq[u] = sptr[g * N];
        else sq[u] = 0;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const v4u *ap = reinterpret_cast<const v4u *>(aptr[t] + g * G128);
            aq[u][t][0] = ap[0];
            aq[u][t][1] = ap[1];
        }
    };

    // prologue in the same slot order as the loop, so the wait counts at the loop
    // head agree on both incoming paths
#pragma unroll
    for (int u = 0; u < U; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        load_group(u, u);
    }
    __builtin_amdgcn_sched_barrier(0);

    for (int64_t g0 = 0; g0 < G; g0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t g = g0 + u;
            // consume slot u in place ...
            const uint32_t zadd = zp_add_const(zq[u]);
            uint32_t w[8];
            unpack8(bq[u].x, zadd, w[0], w[1]);
            unpack8(bq[u].y, zadd, w[2], w[3]);
            unpack8(bq[u].z, zadd, w[4], w[5]);
            unpack8(bq[u].w, zadd, w[6], w[7]);
            const v4i b0 = {(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
            const v4i b1 = {(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
            const float sc = half_bits_to_float(sq[u]);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const v4i zero = {0, 0, 0, 0};
                const v4i a0 = avalid[t] ? __builtin_bit_cast(v4i, aq[u][t][0]) : zero;
                const v4i a1 = avalid[t] ? __builtin_bit_cast(v4i, aq[u][t][1]) : zero;
                v4i d = {0, 0, 0, 0};
                d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, d, 0, 0, 0);
                d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, d, 0, 0, 0);
                if (ISUMS) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int m = t * 16 + 4 * kq + r;
                        if (m < rows.rows) isums[(g * M_isums + rows.slot0 + m) * N + col] = d[r];
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[t][r] = fmaf(sc, (float)d[r], acc[t][r]);
                }
            }
            // ... then refill it U groups ahead (past the end: the last group again, never
            // consumed).  The fences keep the ring in program order so that the wait
            // before each slot's use only covers that slot's loads.
            const int64_t gn = (g + U < G) ? g + U : G - 1;
            __builtin_amdgcn_sched_barrier(0);
            load_group(u, gn);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    if (!ISUMS) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = t * 16 + 4 * kq + r;
                if (m < rows.rows) {
                    const int64_t slot = rows.slot0 + m;
                    const int64_t row = row_index ? (int64_t)row_index[slot] : slot;
                    if (row >= 0 && row < R) out[slot * ldo + col] = a_scale[row] * acc[t][r];
                }
            }
    }
}

// ------------------------------------------------------------------ streaming loop, line-wide
// The packed weights are read with every load instruction covering whole 128-byte
// lines: 8 columns x 128 B (two groups), 8 lanes per column.  Lane L of load j
// reads column 8j + (L & 7), group (L >> 3) & 1 of the two-group window, quarter
// L >> 4 (16 bytes = 32 codes).  A DPP rotate by 8 within each 16-lane row plus a
// select turns the two loads into the 16x16x64 MFMA operand layout: X (first
// group) and Y (second group) hold column L & 15, quarter L >> 4.
// Zero points are applied on the matrix cores: sum_k a_k (q_k - zp) is the MFMA of
// the raw codes plus the MFMA of the same activations with a B operand whose
// bytes are all -zp, so the weights only need their nibbles spread to bytes.
// SPLIT waves of a workgroup take disjoint halves of the groups; their fp32 sums
// are added in a fixed order through LDS at the end.
__device__ __forceinline__ uint32_t dpp_ror8(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false);
}

// nibbles of one packed dword -> 8 codes (k order) as two dwords of bytes
__device__ __forceinline__ void spread8(uint32_t d, uint32_t &w0, uint32_t &w1) {
    const uint32_t lo = d & 0x0F0F0F0Fu;
    const uint32_t hi = (d >> 4) & 0x0F0F0F0Fu;
    w0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    w1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

template <int MT, int U, int SPLIT, bool ISUMS>
__device__ __forceinline__ void stream2_unit(float *lds_red, const int8_t *__restrict__ qa,
                                             const float *__restrict__ a_scale,
                                             const int32_t *__restrict__ row_index, int64_t R, StreamRows rows,
                                             int64_t K, const uint8_t *__restrict__ wpk,
                                             const uint16_t *__restrict__ wsc, const uint16_t *__restrict__ wzp,
                                             int64_t N, int64_t n0, float *__restrict__ out, int64_t ldo,
                                             int32_t *__restrict__ isums, int64_t M_isums) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;     // split index
    const int kq = lane >> 4;
    const int64_t col = n0 + (lane & 15);  // MFMA column of this lane
    const int64_t G = K / G128;
    const int64_t nwin = G / 2 / SPLIT;    // two-group windows of this wave
    const int64_t win0 = wave * nwin;

    // weight loads: column n0 + 8j + (lane & 7), byte (lane >> 3 & 1) * 64 + kq * 16 of each window
    const int lchunk = ((lane >> 3) & 1) * 64 + kq * 16;
    const v4u *b0p = reinterpret_cast<const v4u *>(wpk + (n0 + (lane & 7)) * (K / 2) + lchunk);
    const v4u *b1p = reinterpret_cast<const v4u *>(wpk + (n0 + 8 + (lane & 7)) * (K / 2) + lchunk);
    const uint16_t *sptr = wsc + col;
    const uint16_t *zptr = wzp + col;
    const bool hi8 = (lane & 8) != 0;

    // activation rows; rows outside the unit read row 0 and are never stored
    const int8_t *aptr[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int r = t * 16 + (lane & 15);
        int64_t row = -1;
        if (r < rows.rows) row = row_index ? (int64_t)row_index[rows.slot0 + r] : rows.slot0 + r;
        aptr[t] = qa + ((row >= 0 && row < R) ? row : 0) * K + kq * 32;
    }

    float acc[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][r] = 0.0f;

    v4u rb0[U], rb1[U];
    v4u ra[U][MT][2][2];   // [slot][row tile][group of window][step]
    uint16_t rs[U][2], rz[U][2];

    auto load_window = [&](int u, int64_t w) {
        rb0[u] = __builtin_nontemporal_load(b0p + w * 8);
        rb1[u] = __builtin_nontemporal_load(b1p + w * 8);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if constexpr (!ISUMS) rs[u][h] = sptr[(2 * w + h) * N];
            else rs[u][h] = 0;
            rz[u][h] = zptr[(2 * w + h) * N];
        }
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const v4u *ap = reinterpret_cast<const v4u *>(aptr[t] + (2 * w + h) * G128);
                ra[u][t][h][0] = ap[0];
                ra[u][t][h][1] = ap[1];
            }
    };

#pragma unroll
    for (int u = 0; u < U; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        load_window(u, win0 + u);
    }
    __builtin_amdgcn_sched_barrier(0);

    for (int64_t w0 = 0; w0 < nwin; w0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t w = win0 + w0 + u;
            // operand layout: X = first group, Y = second group of the window
            uint32_t xy[2][4];
            {
                const uint32_t r0[4] = {rb0[u].x, rb0[u].y, rb0[u].z, rb0[u].w};
                const uint32_t r1[4] = {rb1[u].x, rb1[u].y, rb1[u].z, rb1[u].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t t1 = dpp_ror8(r1[i]);
                    const uint32_t t0 = dpp_ror8(r0[i]);
                    xy[0][i] = hi8 ? t1 : r0[i];
                    xy[1][i] = hi8 ? r1[i] : t0;
                }
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t q[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) spread8(xy[h][i], q[2 * i], q[2 * i + 1]);
                const v4i bq0 = {(int)q[0], (int)q[1], (int)q[2], (int)q[3]};
                const v4i bq1 = {(int)q[4], (int)q[5], (int)q[6], (int)q[7]};
                const int zneg = -(int)half_bits_to_float(rz[u][h]);
                const int z4 = (int)((uint32_t)(zneg & 0xFF) * 0x01010101u);
                const v4i bz = {z4, z4, z4, z4};
                const float sc = half_bits_to_float(rs[u][h]);
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const v4i a0 = __builtin_bit_cast(v4i, ra[u][t][h][0]);
                    const v4i a1 = __builtin_bit_cast(v4i, ra[u][t][h][1]);
                    v4i d = {0, 0, 0, 0};
                    d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, bq0, d, 0, 0, 0);
                    d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, bq1, d, 0, 0, 0);
                    d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, bz, d, 0, 0, 0);
                    d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, bz, d, 0, 0, 0);
                    if (ISUMS) {
                        const int64_t g = 2 * w + h;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int m = t * 16 + 4 * kq + r;
                            if (m < rows.rows) isums[(g * M_isums + rows.slot0 + m) * N + col] = d[r];
                        }
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[t][r] = fmaf(sc, (float)d[r], acc[t][r]);
                    }
                }
            }
            // refill the slot U windows ahead (past the end: the last window, never consumed)
            const int64_t wn = (w0 + u + U < nwin) ? w + U : win0 + nwin - 1;
            __builtin_amdgcn_sched_barrier(0);
            load_window(u, wn);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    if (!ISUMS) {
        if (SPLIT > 1) {
            // fixed-order reduction of the K halves: wave 0 + wave 1
            if (wave == 1) {
#pragma unroll
                for (int t = 0; t < MT; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) lds_red[(t * 4 + r) * 64 + lane] = acc[t][r];
            }
            __syncthreads();
            if (wave == 1) return;
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[t][r] += lds_red[(t * 4 + r) * 64 + lane];
        }
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = t * 16 + 4 * kq + r;
                if (m < rows.rows) {
                    const int64_t slot = rows.slot0 + m;
                    const int64_t row = row_index ? (int64_t)row_index[slot] : slot;
                    if (row >= 0 && row < R) out[slot * ldo + col] = a_scale[row] * acc[t][r];
                }
            }
    }
}

// ------------------------------------------------------------------ decode loop, activations in LDS
// For M <= 16 every wave needs the same activation rows; reading them through the
// vector memory path costs twice the address-unit time of the weights.  Here one
// 1024-thread workgroup per CU stages qa[M][K] in LDS once (rows padded by 16 bytes
// so the 16 rows of an MFMA fragment fall in different banks); its 16 waves then
// stream full-line weight windows (as in the loop above) and read activation
// fragments from LDS.  Workgroup b owns a contiguous range of 16-column tiles; wave
// w takes tile w / SPLIT, K part w % SPLIT of each round, and the parts are added
// through LDS at the end of the round (fixed order: part 0 + part 1 + ...).
constexpr int kDecWaves = 16;
constexpr int kDecThreads = kDecWaves * 64;

__host__ __device__ inline int64_t dec_lds_bytes(int64_t M, int64_t K) { return M * (K + 16); }
// partial sums of K parts 1..split-1 of one round: [part][tile][4][64] fp32
__host__ __device__ inline int64_t dec_red_bytes(int split) { return (int64_t)(split - 1) * (kDecWaves / split) * 1024; }
constexpr int64_t kDecLdsMax = 140 * 1024;
// packed bytes of one matrix the decode loop can address (32-bit buffer offsets; the
// offset 0xFFFFFFF0 must stay past the end)
constexpr int64_t kDecCodesMax = 0xFFFFFFF0ll;

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// s_waitcnt immediate for "vmcnt <= vm, lgkmcnt <= lgkm" (gfx9 encoding; expcnt not waited)
constexpr int t3_waitcnt(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

// Raw buffer resource over [p, p + 4 GB): no stride, no format conversion.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)0xFFFFFFFF, 0x00020000);
}

// Copy `nrows` activation rows of K bytes (source row src_row(r)) into LDS rows of
// stride lda, straight from memory to LDS (buffer_load ... lds: lane L of a load
// fills bytes [16 L, 16 L + 16) of a 1 KB block); lanes past the end of a row are
// switched off.  Source offsets src_row(r) * K must stay below 2^32.  The caller
// waits for the loads (vmcnt) before the rows are read.
template <typename SrcRow>
__device__ __forceinline__ void stage_rows_dma(uint8_t *lds, int64_t lda, const int8_t *qa, int64_t K, int nrows,
                                               SrcRow src_row) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(qa);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
    const int bpr = (int)((K + 1023) / 1024);  // 1 KB blocks per row
    for (int i = wave; i < nrows * bpr; i += nwaves) {
        const int r = i / bpr;
        const int b = i - r * bpr;
        if (b * 1024 + lane * 16 < K) {
            const uint32_t off = (uint32_t)(src_row(r) * K + b * 1024 + lane * 16);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(lds + r * lda + b * 1024), 16, (int)off, 0, 0, 0);
        }
    }
}

// Tiles [t0, t1) of 16 columns for the M <= 16 activation rows staged in `rows`
// (row stride K + 16).  `store(m, col, v)` receives a_scale-free fp32 sums; with
// ISUMS the per-group int32 sums go to `istore(g, m, col, v)` instead.
// `stage(0)` runs before the first weight windows are issued and may start loading the
// rows; `stage(1)` runs after them (so their latency overlaps it) and is followed by a
// workgroup barrier: it fills `rows` when they change.
// Tile-major weights (TM): for 16-column tile t and two-group window w, block
// (t * G/2 + w) of kTmBlock bytes holds the first group's codes (the 16 bytes at 16 l:
// column 16 t + (l & 15), codes 32 (l >> 4) + [0, 32) of that column's group, l = 0..63,
// each run of 8 codes c0..c7 as 4 bytes c_b | c_{b+4} << 4), the second group's the same
// way, then for each column c = 0..15 eight bytes at 2048 + 8 c: the fp16 scales of
// groups 2 w and 2 w + 1, then the bytes -zp of the two groups (two's complement), then
// two zero bytes.  A wave's windows are then one contiguous stream, lane l's 16-byte
// loads land directly in the 16x16x64 MFMA operand layout, a dword's low and high
// nibbles are codes 0-3 and 4-7 in order (a mask and a shift, no byte permutes), one
// 8-byte load gives a lane its column's scales and zero points (no cross-lane moves),
// and the -zp operand of the zero-point MFMA is one byte replicated (one v_perm).
constexpr int64_t kTmBlock = 2 * 1024 + 128;

// Group size GS (standard layout only; the tile-major array is defined for 128): a window
// always covers 256 k.  GS = 256: the window is one group, its two 128-k halves add into the
// same int32 sums, one fp32 fold per window.  GS = 64: each 128-k half holds two groups, k
// 0..63 in lanes kq < 2 and k 64..127 in lanes kq >= 2, so each half runs its MFMAs twice,
// with the A operand zeroed in the other lanes, and folds the two sums with their own scales;
// the -zp operand of each lane is its own group's.
template <int U, int SPLIT, bool ISUMS, bool TM, int GS, typename Stage, typename Store, typename IStore>
__device__ __forceinline__ void dec_tiles(const uint8_t *rows, float *red, int M, int64_t K,
                                          const uint8_t *__restrict__ wpk, const uint16_t *__restrict__ wsc,
                                          const uint16_t *__restrict__ wzp, int64_t N, int64_t t0, int64_t t1,
                                          Stage stage, Store store, IStore istore) {
    const int64_t lda = K + 16;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int kq = lane >> 4;
    const int half = wave % SPLIT;
    const int64_t G = K / G128;
    const int64_t nwin = G / 2 / SPLIT;
    const int64_t win0 = half * nwin;
    constexpr int per_round = kDecWaves / SPLIT;
    const int arow = (lane & 15) < M ? (lane & 15) : 0;
    const uint8_t *abase = rows + arow * lda + kq * 32;
    const int lchunk = ((lane >> 3) & 1) * 64 + kq * 16;
    const bool hi8 = (lane & 8) != 0;

    // Each wave streams tile t0 + wave / SPLIT, then the tile per_round further, and so
    // on; the window ring runs on across tiles, so the first windows of a wave's
    // next tile are already in flight while it finishes the current one.
    // Codes are read through a range-checked buffer over the N x K/2 packed bytes (its
    // size is below 2^32, which the launcher checks): 32-bit offsets, and an offset past
    // the end reads zeros without touching memory.
    // (TM: the buffer covers the whole tile-major array, codes and scales)
    const int64_t wbytes = TM ? (N / 16) * (G / 2) * kTmBlock : N * (K / 2);
    const __amdgpu_buffer_rsrc_t wrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(wpk), (short)0, (int)(uint32_t)wbytes, 0x00020000);
    const uint32_t colbyte = TM ? (uint32_t)(16 * lane) : (uint32_t)((lane & 7) * (K / 2) + lchunk);
    const uint32_t szbyte = 2048u + 8u * (uint32_t)(lane & 15);  // TM: this lane's column's words
    static_assert(GS == 128 || (!TM && (GS == 64 || GS == 256)), "group size");
    // Standard layout, fp16 words per window and column, one per lane (spread with ds_bpermute):
    //  GS 128: lanes kq = 0..3 read scale[2w], scale[2w+1], zp[2w], zp[2w+1]
    //  GS 256: lanes kq < 2 read scale[w], lanes kq >= 2 read zp[w]
    //  GS 64:  lane kq reads scale[4w + kq] (rsz) and zp[4w + kq] (rszb)
    // (the debug form stores int32 sums and reads no scales: the lanes that hold scale words
    // load nothing; their address is formed over the zero points)
    const bool sz_load = !ISUMS || (GS != 64 && kq >= 2);
    const uint16_t *szbase =
        TM ? nullptr
           : (GS == 64 ? (ISUMS ? wzp : wsc) + kq * N
                       : ((kq < 2 && !ISUMS) ? wsc : wzp) + (GS == 128 ? (kq & 1) * N : 0)) + (lane & 15);
    const uint16_t *zbase64 = wzp + kq * N + (lane & 15);
    constexpr int SZSTEP = GS == 64 ? 4 : (GS == 128 ? 2 : 1);  // scale/zp rows per window
    v4u rb0[U], rb1[U];
    uint32_t rsz[U];   // standard layout: one fp16 word per lane (spread with ds_bpermute)
    uint32_t rszb[U];  // GS 64: this lane's zero-point word
    v2u rsz2[U];       // tile-major: the four words of this lane's column
    // first byte of window w of tile `tile`, less this lane's part
    // TM: 32-bit arithmetic (every offset is below the buffer size), with the product
    // kept apart from the add: fused into a 64-bit multiply-add, its unused high half has
    // been paired with a register that a staging load was still filling, so the first
    // weight loads waited for the staged rows.
    auto window_base = [&](int64_t tile, int64_t w) -> uint32_t {
        if constexpr (TM) {
            uint32_t p = (uint32_t)tile * (uint32_t)(G / 2);
            __asm__("" : "+v"(p));
            return (p + (uint32_t)w) * (uint32_t)kTmBlock;
        } else {
            return (uint32_t)(tile * 16 * (K / 2)) + (uint32_t)w * 128;
        }
    };
    auto load_window = [&](int u, int64_t tile, int64_t w) {
        const uint32_t o = window_base(tile, w) + colbyte;
        if constexpr (TM) {
            rb0[u] = __builtin_amdgcn_raw_buffer_load_b128(wrs, o, 0, 2);
            rb1[u] = __builtin_amdgcn_raw_buffer_load_b128(wrs, o + 1024u, 0, 2);
            rsz2[u] = __builtin_amdgcn_raw_buffer_load_b64(wrs, o - colbyte + szbyte, 0, 2);
        } else {
            rb0[u] = __builtin_amdgcn_raw_buffer_load_b128(wrs, o, 0, 2);
            rb1[u] = __builtin_amdgcn_raw_buffer_load_b128(wrs, o + (uint32_t)(8 * (K / 2)), 0, 2);
            rsz[u] = sz_load ? szbase[tile * 16 + SZSTEP * w * N] : 0u;
            if constexpr (GS == 64) rszb[u] = zbase64[tile * 16 + SZSTEP * w * N];
        }
    };
    stage(0);  // issue the staging loads (older than the ring's, so waiting for them does not wait for the weights)
    {
        // every wave issues its first windows, with no branch (so the memory-counter waits
        // for the staged rows stay exact); a wave without a tile reads past the end of
        // the codes (zeros, no memory traffic) and its scales from a valid tile
        const bool has = (wave / SPLIT) < per_round && t0 + wave / SPLIT < t1;
        const int64_t tile = has ? t0 + wave / SPLIT : t0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            __builtin_amdgcn_sched_barrier(0);
            const uint32_t o = window_base(tile, win0 + u) + colbyte;
            if constexpr (TM) {
                rb0[u] = __builtin_amdgcn_raw_buffer_load_b128(wrs, has ? o : 0xFFFFFFF0u, 0, 2);
                rb1[u] = __builtin_amdgcn_raw_buffer_load_b128(wrs, has ? o + 1024u : 0xFFFFFFF0u, 0, 2);
                rsz2[u] = __builtin_amdgcn_raw_buffer_load_b64(wrs, has ? o - colbyte + szbyte : 0xFFFFFFF0u, 0, 2);
            } else {
                rb0[u] = __builtin_amdgcn_raw_buffer_load_b128(wrs, has ? o : 0xFFFFFFF0u, 0, 2);
                rb1[u] = __builtin_amdgcn_raw_buffer_load_b128(wrs, has ? o + (uint32_t)(8 * (K / 2)) : 0xFFFFFFF0u, 0,
                                                              2);
                rsz[u] = sz_load ? szbase[tile * 16 + SZSTEP * (win0 + u) * N] : 0u;
                if constexpr (GS == 64) rszb[u] = zbase64[tile * 16 + SZSTEP * (win0 + u) * N];
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    stage(1);
    __syncthreads();
    for (int64_t tb = t0; tb < t1; tb += per_round) {
        const int64_t tile = tb + wave / SPLIT;
        const bool active = (wave / SPLIT) < per_round && tile < t1;
        const int64_t ntile = tile + per_round < t1 ? tile + per_round : tile;  // where the ring runs on to
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (active) {
            const int64_t n0 = tile * 16;
            const int64_t col = n0 + (lane & 15);
            for (int64_t w0 = 0; w0 < nwin; w0 += U) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t w = win0 + w0 + u;
                    uint32_t xy[2][4];
                    {
                        const uint32_t r0[4] = {rb0[u].x, rb0[u].y, rb0[u].z, rb0[u].w};
                        const uint32_t r1[4] = {rb1[u].x, rb1[u].y, rb1[u].z, rb1[u].w};
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            if constexpr (TM) {
                                xy[0][i] = r0[i];
                                xy[1][i] = r1[i];
                            } else {
                                const uint32_t t1v = dpp_ror8(r1[i]);
                                const uint32_t t0v = dpp_ror8(r0[i]);
                                xy[0][i] = hi8 ? t1v : r0[i];
                                xy[1][i] = hi8 ? r1[i] : t0v;
                            }
                        }
                    }
                    uint32_t sz[4];  // scale g0, scale g1, zp g0, zp g1 of this lane's column
                    uint32_t sz64[4];  // GS 64: zp of the window's four groups
                    if constexpr (TM) {
                        sz[0] = rsz2[u][0] & 0xFFFFu;
                        sz[1] = rsz2[u][0] >> 16;
                        sz[2] = rsz2[u][1] & 0xFFFFu;
                        sz[3] = rsz2[u][1] >> 16;
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            sz[i] = (uint32_t)__builtin_amdgcn_ds_bpermute((i * 16 + (lane & 15)) * 4, (int)rsz[u]);
                        if constexpr (GS == 64) {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                sz64[i] =
                                    (uint32_t)__builtin_amdgcn_ds_bpermute((i * 16 + (lane & 15)) * 4, (int)rszb[u]);
                        }
                    }
                    v4i dw = {0, 0, 0, 0};  // GS 256: the window's sums
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int64_t g = 2 * w + h;
                        const v4i a0 = *reinterpret_cast<const v4i *>(abase + g * G128);
                        const v4i a1 = *reinterpret_cast<const v4i *>(abase + g * G128 + 16);
                        uint32_t q[8];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            if constexpr (TM) {
                                q[2 * i] = xy[h][i] & 0x0F0F0F0Fu;
                                q[2 * i + 1] = (xy[h][i] >> 4) & 0x0F0F0F0Fu;
                            } else {
                                spread8(xy[h][i], q[2 * i], q[2 * i + 1]);
                            }
                        }
                        const v4i bq0 = {(int)q[0], (int)q[1], (int)q[2], (int)q[3]};
                        const v4i bq1 = {(int)q[4], (int)q[5], (int)q[6], (int)q[7]};
                        int z4;
                        if constexpr (TM) {
                            z4 = (int)__builtin_amdgcn_perm(0u, rsz2[u][1], h ? 0x01010101u : 0u);
                        } else {
                            const uint32_t zb = GS == 64 ? (kq < 2 ? sz64[2 * h] : sz64[2 * h + 1])
                                                         : (GS == 256 ? sz[2] : sz[2 + h]);
                            const int zneg = -(int)half_bits_to_float((uint16_t)zb);
                            z4 = (int)((uint32_t)(zneg & 0xFF) * 0x01010101u);
                        }
                        const v4i bz = {z4, z4, z4, z4};
                        if constexpr (GS == 64) {
                            // the two 64-k groups of this half: lanes kq < 2, then kq >= 2
                            const v4i zero = {0, 0, 0, 0};
#pragma unroll
                            for (int s2 = 0; s2 < 2; ++s2) {
                                const bool mine = (kq >> 1) == s2;
                                const v4i b0 = mine ? a0 : zero, b1 = mine ? a1 : zero;
                                v4i d = {0, 0, 0, 0};
                                d = __builtin_amdgcn_mfma_i32_16x16x64_i8(b0, bq0, d, 0, 0, 0);
                                d = __builtin_amdgcn_mfma_i32_16x16x64_i8(b1, bq1, d, 0, 0, 0);
                                d = __builtin_amdgcn_mfma_i32_16x16x64_i8(b0, bz, d, 0, 0, 0);
                                d = __builtin_amdgcn_mfma_i32_16x16x64_i8(b1, bz, d, 0, 0, 0);
                                const int64_t g64 = 2 * g + s2;
                                if (ISUMS) {
#pragma unroll
                                    for (int r = 0; r < 4; ++r) {
                                        const int m = 4 * kq + r;
                                        if (m < M) istore(g64, m, col, d[r]);
                                    }
                                } else {
                                    float sc = half_bits_to_float((uint16_t)sz[2 * h + s2]);
                                    __asm__ volatile("" : "+v"(sc));
#pragma unroll
                                    for (int r = 0; r < 4; ++r) acc[r] = fmaf(sc, (float)d[r], acc[r]);
                                }
                            }
                        } else {
                            v4i d = GS == 256 ? dw : v4i{0, 0, 0, 0};
                            d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, bq0, d, 0, 0, 0);
                            d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, bq1, d, 0, 0, 0);
                            d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, bz, d, 0, 0, 0);
                            d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, bz, d, 0, 0, 0);
                            if (GS == 256 && h == 0) {
                                dw = d;  // the window's second half adds into the same sums
                            } else if (ISUMS) {
                                const int64_t gg = GS == 256 ? w : g;
#pragma unroll
                                for (int r = 0; r < 4; ++r) {
                                    const int m = 4 * kq + r;
                                    if (m < M) istore(gg, m, col, d[r]);
                                }
                            } else {
                                float sc = half_bits_to_float((uint16_t)sz[GS == 256 ? 0 : h]);
                                __asm__ volatile("" : "+v"(sc));  // one conversion, plain fmas
#pragma unroll
                                for (int r = 0; r < 4; ++r) acc[r] = fmaf(sc, (float)d[r], acc[r]);
                            }
                        }
                    }
                    // refill: window w + U of this tile, else the next tile's window
                    // (w + U - nwin) of the same K half, else (last tile) a repeat
                    const int64_t wa = w0 + u + U;
                    const bool here = wa < nwin;
                    const int64_t lt = here ? tile : ntile;
                    const int64_t lw = here ? win0 + wa : (ntile != tile ? win0 + wa - nwin : win0 + nwin - 1);
                    __builtin_amdgcn_sched_barrier(0);
                    load_window(u, lt, lw);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        if (!ISUMS) {
            if (SPLIT > 1) {  // K parts 1.. leave their sums in LDS; part 0 adds them in order
                if (active && half != 0) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        red[(((half - 1) * per_round + wave / SPLIT) * 4 + r) * 64 + lane] = acc[r];
                }
                __syncthreads();
                if (active && half == 0) {
#pragma unroll
                    for (int h = 1; h < SPLIT; ++h)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[r] += red[(((h - 1) * per_round + wave / SPLIT) * 4 + r) * 64 + lane];
                }
                __syncthreads();
            }
            if (active && half == 0) {
                const int64_t col = tile * 16 + (lane & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = 4 * kq + r;
                    if (m < M) store(m, col, acc[r]);
                }
            }
        }
    }
}

template <int U, int SPLIT, bool ISUMS, int SB, bool TM, int GS = G128>
__global__ __launch_bounds__(kDecThreads) void gemm_decode_kernel(const int8_t *__restrict__ qa,
                                                                 const float *__restrict__ a_scale, int64_t M,
                                                                 int64_t K, const uint8_t *__restrict__ wpk,
                                                                 const uint16_t *__restrict__ wsc,
                                                                 const uint16_t *__restrict__ wzp, int64_t N,
                                                                 int64_t tiles_per_wg, float *__restrict__ out,
                                                                 int32_t *__restrict__ isums) {
    extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
    __shared__ float sasc[16];  // row scales (no global load, and no wait, at the stores)
    const int64_t lda = K + 16;
    const int64_t ntiles = N / 16;
    const int64_t t0 = (int64_t)blockIdx.x * tiles_per_wg;
    const int64_t t1 = (t0 + tiles_per_wg < ntiles) ? t0 + tiles_per_wg : ntiles;
    float *red = reinterpret_cast<float *>(dsm + ((dec_lds_bytes(M, K) + 15) / 16) * 16);
    constexpr int kStageBatch = SB;  // staging loads per thread issued at once
    const bool batched = M * K <= (int64_t)kStageBatch * kDecThreads * 16;
    v4u stg[kStageBatch];
    float asc = 0.0f;
    dec_tiles<U, SPLIT, ISUMS, TM, GS>(
        dsm, red, (int)M, K, wpk, wsc, wzp, N, t0, t1,
        [&](int phase) {  // qa[M][K] -> LDS
            if constexpr (TM) {
                // straight from memory to LDS (no registers, no LDS write instructions);
                // the first U weight windows (three loads each) are issued between the
                // two phases, so waiting for all but 3 U loads covers exactly the rows
                if (phase == 0) {
                    stage_rows_dma(dsm, lda, qa, K, (int)M, [](int r) { return (int64_t)r; });
                    if (threadIdx.x < M) asc = a_scale[threadIdx.x];
                    return;
                }
                __builtin_amdgcn_s_waitcnt(t3_waitcnt(3 * U, 15));
                if (threadIdx.x < M) sasc[threadIdx.x] = asc;
                return;
            }
            if (phase == 0) {  // 16-byte pieces through registers
                // up to eight pieces per thread in flight at once; pieces past the end
                // read as zeros (buffer range check) and are not stored
                if (batched) {
                    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                        const_cast<int8_t *>(qa), (short)0, (int)(M * K), 0x00020000);
#pragma unroll
                    for (int j = 0; j < kStageBatch; ++j)
                        stg[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * ((int)threadIdx.x + j * kDecThreads), 0, 0);
                }
                if (!ISUMS && threadIdx.x < M) asc = a_scale[threadIdx.x];
                return;
            }
            if (batched) {
                // piece i sits at byte 16 i of qa and at 16 (i + i / (K / 16)) in LDS
                const int kp = (int)(K / 16), pieces = (int)M * kp;
#pragma unroll
                for (int j = 0; j < kStageBatch; ++j) {
                    const int i = (int)threadIdx.x + j * kDecThreads;
                    if (i < pieces) *reinterpret_cast<v4u *>(dsm + 16 * (int64_t)(i + i / kp)) = stg[j];
                }
            } else {
                const int64_t pieces = M * (K / 16);
                for (int64_t i = threadIdx.x; i < pieces; i += kDecThreads) {
                    const int64_t r = i / (K / 16), c = i % (K / 16);
                    *reinterpret_cast<v4u *>(dsm + r * lda + c * 16) = reinterpret_cast<const v4u *>(qa + r * K)[c];
                }
            }
            if (!ISUMS && threadIdx.x < M) sasc[threadIdx.x] = asc;
        },
        [&](int m, int64_t col, float v) { out[m * N + col] = sasc[m] * v; },
        [&](int64_t g, int m, int64_t col, int32_t v) { isums[(g * M + m) * N + col] = v; });
}

// Dense layer through the line-wide loop: a workgroup of SPLIT waves per 16-column tile.
template <int MT, int U, int SPLIT, bool ISUMS>
__global__ __launch_bounds__(64 * SPLIT) void gemm_stream2_kernel(const int8_t *__restrict__ qa,
                                                                  const float *__restrict__ a_scale, int64_t M,
                                                                  int64_t K, const uint8_t *__restrict__ packed,
                                                                  const uint16_t *__restrict__ scale,
                                                                  const uint16_t *__restrict__ zp, int64_t N,
                                                                  float *__restrict__ out,
                                                                  int32_t *__restrict__ isums) {
    __shared__ float red[MT * 4 * 64];
    const int64_t ntiles = N / 16;
    const int64_t tile = xcd_tile(blockIdx.x, ntiles);
    stream2_unit<MT, U, SPLIT, ISUMS>(red, qa, a_scale, nullptr, M, StreamRows{0, (int)M}, K, packed, scale, zp, N,
                                      tile * 16, out, N, isums, M);
}

// Dense layer, M <= 16*MT: one wave per 16-column tile.
template <int MT, int U, bool ISUMS>
__global__ __launch_bounds__(kStreamThreads) void gemm_stream_kernel(const int8_t *__restrict__ qa,
                                                                     const float *__restrict__ a_scale, int64_t M,
                                                                     int64_t K, const uint8_t *__restrict__ packed,
                                                                     const uint16_t *__restrict__ scale,
                                                                     const uint16_t *__restrict__ zp, int64_t N,
                                                                     float *__restrict__ out,
                                                                     int32_t *__restrict__ isums) {
    const int64_t ntiles = N / 16;
    const int64_t tile = xcd_tile(blockIdx.x, ntiles);
    stream_unit<MT, U, ISUMS>(qa, a_scale, nullptr, M, StreamRows{0, (int)M}, K, packed, scale, zp, N, tile * 16,
                              out, N, isums, M);
}

// ------------------------------------------------------------------ tiled loop
// A workgroup of WM x WN waves computes a (64 WM) x (64 WN) tile; each wave a 64x64
// sub-tile as 2x2 v_mfma_i32_32x32x32_i8 tiles.  Per group of 128 k the workgroup
// stages the activation rows (INT8) and the weight columns (unpacked once, to INT8
// (q - zp)) in LDS, double-buffered, rows padded to 144 bytes so the 128-bit
// fragment reads of 32 rows are bank-conflict free.  The next group's global loads
// are issued before the current group's MFMAs and only waited on when they are
// written to the idle LDS buffer (one barrier per group).
// Rows/columns outside the matrix read row/column 0: their results are never
// stored, so no masking is needed anywhere in the loop.
// Lane l of a 32x32 tile feeds A row (l&31) / B column (l&31) with k bytes
// ks*32 + (l>>5)*16 + [0,16), and holds accumulator rows 8*(r>>2) + 4*(l>>5) + (r&3),
// r = 0..15, of column l&31.
// Group size GS ([p2 §4.3] and the tuning notes of [p1]/[p2] weigh 64, 128 and 256):
// the LDS stage stays 128 k.  GS = 256 keeps the int32 sums of two stages in the same
// accumulators and runs the fp32 epilogue once per two stages (half the epilogue work);
// GS = 64 runs the MFMAs of each stage as two k halves with an epilogue after each
// (twice the epilogue work), and each thread unpacks its codes with the zero point of
// the 64-group they lie in.
constexpr int kLdsStride = G128 + 16;  // padded row: 144 bytes

struct TileRows {
    int64_t slot0;
    int rows;  // valid rows in this tile
};

template <int WM, int WN>
struct TileShape {
    static constexpr int BM = 64 * WM, BN = 64 * WN, THREADS = 64 * WM * WN;
    static constexpr int A_TPR = THREADS / BM;          // threads per A row
    static constexpr int A_BYTES = G128 / A_TPR;        // A bytes per thread per group
    static constexpr int B_TPC = THREADS / BN;          // threads per B column
    static constexpr int B_PACKED = (G128 / 2) / B_TPC; // packed B bytes per thread per group
    static constexpr int LDS_A = BM * kLdsStride, LDS_B = BN * kLdsStride;
    static constexpr int LDS_STAGE = LDS_A + LDS_B;
    static_assert(A_BYTES % 16 == 0 && B_PACKED % 16 == 0, "loader granularity");
};

template <int WM, int WN, bool ISUMS, int GS = G128>
__device__ __forceinline__ void tile2_unit(uint8_t *lds, const int8_t *__restrict__ qa,
                                           const float *__restrict__ a_scale, const int32_t *__restrict__ row_index,
                                           int64_t R, TileRows rows, int64_t K, const uint8_t *__restrict__ wpk,
                                           const uint16_t *__restrict__ wsc, const uint16_t *__restrict__ wzp,
                                           int64_t N, int64_t n0, float *__restrict__ out, int64_t ldo,
                                           int32_t *__restrict__ isums, int64_t M_isums) {
    using S = TileShape<WM, WN>;
    constexpr int NA = S::A_BYTES / 16, NB = S::B_PACKED / 16;
    static_assert(GS == 64 || GS == 128 || GS == 256, "group size");
    static_assert(GS != 64 || 2 * S::B_PACKED <= 64, "a thread's codes must lie in one 64-group");
    constexpr int NSUB = GS == 64 ? 2 : 1;  // groups per 128-k stage
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int64_t G = K / G128;  // 128-k stages

    // ---- loader state
    const int arow_l = tid / S::A_TPR, apart = tid % S::A_TPR;
    int64_t arow = -1;
    if (arow_l < rows.rows) arow = row_index ? (int64_t)row_index[rows.slot0 + arow_l] : rows.slot0 + arow_l;
    // row scales for the epilogue, read now (they arrive during the group loop instead
    // of stalling the stores at the end); the first barrier below publishes them
    __shared__ float row_as[S::BM];
    __shared__ int8_t row_ok[S::BM];
    if (!ISUMS && apart == 0) {
        const bool ok = arow >= 0 && arow < R;
        row_as[arow_l] = ok ? a_scale[arow] : 0.0f;
        row_ok[arow_l] = ok ? 1 : 0;
    }
    if (arow < 0 || arow >= R) arow = 0;
    const v4u *aglob = reinterpret_cast<const v4u *>(qa + arow * K + apart * S::A_BYTES);
    const int bcol_l = tid / S::B_TPC, bpart = tid % S::B_TPC;
    const int64_t bcol = (n0 + bcol_l < N) ? n0 + bcol_l : 0;
    const v4u *bglob = reinterpret_cast<const v4u *>(wpk + bcol * (K / 2) + bpart * S::B_PACKED);
    const uint16_t *zglob = wzp + bcol;

    // ---- compute state
    const int frow = lane & 31, fk = (lane >> 5) * 16;
    int64_t scol[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) scol[j] = n0 + wn * 64 + j * 32 + (lane & 31);
    const uint16_t *sglob[2] = {wsc + (scol[0] < N ? scol[0] : 0), wsc + (scol[1] < N ? scol[1] : 0)};

    // two register slots of prefetched group data (activation bytes, packed weights,
    // zero point, the two scales of this lane's columns)
    struct Slot {
        v4u ra[NA], rb[NB];
        uint16_t rz, rs[2][NSUB];
    };
    Slot sa, sb;
    // the 64-group (of the two in a stage) that this thread's packed bytes fall in
    const int zsub = GS == 64 ? (bpart * 2 * S::B_PACKED) / 64 : 0;
    auto gload = [&](Slot &sl, int64_t g) {
#pragma unroll
        for (int i = 0; i < NA; ++i) sl.ra[i] = aglob[g * (G128 / 16) + i];
#pragma unroll
        for (int i = 0; i < NB; ++i) sl.rb[i] = __builtin_nontemporal_load(bglob + g * (G128 / 2 / 16) + i);
        if constexpr (GS == 64) {
            sl.rz = zglob[(2 * g + zsub) * N];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                sl.rs[j][0] = ISUMS ? 0 : sglob[j][2 * g * N];
                sl.rs[j][1] = ISUMS ? 0 : sglob[j][(2 * g + 1) * N];
            }
        } else {
            const int64_t gg = GS == 256 ? g >> 1 : g;
            sl.rz = zglob[gg * N];
            sl.rs[0][0] = ISUMS ? 0 : sglob[0][gg * N];
            sl.rs[1][0] = ISUMS ? 0 : sglob[1][gg * N];
        }
    };
    auto lstore = [&](const Slot &sl, int buf) {
        uint8_t *A = lds + buf * S::LDS_STAGE;
        uint8_t *B = A + S::LDS_A;
        v4u *ad = reinterpret_cast<v4u *>(A + arow_l * kLdsStride + apart * S::A_BYTES);
#pragma unroll
        for (int i = 0; i < NA; ++i) ad[i] = sl.ra[i];
        const uint32_t zadd = zp_add_const(sl.rz);
        v4u *bd = reinterpret_cast<v4u *>(B + bcol_l * kLdsStride + bpart * (2 * S::B_PACKED));
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const uint32_t d4[4] = {sl.rb[i].x, sl.rb[i].y, sl.rb[i].z, sl.rb[i].w};
            uint32_t w[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) unpack8(d4[k], zadd, w[2 * k], w[2 * k + 1]);
            bd[2 * i] = v4u{w[0], w[1], w[2], w[3]};
            bd[2 * i + 1] = v4u{w[4], w[5], w[6], w[7]};
        }
    };

    float acc[2][2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // the MFMAs of k steps [KS0, KS1) of one stage (4 steps = 16 MFMAs): 4 independent
    // accumulator chains, k-step outer; RESET starts the sums at zero
    auto mfma_group = [&](auto ks0c, auto ks1c, auto resetc, int buf, v16i (&d)[2][2]) {
        constexpr int KS0 = decltype(ks0c)::value, KS1 = decltype(ks1c)::value;
        const uint8_t *A = lds + buf * S::LDS_STAGE;
        const uint8_t *B = A + S::LDS_A;
        if constexpr (decltype(resetc)::value) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) d[i][j][r] = 0;
        }
#pragma unroll
        for (int ks = KS0; ks < KS1; ++ks) {
            v4i af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *reinterpret_cast<const v4i *>(A + (wm * 64 + i * 32 + frow) * kLdsStride + ks * 32 + fk);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bf[j] = *reinterpret_cast<const v4i *>(B + (wn * 64 + j * 32 + frow) * kLdsStride + ks * 32 + fk);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) d[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], d[i][j], 0, 0, 0);
        }
    };
    // fold one group's int32 sums into the fp32 accumulators (or store them)
    auto epilogue = [&](int64_t g, const v16i (&d)[2][2], const float (&sc)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    if (ISUMS) {
                        const int m = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                        if (m < rows.rows && scol[j] < N)
                            isums[(g * M_isums + rows.slot0 + m) * N + scol[j]] = d[i][j][r];
                    } else {
                        acc[i][j][r] = fmaf(sc[j], (float)d[i][j][r], acc[i][j][r]);
                    }
                }
    };

    // Per group g: issue the global loads of group g+2 into the free register slot,
    // run the 16 MFMAs of group g from LDS (4 independent accumulator chains) and its
    // fp32 epilogue, then write group g+1 (loaded one iteration earlier) into the idle
    // LDS buffer and pass one barrier.  Each global load thus has a whole iteration
    // of compute to arrive.  Unrolled by two so the slots stay in registers; indices
    // past the end re-load the last group, whose copies are never consumed.
    v16i d[2][2];
    float sc[NSUB][2];  // this lane's two columns' scales, per group of the stage
    auto load_scales = [&](const Slot &sl) {
#pragma unroll
        for (int h = 0; h < NSUB; ++h) {
            sc[h][0] = half_bits_to_float(sl.rs[0][h]);
            sc[h][1] = half_bits_to_float(sl.rs[1][h]);
        }
    };
    gload(sa, 0);
    __builtin_amdgcn_sched_barrier(0);
    gload(sb, G > 1 ? 1 : 0);
    __builtin_amdgcn_sched_barrier(0);
    lstore(sa, 0);
    load_scales(sa);
    __syncthreads();
    using I0 = std::integral_constant<int, 0>;
    using I2 = std::integral_constant<int, 2>;
    using I4 = std::integral_constant<int, 4>;
    using T = std::true_type;
    // PAR: parity of the stage index (known at compile time: the loop is unrolled by two)
    auto body = [&](auto parc, int64_t g, Slot &fill, const Slot &next) {
        constexpr int PAR = decltype(parc)::value;
        // compiler fences keep the prefetch where it is written (IR passes would
        // otherwise merge it into the other half of the unrolled loop)
        __asm__ volatile("" ::: "memory");
        gload(fill, g + 2 < G ? g + 2 : G - 1);
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (GS == 128) {
            mfma_group(I0{}, I4{}, T{}, PAR, d);
            epilogue(g, d, sc[0]);
        } else if constexpr (GS == 256) {
            // the two stages of a group add into the same sums; one epilogue per group
            mfma_group(I0{}, I4{}, std::integral_constant<bool, PAR == 0>{}, PAR, d);
            if constexpr (PAR == 1) epilogue(g >> 1, d, sc[0]);
        } else {
            mfma_group(I0{}, I2{}, T{}, PAR, d);
            epilogue(2 * g, d, sc[0]);
            mfma_group(I2{}, I4{}, T{}, PAR, d);
            epilogue(2 * g + 1, d, sc[1]);
        }
        __builtin_amdgcn_sched_barrier(0);
        lstore(next, PAR ^ 1);
        load_scales(next);
        // keep the scales as fp32 values: folding the fp16->fp32 conversion into the
        // epilogue (v_fma_mix_f32) measured slower than converting once per group
#pragma unroll
        for (int h = 0; h < NSUB; ++h) __asm__ volatile("" : "+v"(sc[h][0]), "+v"(sc[h][1]));
        __syncthreads();
    };
    int64_t g = 0;
    for (; g + 1 < G; g += 2) {
        body(I0{}, g, sa, sb);                                   // stage g from LDS; g+1 (slot b) -> LDS
        body(std::integral_constant<int, 1>{}, g + 1, sb, sa);   // stage g+1 from LDS; g+2 (slot a) -> LDS
    }
    if (g < G) body(I0{}, g, sa, sb);   // odd stage count (GS = 64 or 128): the last stage

    if (!ISUMS) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m < rows.rows && row_ok[m]) {
                    const int64_t slot = rows.slot0 + m;
                    const float as = row_as[m];
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        if (scol[j] < N) out[slot * ldo + scol[j]] = as * acc[i][j][r];
                }
            }
    }
}

// ------------------------------------------------------------------ tiled loop, three LDS stages
// The 256x128 workgroup tile for group 128 (large M, and experts with more than 128 slots).
// Same arithmetic and wave layout as tile2_unit (eight waves of 64x64, 2x2
// v_mfma_i32_32x32x32_i8 tiles, groups folded into fp32 in increasing g), different data flow:
//  * activations go straight from memory into LDS (buffer_load ... lds, 16 bytes per lane):
//    each load instruction fills 1 KB of LDS with 8 whole 128-byte rows of one group, so
//    the loads are whole lines and use no registers and no LDS write instructions;
//  * LDS rows are 128 bytes with the 16-byte chunks of row r XOR-swizzled by (r >> 1) & 7
//    (the rows of a fragment read fall in distinct banks without padding), which leaves room
//    for three stages: group g is read from stage g % 3 while the activations of group g + 2
//    stream into stage (g + 2) % 3 and the unpacked weights of group g + 1 are written into
//    stage (g + 1) % 3, so every load has two iterations to arrive;
//  * the packed weights come through registers (four threads per column, 16 bytes = 32
//    codes each) and are unpacked once per workgroup to INT8 (q - zp), one group ahead.
// One barrier per group.  Rows past the tile's last read row 0 and columns past N read
// column 0; neither is stored.  Offsets are 32-bit: R * K and N * K / 2 below 2^32.
constexpr int kT3BM = 256, kT3BN = 128;
constexpr int kT3FI = 2;                         // 32-row fragments per wave (see tile3_unit)
constexpr int kT3Threads = 64 * 16 / kT3FI;      // 512: two waves per SIMD
constexpr int kT3StageA = kT3BM * G128, kT3StageB = kT3BN * G128, kT3Stage = kT3StageA + kT3StageB;
constexpr int kT3Lds = 3 * kT3Stage;  // 147456 bytes

// LDS has 64 banks of 4 bytes: a 128-bit read serves 16 lanes per cycle, here 16 consecutive
// rows of one chunk.  Even and odd rows fall in the two halves of a 256-byte bank window, so
// XOR the chunk index by (row >> 1) & 7: the 8 even rows, and the 8 odd ones, each take 8
// distinct 16-byte slots.
__device__ __forceinline__ int t3_sw(int row, int chunk) { return row * G128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

// Workgroup barrier for the staged loop, with the waits stated here instead of a full
// release fence: this wave's LDS writes complete (lgkmcnt 0) and at most VM of its memory
// loads (the ones issued since the data behind this barrier) still outstanding.  A fence
// would also wait for the activation loads still streaming into a later stage, which defeats
// the prefetch.  The empty asm statements keep the compiler from moving LDS accesses across.
template <int VM>
__device__ __forceinline__ void stage_barrier() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(t3_waitcnt(VM, 0));
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// Epilogues of the three-stage unit besides the plain store (kEpiOut):
//  kEpiSilu  the MoE gate/up product with SiLU(gate) * up folded in.  The weight matrix has
//            2 * half rows (gate rows [0, half), up rows [half, 2 half)); tile n0 covers h
//            columns [n0, n0 + 64), and its 128 MFMA columns are ordered so that each wave's
//            two 32-column blocks are the gate and the up rows of the same 32 h columns: a lane
//            holds gate and up of one (row, column) pair.  The row's out line (stride ldo =
//            2 half) receives h in columns [0, half) and, at half + c / 16, the largest |h| of
//            h columns c .. c + 15 (the per-row maximum is then a maximum of maxima).
//            gate and up are the fp32 values the plain epilogue would store, and h comes from
//            the same silu_mul as the unfused kernel, so h is bit-identical to that path's.
//  kEpiCombine  the MoE down product of the shared expert (rows = tokens), with the weighted
//            combine folded in: out[t][n] = (sum_j w[t][j] * y[slot(t, j)][n], fused multiply-adds
//            in j order from 0) + v[t][n], the same operations in the same order as the
//            combine kernel, where v is this tile's own product (also stored at out as usual).
//            The tile's values go through LDS so that each thread combines whole float4 runs.
constexpr int kEpiOut = 0, kEpiSilu = 1, kEpiCombine = 2;

// FI: 32-row fragments per wave.  FI = 2: 8 waves of 64x64 (two per SIMD); FI = 4: 4 waves of
// 128x64, one per SIMD (each wave's MFMAs and fold then issue from one instruction stream).
template <bool ISUMS, int EPI = kEpiOut, int FI = 2>
__device__ __forceinline__ void tile3_unit(uint8_t *lds, const int8_t *__restrict__ qa,
                                           const float *__restrict__ a_scale, const int32_t *__restrict__ row_index,
                                           int64_t R, TileRows rows, int64_t K, const uint8_t *__restrict__ wpk,
                                           const uint16_t *__restrict__ wsc, const uint16_t *__restrict__ wzp,
                                           int64_t N, int64_t n0, float *__restrict__ out, int64_t ldo,
                                           int32_t *__restrict__ isums, int64_t M_isums, const T3Epi &ep = T3Epi{}) {
    static_assert(EPI == kEpiOut || !ISUMS, "the debug form stores int32 sums only");
    static_assert(FI == 2 || FI == 4, "fragments per wave");
    constexpr int NWAVE = 16 / FI, NT = 64 * NWAVE;  // waves and threads of the workgroup
    constexpr int LA = 32 / NWAVE;                  // 1 KB activation loads per wave and group
    constexpr int NB = 512 / NT;                    // weight pieces per thread and group
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t G = K / G128;
    auto clampg = [&](int64_t g) { return g < G ? g : G - 1; };
    // weight row of MFMA column c of the tile (-1: past the matrix)
    auto wrow = [&](int c) -> int64_t {
        if constexpr (EPI == kEpiSilu) {
            const int64_t hc = n0 + (c >> 6) * 32 + (c & 31);
            return hc < ep.half ? ((c & 32) ? ep.half + hc : hc) : -1;
        } else {
            return n0 + c < N ? n0 + c : -1;
        }
    };

    // row scales and validity of the tile's rows (published by the prologue's barriers)
    __shared__ float row_as[kT3BM];
    __shared__ int8_t row_ok[kT3BM];
    for (int t = tid; t < kT3BM; t += NT) {
        int64_t r = -1;
        if (t < rows.rows) r = row_index ? (int64_t)row_index[rows.slot0 + t] : rows.slot0 + t;
        const bool ok = r >= 0 && r < R;
        row_ok[t] = ok ? 1 : 0;
        if (!ISUMS) row_as[t] = ok ? a_scale[r] : 0.0f;
    }

    // ---- activation loads: load j (0..LA-1) of wave w fills LDS rows 8 (LA w + j) + [0, 8);
    // lane l brings row 8 (LA w + j) + (l >> 3), chunk (l & 7) of the swizzled layout
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(qa);
    uint32_t aoff[LA];
#pragma unroll
    for (int j = 0; j < LA; ++j) {
        const int rl = 8 * (LA * wave + j) + (lane >> 3);
        int64_t r = -1;
        if (rl < rows.rows) r = row_index ? (int64_t)row_index[rows.slot0 + rl] : rows.slot0 + rl;
        if (r < 0 || r >= R) r = 0;
        aoff[j] = (uint32_t)r * (uint32_t)K + (uint32_t)(((lane & 7) ^ ((rl >> 1) & 7)) << 4);
    }
    auto a_dma = [&](int st, int64_t g) {
        uint8_t *dst = lds + st * kT3Stage + 1024 * (LA * wave);
#pragma unroll
        for (int j = 0; j < LA; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(dst + 1024 * j), 16, (int)aoff[j],
                                                     (int)(g * G128), 0, 0);
    };

    // ---- packed weights: thread t takes column (t >> 2) + (NT / 4) q for q < NB, bytes
    // 16 (t & 3) + [0, 16) of a group, with that column's zero point; and this lane's two output
    // columns' scales
    const int bcol = tid >> 2, bpart = tid & 3;
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(wpk);
    const __amdgpu_buffer_rsrc_t rz = make_rsrc(wzp);
    const __amdgpu_buffer_rsrc_t rsc = make_rsrc(ISUMS ? wzp : wsc);  // (unused by the debug form)
    uint32_t boff[NB], zoff[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) {
        const int c = bcol + (NT / 4) * q;
        const int64_t gc = wrow(c) >= 0 ? wrow(c) : 0;
        boff[q] = (uint32_t)(gc * (K / 2)) + (uint32_t)(16 * bpart);
        zoff[q] = (uint32_t)(gc * 2);
    }
    int64_t scol[2];
    uint32_t soff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t wr = wrow(wn * 64 + j * 32 + (lane & 31));
        scol[j] = wr >= 0 ? wr : N;  // (kEpiOut / kEpiCombine: the output column)
        soff[j] = (uint32_t)((wr >= 0 ? wr : 0) * 2);
    }
    struct Slot {
        v4u rb[NB];
        uint32_t rz[NB], rs0, rs1;
    };
    auto b_load = [&](Slot &x, int64_t g) {
        const int gs = (int)(g * N * 2);
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            x.rb[q] = __builtin_amdgcn_raw_buffer_load_b128(rb, boff[q], (int)(g * (G128 / 2)), 0);
            x.rz[q] = __builtin_amdgcn_raw_buffer_load_b16(rz, zoff[q], gs, 0);
        }
        if constexpr (!ISUMS) {
            x.rs0 = __builtin_amdgcn_raw_buffer_load_b16(rsc, soff[0], gs, 0);
            x.rs1 = __builtin_amdgcn_raw_buffer_load_b16(rsc, soff[1], gs, 0);
        } else {
            x.rs0 = x.rs1 = 0;
        }
    };
    // loads per wave and group (the debug form reads no scales)
    constexpr int LPG = LA + 2 * NB + (ISUMS ? 0 : 2);
    auto b_store = [&](const Slot &x, int st) {
        uint8_t *B = lds + st * kT3Stage + kT3StageA;
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            const uint32_t zadd = zp_add_const((uint16_t)x.rz[q]);
            const uint32_t d4[4] = {x.rb[q].x, x.rb[q].y, x.rb[q].z, x.rb[q].w};
            uint32_t w[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) unpack8(d4[k], zadd, w[2 * k], w[2 * k + 1]);
            const int c = bcol + (NT / 4) * q;
            *reinterpret_cast<v4u *>(B + t3_sw(c, 2 * bpart)) = v4u{w[0], w[1], w[2], w[3]};
            *reinterpret_cast<v4u *>(B + t3_sw(c, 2 * bpart + 1)) = v4u{w[4], w[5], w[6], w[7]};
        }
    };

    // ---- compute: lane l feeds A row (l & 31) / B column (l & 31) of a 32x32 tile with the
    // 16 bytes of chunk 2 ks + (l >> 5); it holds accumulator rows 8 (r >> 2) + 4 (l >> 5) + (r & 3)
    // (rows i * 32 + frow of a fragment differ from row frow by a multiple of 16, so the second
    // fragment's address is the first one's plus an immediate 4096)
    const int frow = lane & 31, fch = lane >> 5;
    int aofs[4], bofs[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        aofs[ks] = t3_sw(wm * 32 * FI + frow, 2 * ks + fch);
        bofs[ks] = kT3StageA + t3_sw(wn * 64 + frow, 2 * ks + fch);
    }
    float acc[FI][2][16];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    float sc[2] = {0.0f, 0.0f}, scn[2];
    // Rolling fold (plain epilogue): the four 32x32 chains of a group run one after the
    // other, (0,0), (0,1), (1,0), (1,1), and each chain's 16 int32 sums are folded into fp32
    // while the next chain's four MFMAs execute, so the conversions and fused multiply-adds
    // issue between MFMAs instead of after them.  The last chain of group g is folded during
    // the first chain of group g + 1 (prev, with that group's scale).  Every element still
    // takes its groups in increasing g, one fmaf each: the same operations as the plain loop.
    v16i prev = {};
    float prev_sc = 0.0f;  // fmaf(0, 0, acc) == acc before the first group
    auto fold = [&](const v16i &dd, int i, int j, float s_) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = fmaf(s_, (float)dd[r], acc[i][j][r]);
    };
    auto chain = [&](const v4i *a, const v4i *b) {
        v16i dd = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[0], b[0], v16i{}, 0, 0, 0);
#pragma unroll
        for (int ks = 1; ks < 4; ++ks) dd = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[ks], b[ks], dd, 0, 0, 0);
        return dd;
    };
    auto interleave = [&]() {  // four MFMAs, each followed by eight VALU instructions
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        }
    };
    auto group_rolling = [&](int st) {
        const uint8_t *base = lds + st * kT3Stage;
        // every fragment of the group is requested up front (in the order the chains use them)
        v4i a[FI][4], b[2][4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            a[0][ks] = *reinterpret_cast<const v4i *>(base + aofs[ks]);
            b[0][ks] = *reinterpret_cast<const v4i *>(base + bofs[ks]);
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) b[1][ks] = *reinterpret_cast<const v4i *>(base + bofs[ks] + 4096);
#pragma unroll
        for (int i = 1; i < FI; ++i)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) a[i][ks] = *reinterpret_cast<const v4i *>(base + aofs[ks] + 4096 * i);
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * (FI + 2), 0);
        // chains (i, j) in order; each folds the one before it (the first, the last of the group before)
        v16i d = chain(a[0], b[0]);
        fold(prev, FI - 1, 1, prev_sc);
        interleave();
#pragma unroll
        for (int c = 1; c < 2 * FI; ++c) {
            const int i = c >> 1, j = c & 1;
            const v16i dn = chain(a[i], b[j]);
            fold(d, (c - 1) >> 1, (c - 1) & 1, sc[(c - 1) & 1]);
            interleave();
            d = dn;
        }
        prev = d;
        prev_sc = sc[1];
    };
    auto group = [&](int st, int64_t g) {
        const uint8_t *base = lds + st * kT3Stage;
        v16i d[FI][2];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            v4i af[FI], bf[2];
            const uint8_t *pa = base + aofs[ks], *pb = base + bofs[ks];
#pragma unroll
            for (int i = 0; i < FI; ++i) af[i] = *reinterpret_cast<const v4i *>(pa + 4096 * i);
#pragma unroll
            for (int j = 0; j < 2; ++j) bf[j] = *reinterpret_cast<const v4i *>(pb + 4096 * j);
#pragma unroll
            for (int i = 0; i < FI; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    d[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], ks ? d[i][j] : v16i{}, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    if (ISUMS) {
                        const int m = wm * 32 * FI + i * 32 + 8 * (r >> 2) + 4 * fch + (r & 3);
                        if (m < rows.rows && scol[j] < N)
                            isums[(g * M_isums + rows.slot0 + m) * N + scol[j]] = d[i][j][r];
                    } else {
                        acc[i][j][r] = fmaf(sc[j], (float)d[i][j][r], acc[i][j][r]);
                    }
                }
    };

    // ---- prologue: groups 0 and 1 in flight, group 0's weights unpacked into stage 0
    Slot sl[2];
    a_dma(0, 0);
    b_load(sl[0], 0);
    __builtin_amdgcn_sched_barrier(0);
    a_dma(1, clampg(1));
    b_load(sl[1], clampg(1));
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(t3_waitcnt(LPG, 15));  // group 0: all but group 1's loads
    b_store(sl[0], 0);
    scn[0] = half_bits_to_float((uint16_t)sl[0].rs0);
    scn[1] = half_bits_to_float((uint16_t)sl[0].rs1);
    stage_barrier<LPG>();

    // ---- main loop: iteration g computes group g from stage g % 3; register slot g & 1 held
    // group g's weights (unpacked last iteration) and now takes group g + 2's.  Unrolled by
    // two so the slots stay in registers.  Per iteration each wave issues 4 activation loads
    // of group g + 2 and then 4 weight, zero-point and scale loads (2, without the scales, in
    // the debug form); before group g + 1's weights are unpacked and the barrier passed, group
    // g + 1's activations (issued one iteration earlier, with LPG loads after them) are waited for.
    int st0 = 0, st1 = 1, st2 = 2;
    auto body = [&](auto parc, int64_t g) {
        constexpr int PAR = decltype(parc)::value;
        Slot &fill = sl[PAR];
        const Slot &next = sl[PAR ^ 1];
        sc[0] = scn[0];
        sc[1] = scn[1];
        __asm__ volatile("" ::: "memory");
        a_dma(st2, clampg(g + 2));
        __builtin_amdgcn_sched_barrier(0);
        b_load(fill, clampg(g + 2));
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (ISUMS) group(st0, g);
        else group_rolling(st0);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(t3_waitcnt(LPG, 15));
        b_store(next, st1);
        scn[0] = half_bits_to_float((uint16_t)next.rs0);
        scn[1] = half_bits_to_float((uint16_t)next.rs1);
#pragma unroll
        for (int h = 0; h < 2; ++h) __asm__ volatile("" : "+v"(scn[h]));
        stage_barrier<LPG>();
        const int t = st0;
        st0 = st1;
        st1 = st2;
        st2 = t;
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    int64_t g = 0;
    for (; g + 1 < G; g += 2) {
        body(I0{}, g);
        body(I1{}, g + 1);
    }
    if (g < G) body(I0{}, g);
    __builtin_amdgcn_s_waitcnt(0);  // the last (unused) prefetches
    if constexpr (!ISUMS) fold(prev, FI - 1, 1, prev_sc);  // the last group's last chain

    if constexpr (!ISUMS && EPI == kEpiOut) {
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = wm * 32 * FI + i * 32 + 8 * (r >> 2) + 4 * fch + (r & 3);
                if (m < rows.rows && row_ok[m]) {
                    const int64_t slot = rows.slot0 + m;
                    const float as = row_as[m];
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        if (scol[j] < N) out[slot * ldo + scol[j]] = as * acc[i][j][r];
                }
            }
    } else if constexpr (EPI == kEpiSilu) {
        const int64_t hc = n0 + wn * 32 + (lane & 31);  // this lane's h column
        const bool col_ok = hc < ep.half;
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = wm * 32 * FI + i * 32 + 8 * (r >> 2) + 4 * fch + (r & 3);
                const bool ok = m < rows.rows && row_ok[m];
                const float as = row_as[m];
                const float gate = as * acc[i][0][r], up = as * acc[i][1][r];
                const float h = silu_mul(gate, up);
                float hm = (ok && col_ok) ? fabsf(h) : 0.0f;
                // largest |h| over each 16-lane row (one tile row, 16 h columns): DPP steps,
                // no LDS traffic
                hm = dpp_max<0xB1>(hm);   // quad_perm [1,0,3,2]
                hm = dpp_max<0x4E>(hm);   // quad_perm [2,3,0,1]
                hm = dpp_max<0x124>(hm);  // row_ror:4
                hm = dpp_max<0x128>(hm);  // row_ror:8
                if (ok) {
                    float *line = out + (rows.slot0 + m) * ldo;
                    if (col_ok) line[hc] = h;
                    if ((lane & 15) == 0) line[ep.half + (n0 + wn * 32 + (lane & 16)) / 16] = hm;
                }
            }
    } else if constexpr (EPI == kEpiCombine) {
        // the tile's products -> LDS [256][128] fp32 (the stages are free once every wave is
        // past its last group), the rows' slots and weights after them
        __syncthreads();
        float *ct = reinterpret_cast<float *>(lds);
        int32_t *tsop = reinterpret_cast<int32_t *>(lds + kT3BM * kT3BN * 4);
        float *tw = reinterpret_cast<float *>(lds + kT3BM * kT3BN * 4 + kT3BM * 8 * 4);
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = wm * 32 * FI + i * 32 + 8 * (r >> 2) + 4 * fch + (r & 3);
                const float as = row_as[m];
#pragma unroll
                for (int j = 0; j < 2; ++j) ct[m * kT3BN + wn * 64 + j * 32 + (lane & 31)] = as * acc[i][j][r];
            }
        for (int idx = tid; idx < rows.rows * ep.k; idx += NT) {
            const int m = idx / ep.k, jj = idx - m * ep.k;
            const int64_t pr = (rows.slot0 + m) * ep.k + jj;
            tsop[m * 8 + jj] = ep.sop[pr];
            tw[m * 8 + jj] = ep.tw[pr];
        }
        __syncthreads();
        // thread: float4 column c4 of rows tid / 32 + 16 i; two rows at a time, all their
        // routed rows' loads issued before the multiply-adds (16 loads in flight per thread)
        const int c4 = tid & 31;
        const int64_t col = n0 + 4 * c4;
        if (col < N) {
            for (int mb = tid >> 5; mb < rows.rows; mb += 2 * (NT / 32)) {
                float4 v[2][8];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int m = mb + q * (NT / 32);
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj)
                        if (m < rows.rows && jj < ep.k)
                            v[q][jj] = *reinterpret_cast<const float4 *>(ep.y + (int64_t)tsop[m * 8 + jj] * N + col);
                }
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int m = mb + q * (NT / 32);
                    if (m >= rows.rows) continue;
                    const int64_t t = rows.slot0 + m;
                    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) {
                        if (jj < ep.k) {
                            const float wj = tw[m * 8 + jj];
                            o.x = fmaf(wj, v[q][jj].x, o.x);
                            o.y = fmaf(wj, v[q][jj].y, o.y);
                            o.z = fmaf(wj, v[q][jj].z, o.z);
                            o.w = fmaf(wj, v[q][jj].w, o.w);
                        }
                    }
                    const float4 sh = *reinterpret_cast<const float4 *>(ct + m * kT3BN + 4 * c4);
                    o.x += sh.x;
                    o.y += sh.y;
                    o.z += sh.z;
                    o.w += sh.w;
                    *reinterpret_cast<float4 *>(ep.fin + t * N + col) = o;
                    *reinterpret_cast<float4 *>(out + t * ldo + col) = sh;
                }
            }
        }
    }
}

template <bool ISUMS, int EPI = kEpiOut>
__global__ __launch_bounds__(kT3Threads) void gemm_tiled3_kernel(const int8_t *__restrict__ qa,
                                                                 const float *__restrict__ a_scale, int64_t M,
                                                                 int64_t K, const uint8_t *__restrict__ packed,
                                                                 const uint16_t *__restrict__ scale,
                                                                 const uint16_t *__restrict__ zp, int64_t N,
                                                                 float *__restrict__ out,
                                                                 int32_t *__restrict__ isums, T3Epi ep) {
    extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
    const int64_t mt = (M + kT3BM - 1) / kT3BM, nt = (N + kT3BN - 1) / kT3BN;
    int64_t tm, tn;
    panel_tile<4>(xcd_tile(blockIdx.x, mt * nt), mt, nt, tm, tn);
    const int64_t m0 = tm * kT3BM;
    const int rows = (int)((M - m0) < kT3BM ? (M - m0) : kT3BM);
    tile3_unit<ISUMS, EPI, kT3FI>(dsm, qa, a_scale, nullptr, M, TileRows{m0, rows}, K, packed, scale, zp, N, tn * kT3BN, out,
                           N, isums, M, ep);
}

// ------------------------------------------------------------------ tiled loop, 256x256 tiles
// The same arithmetic as tile3_unit (per-group int32 sums, folded into fp32 in increasing g with
// one fmaf per element and group) on a 256x256 workgroup tile: eight waves of 128x64, two per
// SIMD, and two LDS stages of 64 KB (the 256 activation rows and the 256 unpacked weight columns
// of one group, in the swizzled layout of t3_sw).  Per output element and group a wave reads 25%
// fewer fragment bytes from LDS than with 64x64 wave tiles, and the workgroup moves 40% fewer
// bytes through the vector memory path than with 256x128 tiles (one activation tile serves 256
// columns).
// Iteration g computes group g from stage g % 2; at its top the activations of group g + 1 are
// requested straight into the other stage (that stage was last read before the previous
// barrier).  The packed weights come through registers with two groups of lead: those of group
// g + 1, requested during iteration g - 1, are unpacked into the other stage a quarter at a time
// between the MFMA chains of the second half of iteration g, and group g + 2's are requested
// after them, so that no unpack work or LDS store waits in front of the barrier.
constexpr int kT4BM = 256, kT4BN = 256;
constexpr int kT4Threads = 512;
constexpr int kT4StageA = kT4BM * G128, kT4Stage = kT4StageA + kT4BN * G128;
constexpr int kT4Lds = 2 * kT4Stage;  // 131072 bytes

// Chains of v_mfma_i32_16x16x64_i8: a wave's 128x64 block is 8 x 4 chains of 16x16 outputs, two
// MFMAs (k steps of 64) per chain and group, so a chain's int32 sums take 4 registers (the
// 32x32x32 form needs 16 per chain, and then the packed weights do not fit beside them).
// During chains 16-31 a quarter of the next group's weights is unpacked every four chains.
// Step ks of a group: lane quarter qd = l >> 4 supplies codes 16 (4 ks + qd) + [0, 16) of its row
// (A: row (l & 15) of the row block) and of its column (B: column (l & 15) of the column block);
// accumulator register r of a chain holds row 4 qd + r, column l & 15.
// TM: the weights are the tile-major array (wpk; wsc and wzp unused): the same codes with each
// dword's nibbles already in code order (no byte permutes in the unpack), and each column's
// scales and -zp bytes of a group pair in the tile's 8-byte word.
template <bool ISUMS, int EPI = kEpiOut, bool TM = false>
__device__ __forceinline__ void tile4_unit(uint8_t *lds, const int8_t *__restrict__ qa,
                                           const float *__restrict__ a_scale, const int32_t *__restrict__ row_index,
                                           int64_t R, TileRows rows, int64_t K, const uint8_t *__restrict__ wpk,
                                           const uint16_t *__restrict__ wsc, const uint16_t *__restrict__ wzp,
                                           int64_t N, int64_t n0, float *__restrict__ out, int64_t ldo,
                                           int32_t *__restrict__ isums, int64_t M_isums, const T3Epi &ep = T3Epi{}) {
    static_assert(EPI == kEpiOut || EPI == kEpiSilu, "plain and SiLU epilogues");
    static_assert(EPI == kEpiOut || !ISUMS, "the debug form stores int32 sums only");
    static_assert(!TM || (EPI == kEpiOut && !ISUMS), "tile-major weights: plain epilogue");
    constexpr int NT = kT4Threads, LA = 4;
    constexpr int NBL = ISUMS ? 3 : 7;  // weight loads per thread and group (codes 2, zp 1, scales 4)
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int64_t G = K / G128;
    auto wrow = [&](int c) -> int64_t {
        if constexpr (EPI == kEpiSilu) {
            const int64_t hc = n0 + (c >> 6) * 32 + (c & 31);
            return hc < ep.half ? ((c & 32) ? ep.half + hc : hc) : -1;
        } else {
            return n0 + c < N ? n0 + c : -1;
        }
    };

    __shared__ float row_as[kT4BM];
    __shared__ int8_t row_ok[kT4BM];
    for (int t = tid; t < kT4BM; t += NT) {
        int64_t r = -1;
        if (t < rows.rows) r = row_index ? (int64_t)row_index[rows.slot0 + t] : rows.slot0 + t;
        const bool ok = r >= 0 && r < R;
        row_ok[t] = ok ? 1 : 0;
        if (!ISUMS) row_as[t] = ok ? a_scale[r] : 0.0f;
    }

    // ---- activation loads (as tile4_unit)
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(qa);
    uint32_t aoff[LA];
#pragma unroll
    for (int j = 0; j < LA; ++j) {
        const int rl = 8 * (LA * wave + j) + (lane >> 3);
        int64_t r = -1;
        if (rl < rows.rows) r = row_index ? (int64_t)row_index[rows.slot0 + rl] : rows.slot0 + rl;
        if (r < 0 || r >= R) r = 0;
        aoff[j] = (uint32_t)r * (uint32_t)K + (uint32_t)(((lane & 7) ^ ((rl >> 1) & 7)) << 4);
    }
    auto a_dma = [&](int st, int64_t g) {
        uint8_t *dst = lds + st * kT4Stage + 1024 * (LA * wave);
#pragma unroll
        for (int j = 0; j < LA; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(dst + 1024 * j), 16, (int)aoff[j],
                                                     (int)(g * G128), 0, 0);
    };

    // ---- packed weights (as tile4_unit: thread t unpacks column t >> 1, codes 64 (t & 1) + [0, 64));
    // this lane's four output columns' scales
    const int bcol = tid >> 1, bpart = tid & 1;
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(wpk);
    const __amdgpu_buffer_rsrc_t rz = make_rsrc(TM ? (const void *)wpk : (const void *)wzp);
    const __amdgpu_buffer_rsrc_t rsc = make_rsrc(TM ? (const void *)wpk : (const void *)(ISUMS ? wzp : wsc));
    // TM: the first block of column c's 16-column tile, tile-major offsets below 2^32
    auto tm_tile = [&](int64_t c) -> uint32_t { return (uint32_t)(c >> 4) * (uint32_t)(G / 2) * (uint32_t)kTmBlock; };
    uint32_t boff, zoff;
    {
        const int64_t gc = wrow(bcol) >= 0 ? wrow(bcol) : 0;
        if constexpr (TM) {
            boff = tm_tile(gc) + 16u * (uint32_t)(gc & 15) + 512u * (uint32_t)bpart;
            zoff = tm_tile(gc) + 2048u + 8u * (uint32_t)(gc & 15) + 4u;
        } else {
            boff = (uint32_t)(gc * (K / 2)) + (uint32_t)(32 * bpart);
            zoff = (uint32_t)(gc * 2);
        }
    }
    const int frow = lane & 15, qd = lane >> 4;
    uint32_t soff[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const int64_t wr = wrow(wn * 64 + 16 * cb + frow);
        const int64_t wc = wr >= 0 ? wr : 0;
        soff[cb] = TM ? tm_tile(wc) + 2048u + 8u * (uint32_t)(wc & 15) : (uint32_t)(wc * 2);
    }
    struct Slot {
        v4u rb0, rb1;
        uint32_t rz, rs[4];
    };
    auto b_load = [&](Slot &x, int64_t g) {
        if constexpr (TM) {  // window g / 2 of the tile, group g % 2 in it
            const int gw = (int)((g >> 1) * kTmBlock), h = (int)(g & 1);
            x.rb0 = __builtin_amdgcn_raw_buffer_load_b128(rb, boff, gw + 1024 * h, 0);
            x.rb1 = __builtin_amdgcn_raw_buffer_load_b128(rb, boff + 256, gw + 1024 * h, 0);
            x.rz = __builtin_amdgcn_raw_buffer_load_b8(rz, zoff, gw + h, 0);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) x.rs[cb] = __builtin_amdgcn_raw_buffer_load_b16(rsc, soff[cb], gw + 2 * h, 0);
            return;
        }
        const int gs = (int)(g * N * 2);
        x.rb0 = __builtin_amdgcn_raw_buffer_load_b128(rb, boff, (int)(g * (G128 / 2)), 0);
        x.rb1 = __builtin_amdgcn_raw_buffer_load_b128(rb, boff + 16, (int)(g * (G128 / 2)), 0);
        x.rz = __builtin_amdgcn_raw_buffer_load_b16(rz, zoff, gs, 0);
        if constexpr (!ISUMS) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) x.rs[cb] = __builtin_amdgcn_raw_buffer_load_b16(rsc, soff[cb], gs, 0);
        } else {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) x.rs[cb] = 0;
        }
    };
    // quarter q of the unpack: codes 16 q + [0, 16) of this thread's 64 into chunk 4 bpart + q
    auto b_part = [&](const Slot &x, int st, int q, uint32_t zadd) {
        uint8_t *B = lds + st * kT4Stage + kT4StageA;
        const uint32_t d0 = q == 0 ? x.rb0.x : (q == 1 ? x.rb0.z : (q == 2 ? x.rb1.x : x.rb1.z));
        const uint32_t d1 = q == 0 ? x.rb0.y : (q == 1 ? x.rb0.w : (q == 2 ? x.rb1.y : x.rb1.w));
        uint32_t w0, w1, w2, w3;
        if constexpr (TM) {  // nibbles already in code order: codes 0-3 low, 4-7 high
            w0 = ((d0 & 0x0F0F0F0Fu) + zadd) ^ 0x80808080u;
            w1 = (((d0 >> 4) & 0x0F0F0F0Fu) + zadd) ^ 0x80808080u;
            w2 = ((d1 & 0x0F0F0F0Fu) + zadd) ^ 0x80808080u;
            w3 = (((d1 >> 4) & 0x0F0F0F0Fu) + zadd) ^ 0x80808080u;
        } else {
            unpack8(d0, zadd, w0, w1);
            unpack8(d1, zadd, w2, w3);
        }
        *reinterpret_cast<v4u *>(B + t3_sw(bcol, 4 * bpart + q)) = v4u{w0, w1, w2, w3};
    };

    // ---- fragments: row block rb (16 rows) and column block cb (16 columns) are the first
    // block's addresses plus 2048 rb / 2048 cb (the swizzle repeats every 16 rows)
    int aofs[2], bofs[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        aofs[ks] = t3_sw(wm * 128 + frow, 4 * ks + qd);
        bofs[ks] = kT4StageA + t3_sw(wn * 64 + frow, 4 * ks + qd);
    }
    auto scol = [&](int cb) -> int64_t {
        const int64_t wr = wrow(wn * 64 + 16 * cb + frow);
        return wr >= 0 ? wr : N;
    };
    float acc[8][4][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;

    // Rolling consumption: chain c = 4 rb + cb runs while chain c - 1 is folded; the last chain of
    // a group is folded during the first chain of the next (every element takes its groups in
    // increasing g)
    v4i prev = {};
    float prev_sc = 0.0f;
    int64_t prev_g = -1;
    auto consume = [&](const v4i &dd, int rb, int cb, float s_, int64_t g) {
        if constexpr (ISUMS) {
            if (g < 0) return;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = wm * 128 + 16 * rb + 4 * qd + r;
                if (m < rows.rows && scol(cb) < N) isums[(g * M_isums + rows.slot0 + m) * N + scol(cb)] = dd[r];
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[rb][cb][r] = fmaf(s_, (float)dd[r], acc[rb][cb][r]);
        }
    };
    auto pin = [&](int rb, int cb) {
        if constexpr (!ISUMS) {
#pragma unroll
            for (int r = 0; r < 4; ++r) __asm__ volatile("" : "+v"(acc[rb][cb][r]));
        }
    };

    float sc[4] = {0.0f, 0.0f, 0.0f, 0.0f}, scn[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    Slot sl;
    uint32_t zadd = 0;
    // group g from stage st; during chains 16-31 the next group's weights (in sl) are unpacked into
    // stage st ^ 1 and group g2's requested
    auto group = [&](int st, int64_t g, int64_t g2) {
        const uint8_t *base = lds + st * kT4Stage;
        v4i b[4][2], a[2], an[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) a[ks] = *reinterpret_cast<const v4i *>(base + aofs[ks]);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) b[cb][ks] = *reinterpret_cast<const v4i *>(base + bofs[ks] + 2048 * cb);
        consume(prev, 7, 3, prev_sc, prev_g);
        __builtin_amdgcn_sched_group_barrier(0x100, 10, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        pin(7, 3);
        __builtin_amdgcn_sched_barrier(0);
        v4i d = {};
#pragma unroll
        for (int c = 0; c < 32; ++c) {
            const int rb = c >> 2, cb = c & 3;
            v4i dn = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[0], b[cb][0], v4i{0, 0, 0, 0}, 0, 0, 0);
            dn = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[1], b[cb][1], dn, 0, 0, 0);
            if (cb == 0 && rb < 7) {  // the next row block's fragments
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) an[ks] = *reinterpret_cast<const v4i *>(base + aofs[ks] + 2048 * (rb + 1));
            }
            if (c > 0) consume(d, (c - 1) >> 2, (c - 1) & 3, sc[(c - 1) & 3], g);
            const bool piece = c >= 16 && (c & 3) == 0;
            if (piece) {
                const int q = (c - 16) >> 2;
                if (q == 0) zadd = TM ? zp_add_const_neg(sl.rz) : zp_add_const((uint16_t)sl.rz);
                b_part(sl, st ^ 1, q, zadd);
                if (q == 3) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) scn[j] = half_bits_to_float((uint16_t)sl.rs[j]);
                    b_load(sl, g2);
                }
            }
            // both MFMAs of the chain first, then the previous chain's fold (measured 3-4% faster
            // than one MFMA, four fold instructions, the other MFMA, the other four)
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            if (cb == 0 && rb < 7) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            if (c > 0) __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
            if (piece) {
                __builtin_amdgcn_sched_group_barrier(0x002, 20, 0);
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                if (c == 28) {
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, NBL, 0);
                }
            }
            if (c > 0) pin((c - 1) >> 2, (c - 1) & 3);
            __builtin_amdgcn_sched_barrier(0);
            d = dn;
            if (cb == 3 && rb < 7) {
                a[0] = an[0];
                a[1] = an[1];
            }
        }
        prev = d;
        prev_sc = sc[3];
        prev_g = g;
    };

    // ---- prologue: group 0 into stage 0; group 1's weights requested
    a_dma(0, 0);
    b_load(sl, 0);
    __builtin_amdgcn_s_waitcnt(t3_waitcnt(0, 15));
    {
        const uint32_t z0 = TM ? zp_add_const_neg(sl.rz) : zp_add_const((uint16_t)sl.rz);
#pragma unroll
        for (int q = 0; q < 4; ++q) b_part(sl, 0, q, z0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) scn[j] = half_bits_to_float((uint16_t)sl.rs[j]);
    b_load(sl, G > 1 ? 1 : 0);
    stage_barrier<NBL>();

    // ---- main loop, unrolled by two so that the stage index is a constant; past the last group
    // the loads repeat group G - 1 into a stage no longer read (the waits stay the same)
    auto body = [&](auto stc, int64_t g) {
        constexpr int ST = decltype(stc)::value;
        const int64_t g1 = g + 1 < G ? g + 1 : G - 1, g2 = g + 2 < G ? g + 2 : G - 1;
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[j] = scn[j];
        __asm__ volatile("" ::: "memory");
        a_dma(ST ^ 1, g1);
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        group(ST, g, g2);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j) __asm__ volatile("" : "+v"(scn[j]));
        stage_barrier<NBL>();  // group g + 1 is in its stage; g + 2's weights may still be in flight
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    int64_t g = 0;
    for (; g + 1 < G; g += 2) {
        body(I0{}, g);
        body(I1{}, g + 1);
    }
    if (g < G) body(I0{}, g);
    __builtin_amdgcn_s_waitcnt(0);  // the last (unused) weight loads
    consume(prev, 7, 3, prev_sc, prev_g);

    if constexpr (!ISUMS && EPI == kEpiOut) {
#pragma unroll
        for (int rbk = 0; rbk < 8; ++rbk)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = wm * 128 + 16 * rbk + 4 * qd + r;
                if (m < rows.rows && row_ok[m]) {
                    const int64_t slot = rows.slot0 + m;
                    const float as = row_as[m];
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb)
                        if (scol(cb) < N) out[slot * ldo + scol(cb)] = as * acc[rbk][cb][r];
                }
            }
    } else if constexpr (EPI == kEpiSilu) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const int64_t hc = n0 + wn * 32 + 16 * hb + frow;  // this lane's h column
            const bool col_ok = hc < ep.half;
#pragma unroll
            for (int rbk = 0; rbk < 8; ++rbk)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = wm * 128 + 16 * rbk + 4 * qd + r;
                    const bool ok = m < rows.rows && row_ok[m];
                    const float as = row_as[m];
                    const float gate = as * acc[rbk][hb][r], up = as * acc[rbk][hb + 2][r];
                    const float hv = silu_mul(gate, up);
                    float hm = (ok && col_ok) ? fabsf(hv) : 0.0f;
                    hm = dpp_max<0xB1>(hm);   // quad_perm [1,0,3,2]
                    hm = dpp_max<0x4E>(hm);   // quad_perm [2,3,0,1]
                    hm = dpp_max<0x124>(hm);  // row_ror:4
                    hm = dpp_max<0x128>(hm);  // row_ror:8
                    if (ok) {
                        float *line = out + (rows.slot0 + m) * ldo;
                        if (col_ok) line[hc] = hv;
                        if (frow == 0) line[ep.half + (n0 + wn * 32 + 16 * hb) / 16] = hm;
                    }
                }
        }
    }
}

template <bool ISUMS, int EPI = kEpiOut, bool TM = false>
__global__ __launch_bounds__(kT4Threads) void gemm_tiled4_kernel(const int8_t *__restrict__ qa,
                                                                 const float *__restrict__ a_scale, int64_t M,
                                                                 int64_t K, const uint8_t *__restrict__ packed,
                                                                 const uint16_t *__restrict__ scale,
                                                                 const uint16_t *__restrict__ zp, int64_t N,
                                                                 float *__restrict__ out,
                                                                 int32_t *__restrict__ isums) {
    extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
    const int64_t mt = (M + kT4BM - 1) / kT4BM, nt = (N + kT4BN - 1) / kT4BN;
    int64_t tm, tn;
    panel_tile<4>(xcd_tile(blockIdx.x, mt * nt), mt, nt, tm, tn);
    const int64_t m0 = tm * kT4BM;
    const int rows = (int)((M - m0) < kT4BM ? (M - m0) : kT4BM);
    tile4_unit<ISUMS, EPI, TM>(dsm, qa, a_scale, nullptr, M, TileRows{m0, rows}, K, packed, scale, zp, N, tn * kT4BN,
                               out, N, isums, M);
}

template <int WM, int WN, bool ISUMS, int GS>
__global__ __launch_bounds__(64 * WM * WN) void gemm_tiled_kernel(const int8_t *__restrict__ qa,
                                                                  const float *__restrict__ a_scale, int64_t M,
                                                                  int64_t K, const uint8_t *__restrict__ packed,
                                                                  const uint16_t *__restrict__ scale,
                                                                  const uint16_t *__restrict__ zp, int64_t N,
                                                                  float *__restrict__ out,
                                                                  int32_t *__restrict__ isums) {
    using S = TileShape<WM, WN>;
    extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
    const int64_t mt = (M + S::BM - 1) / S::BM, nt = (N + S::BN - 1) / S::BN;
    int64_t tm, tn;
    panel_tile<4>(xcd_tile(blockIdx.x, mt * nt), mt, nt, tm, tn);
    const int64_t m0 = tm * S::BM;
    const int rows = (int)((M - m0) < S::BM ? (M - m0) : S::BM);
    tile2_unit<WM, WN, ISUMS, GS>(dsm, qa, a_scale, nullptr, M, TileRows{m0, rows}, K, packed, scale, zp, N,
                                  tn * S::BN, out, N, isums, M);
}

// ------------------------------------------------------------------ expert-grouped forms
// Each expert takes the loop for its slot count (the launcher picks the classes):
// the decode loop up to 16 slots, the weight-streaming loop for 17..128, the tiled
// loop above; when the group count rules the first two out, the streaming loop up to
// kSmallRows slots and the tiled loop above.  Each workgroup reads expert_offsets
// itself and walks a persistent unit list, so the slot counts never travel to the
// host.
constexpr int kSmallRows = 64;
constexpr int kMaxExperts = 1024;
// slot-count class of the weight-streaming loop: (kMidMin, kMidMax], 64-row blocks
// of 256 columns as work units
constexpr int kMidMin = 16, kMidMax = 128, kMidRows = 64;

// Exclusive prefix over experts of units(e) into lds_pfx[0..E]; returns the
// total.  Run by the whole workgroup (nthreads = blockDim.x <= 1024): thread t
// sums a contiguous run of experts, the runs are scanned with wave shuffles and
// one LDS step, then each thread writes its run's prefixes.
template <typename UnitsFn>
__device__ __forceinline__ int64_t expert_prefix(int32_t E, int64_t *lds_pfx, int nthreads, UnitsFn units) {
    __shared__ int64_t wave_tot[16];
    const int t = threadIdx.x;
    const int chunk = (E + nthreads - 1) / nthreads;
    const int e0 = t * chunk;
    const int e1 = (e0 + chunk < E) ? e0 + chunk : E;
    int64_t local = 0;
    for (int e = e0; e < e1; ++e) local += units(e);
    // inclusive wave scan
    const int lane = t & 63, wave = t >> 6;
    int64_t v = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    if (lane == 63) wave_tot[wave] = v;
    __syncthreads();
    int64_t base = 0;
    for (int w = 0; w < wave; ++w) base += wave_tot[w];
    int64_t run = base + v - local;  // exclusive prefix of this thread's run
    for (int e = e0; e < e1; ++e) {
        lds_pfx[e] = run;
        run += units(e);
    }
    if (t == nthreads - 1) lds_pfx[E] = base + v;
    __syncthreads();
    return lds_pfx[E];
}

__device__ __forceinline__ int find_expert(const int64_t *pfx, int32_t E, int64_t u) {
    int lo = 0, hi = E - 1;  // largest e with pfx[e] <= u
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pfx[mid] <= u) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ int64_t clamp_slots(int64_t v, int64_t max_slots) {
    return v < 0 ? 0 : (v > max_slots ? max_slots : v);
}

// Work units of the weight-streaming loop's slot class.  When they are too few for the
// machine (a lone mid-size expert, say), that loop would leave most CUs idle; the
// decode loop then takes those experts in 16-row chunks instead.  Both
// kernels compute this from the device-side offsets, so they agree without the host.
// Uses lds_pfx as scratch (as expert_prefix does).
__device__ __forceinline__ int64_t mid_class_units(int32_t E, int64_t *lds_pfx, int nthreads,
                                                   const int32_t *__restrict__ offsets, int64_t max_slots,
                                                   int64_t N) {
    const int64_t nblk = (N + 255) / 256;
    const int64_t total = expert_prefix(E, lds_pfx, nthreads, [&](int e) -> int64_t {
        const int64_t c = clamp_slots(offsets[e + 1], max_slots) - clamp_slots(offsets[e], max_slots);
        return (c > kMidMin && c <= kMidMax) ? ((c + kMidRows - 1) / kMidRows) * nblk : 0;
    });
    __syncthreads();  // every thread has read the total before lds_pfx is reused
    return total;
}

// ISUMS (test aid, in every expert loop): the per-group int32 sums of each slot go to
// isums[g][slot][n] (g < K/GS, slot < max_slots) instead of the fp32 output, and no
// scale is read; slots whose row index is outside [0, R) get unspecified sums.
template <int U, bool ISUMS>
__global__ __launch_bounds__(kStreamThreads) void grouped_stream_kernel(
    const int8_t *__restrict__ qa, const float *__restrict__ a_scale, int64_t R, const int32_t *__restrict__ row_index,
    const int32_t *__restrict__ offsets, int32_t E, int64_t K, const uint8_t *__restrict__ packed,
    const uint16_t *__restrict__ scale, const uint16_t *__restrict__ zp, int64_t N, int64_t max_slots,
    float *__restrict__ out, int32_t *__restrict__ isums) {
    __shared__ int64_t pfx[kMaxExperts + 1];
    const int64_t ntn = N / 16;
    const int64_t total = expert_prefix(E, pfx, kStreamThreads, [&](int e) -> int64_t {
        const int64_t c = clamp_slots(offsets[e + 1], max_slots) - clamp_slots(offsets[e], max_slots);
        return (c > 0 && c <= kSmallRows) ? ntn : 0;
    });
    const int64_t G = K / G128;
    constexpr int U2 = U < 4 ? U : 4, U4 = U < 2 ? U : 2;
    for (int64_t u = blockIdx.x; u < total; u += gridDim.x) {
        const int e = find_expert(pfx, E, u);
        const int64_t tn = u - pfx[e];
        const int64_t s0 = clamp_slots(offsets[e], max_slots);
        const int rows = (int)(clamp_slots(offsets[e + 1], max_slots) - s0);
        const uint8_t *wp = packed + (int64_t)e * N * (K / 2);
        const uint16_t *ws = scale + (int64_t)e * G * N;
        const uint16_t *wz = zp + (int64_t)e * G * N;
        const StreamRows sr{s0, rows};
        if (rows <= 16)
            stream_unit<1, U, ISUMS>(qa, a_scale, row_index, R, sr, K, wp, ws, wz, N, tn * 16, out, N, isums,
                                     max_slots);
        else if (rows <= 32)
            stream_unit<2, U2, ISUMS>(qa, a_scale, row_index, R, sr, K, wp, ws, wz, N, tn * 16, out, N, isums,
                                      max_slots);
        else
            stream_unit<4, U4, ISUMS>(qa, a_scale, row_index, R, sr, K, wp, ws, wz, N, tn * 16, out, N, isums,
                                      max_slots);
    }
}

// Experts with at most small_max slots, decode style: one 1024-thread workgroup
// per CU stages 16 gathered activation rows of one expert in LDS and streams
// 16-column tiles of that expert's weights (the loop of the dense decode kernel).
// Work units are (expert, 16-row chunk, tile); each workgroup takes a contiguous
// range of units, so it restages rows only when the chunk changes, and its tiles of
// one chunk run as one stream.  Each tile is split over SPLIT K parts: four when no
// workgroup can get more than four tiles (so that all 16 waves stream), else two.
template <int U, int SPLIT, bool ISUMS, int GS = G128>
__global__ __launch_bounds__(kDecThreads) void grouped_decode_kernel(
    const int8_t *__restrict__ qa, const float *__restrict__ a_scale, int64_t R, const int32_t *__restrict__ row_index,
    const int32_t *__restrict__ offsets, int32_t E, int64_t K, const uint8_t *__restrict__ packed,
    const uint16_t *__restrict__ scale, const uint16_t *__restrict__ zp, int64_t N, int64_t max_slots,
    float *__restrict__ out, int32_t *__restrict__ isums, int small_max, int64_t mid_floor) {
    extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
    __shared__ int64_t pfx[kMaxExperts + 1];
    __shared__ int32_t srow[16];
    __shared__ float sasc[16];  // row scales of the staged rows (no global load at the stores)
    const int64_t ntiles = N / 16;
    // also the weight-streaming loop's experts when that loop has too few units
    // (mid_floor > 0: it is launched too, and skips them then)
    const int small_eff =
        (mid_floor > 0 && mid_class_units(E, pfx, kDecThreads, offsets, max_slots, N) < mid_floor) ? kMidMax
                                                                                                    : small_max;
    const int64_t total = expert_prefix(E, pfx, kDecThreads, [&](int e) -> int64_t {
        const int64_t c = clamp_slots(offsets[e + 1], max_slots) - clamp_slots(offsets[e], max_slots);
        return (c > 0 && c <= small_eff) ? ((c + 15) / 16) * ntiles : 0;
    });
    const int64_t lda = K + 16;
    float *red = reinterpret_cast<float *>(dsm + ((dec_lds_bytes(16, K) + 15) / 16) * 16);
    // Contiguous unit ranges of one length, rounded up to whole rounds of the 16 waves
    // (16 / SPLIT tiles), when at least 7/8 of the workgroups still get units: every
    // wave streams, as in the dense decode launch (an even split would leave some
    // workgroups a tile short of a round); else the even split.
    int64_t u0, u1;
    {
        const int64_t nb = gridDim.x, per_round = kDecWaves / SPLIT;
        const int64_t span = (total + nb - 1) / nb;
        const int64_t up = (span + per_round - 1) / per_round * per_round;
        if (span > 0 && 8 * ((total + up - 1) / up) >= 7 * nb) {
            u0 = (int64_t)blockIdx.x * up < total ? (int64_t)blockIdx.x * up : total;
            u1 = u0 + up < total ? u0 + up : total;
        } else {
            u0 = total * blockIdx.x / nb;
            u1 = total * (blockIdx.x + 1) / nb;
        }
    }
    int staged_e = -1;
    int64_t staged_chunk = -1;
    for (int64_t u = u0; u < u1;) {
        const int e = find_expert(pfx, E, u);
        const int64_t local = u - pfx[e];
        const int64_t chunk = local / ntiles, t0 = local % ntiles;
        const int64_t t1 = (t0 + (u1 - u) < ntiles) ? t0 + (u1 - u) : ntiles;
        u += t1 - t0;
        const int64_t c = clamp_slots(offsets[e + 1], max_slots) - clamp_slots(offsets[e], max_slots);
        const int64_t s0 = clamp_slots(offsets[e], max_slots) + chunk * 16;
        const int rows = (int)((c - chunk * 16) < 16 ? (c - chunk * 16) : 16);
        const bool restage = e != staged_e || chunk != staged_chunk;
        if (restage) {
            __syncthreads();  // every wave is done with the previous rows
            staged_e = e;
            staged_chunk = chunk;
        }
        const uint8_t *wpk = packed + (int64_t)e * N * (K / 2);
        const uint16_t *wsc = scale + (int64_t)e * (K / GS) * N, *wzp = zp + (int64_t)e * (K / GS) * N;
        // This chunk's row indices are requested in stage(0), before the first weight windows,
        // by every thread (thread t reads slot s0 + min(t % 16, rows - 1): one uniform load, no
        // branch), so that waiting for them later waits for none of the weight loads (the
        // memory counter retires loads in order).  Only the expert's offsets then stand
        // between the launch and the first weight load.
        int32_t ridx = 0;
        auto stage = [&](int phase) {  // the chunk's activation rows -> LDS (only when they
                                       // changed); rows outside [0, R) read row 0 and are
                                       // never stored.  The row scales load alongside.
            if (!restage) return;
            if (phase == 0) {
                const int tr = (int)(threadIdx.x & 15) < rows ? (int)(threadIdx.x & 15) : rows - 1;
                // (an always-valid address when there is no row index: no branch around the load)
                const int32_t *src = row_index ? row_index + s0 + tr : offsets;
                const int32_t v = *src;
                ridx = row_index ? v : (int32_t)(s0 + tr);
                return;
            }
            if (threadIdx.x < 16) {
                const bool ok = (int)threadIdx.x < rows && ridx >= 0 && (int64_t)ridx < R;
                srow[threadIdx.x] = ok ? ridx : -1;
            }
            __syncthreads();
            stage_rows_dma(dsm, lda, qa, K, rows, [&](int r) { return (int64_t)(srow[r] >= 0 ? srow[r] : 0); });
            float asc = 0.0f;
            if (!ISUMS && threadIdx.x < 16) {
                const int32_t row = srow[threadIdx.x];
                asc = a_scale[row >= 0 ? row : 0];
            }
            __builtin_amdgcn_s_waitcnt(0);
            if (threadIdx.x < 16) sasc[threadIdx.x] = srow[threadIdx.x] >= 0 ? asc : 0.0f;
        };
        auto store = [&](int m, int64_t col, float v) {
            if (srow[m] >= 0) out[(s0 + m) * N + col] = sasc[m] * v;
        };
        dec_tiles<U, SPLIT, ISUMS, false, GS>(
            dsm, red, rows, K, wpk, wsc, wzp, N, t0, t1, stage, store,
            [&](int64_t g, int m, int64_t col, int32_t v) {
                if (srow[m] >= 0) isums[(g * max_slots + s0 + m) * N + col] = v;
            });
    }
}

// Experts with a middle number of slots (cmin, cmax]: one weight pass per block of
// 32 * MF of their rows with full-rate 32x32x32 INT8 MFMAs.  A work unit is (expert,
// row block, block of 256 columns); a 512-thread workgroup takes a contiguous range of
// units, and wave w owns the 32 columns [256 b + 32 w, +32) of the unit for all its
// rows and all K.
//
// Weights go straight from memory to registers: lane l holds column l % 32 and, per
// group, the packed bytes [32 h, 32 h + 32) (h = l / 32), i.e. codes 64 h + [0, 64) of
// the group.  MFMA step s of the group takes the 16 codes 64 h + 16 s + [0, 16); each
// packed dword splits into its low nibbles (codes 0 2 4 6) and high nibbles (1 3 5 7)
// with two operations, so operand byte order within every 8 codes is 0 2 4 6 1 3 5 7.
// The activation rows are staged in LDS with the same byte order (one v_perm per four
// bytes, once per workgroup instead of once per wave), so both operands agree.
//
// Activations are staged in K slices of kMidSlice groups (all rows of the unit,
// double-buffered, issued one slice ahead through registers); the slice sequence runs
// on from one unit into the next, and so does each wave's ring of U groups of
// weights, so a workgroup streams without draining between units.
constexpr int kMidThreads = 512;
constexpr int kMidSlice = 4;                       // groups per activation slice
constexpr int kMidRow = kMidSlice * G128 + 16;     // LDS bytes per staged row and slice
__host__ __device__ inline int64_t mid_lds_bytes(int mf) { return 2ll * 32 * mf * kMidRow; }

template <int MF, int U, bool ISUMS>
__global__ __launch_bounds__(kMidThreads) void grouped_mid_kernel(
    const int8_t *__restrict__ qa, const float *__restrict__ a_scale, int64_t R, const int32_t *__restrict__ row_index,
    const int32_t *__restrict__ offsets, int32_t E, int64_t K, const uint8_t *__restrict__ packed,
    const uint16_t *__restrict__ scale, const uint16_t *__restrict__ zp, int64_t N, int64_t max_slots,
    float *__restrict__ out, int32_t *__restrict__ isums, int64_t cmin, int64_t cmax, int64_t mid_floor) {
    constexpr int RM = 32 * MF;                    // staged rows
    constexpr int BUF = RM * kMidRow;
    constexpr int TPR = kMidThreads / RM;          // staging threads per row
    constexpr int NV = kMidSlice * G128 / TPR / 16; // 16-byte pieces per thread and slice
    static_assert(kMidSlice % U == 0, "ring slots must repeat within a slice");
    extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
    __shared__ int64_t pfx[kMaxExperts + 1];
    __shared__ float sasc[2][RM];                  // row scale per unit parity; -1: no store
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5;
    const int64_t G = K / G128;
    const int nsl = (int)(G / kMidSlice);
    const int64_t nblk = (N + 255) / 256;
    const int64_t total = expert_prefix(E, pfx, kMidThreads, [&](int e) -> int64_t {
        const int64_t c = clamp_slots(offsets[e + 1], max_slots) - clamp_slots(offsets[e], max_slots);
        return (c > cmin && c <= cmax) ? ((c + RM - 1) / RM) * nblk : 0;
    });
    // too few units for the machine: the decode loop has taken these experts (the same
    // count as mid_class_units when cmin, cmax, RM are the class bounds)
    if (total < mid_floor) return;
    const int64_t u0 = total * blockIdx.x / gridDim.x, u1 = total * (blockIdx.x + 1) / gridDim.x;
    if (u0 >= u1) return;  // the whole workgroup

    struct Unit {
        int e;
        int64_t s0, c;                 // slot base, slots
        bool store;                    // this lane's column is inside [0, N)
        int64_t col;                   // this lane's column (clamped into [0, N))
        __amdgpu_buffer_rsrc_t rw, rs, rz;  // the expert's codes, scales, zero points
        uint32_t vw, vs;               // this lane's byte offsets in them (group 0)
    };
    auto unit_of = [&](int64_t u) {
        Unit x;
        x.e = find_expert(pfx, E, u);
        const int64_t local = u - pfx[x.e];
        const int64_t rb = local / nblk, b = local % nblk;  // row block, column block
        const int64_t e0 = clamp_slots(offsets[x.e], max_slots);
        x.s0 = e0 + rb * RM;
        const int64_t left = clamp_slots(offsets[x.e + 1], max_slots) - x.s0;
        x.c = left < RM ? left : RM;
        const int64_t col = b * 256 + wave * 32 + (lane & 31);
        x.store = col < N;
        x.col = col < N ? col : N - 1;
        x.rw = make_rsrc(packed + (int64_t)x.e * N * (K / 2));
        x.rs = make_rsrc((ISUMS ? zp : scale) + (int64_t)x.e * G * N);  // (unused by the debug form)
        x.rz = make_rsrc(zp + (int64_t)x.e * G * N);
        x.vw = (uint32_t)(x.col * (K / 2) + 32 * h);
        x.vs = (uint32_t)(x.col * 2);
        return x;
    };
    // activation row of slot row r of a unit (rows past the expert read row 0: never stored)
    auto qa_row = [&](const Unit &x, int r) -> int64_t {
        if (r >= x.c) return 0;
        const int64_t q = row_index ? (int64_t)row_index[x.s0 + r] : x.s0 + r;
        return (q >= 0 && q < R) ? q : 0;
    };
    auto row_scale = [&](const Unit &x, int r) -> float {
        if (r >= x.c) return -1.0f;
        const int64_t q = row_index ? (int64_t)row_index[x.s0 + r] : x.s0 + r;
        if constexpr (ISUMS) return (q >= 0 && q < R) ? 1.0f : -1.0f;
        return (q >= 0 && q < R) ? a_scale[q] : -1.0f;
    };

    // ---- activation staging: thread -> (row srow_t, bytes [spart * 16 NV, +16 NV) of a
    // slice); offsets stay below 2^32 (R * K < 2^32 is required)
    const int srow_t = tid / TPR, spart = tid % TPR;
    const __amdgpu_buffer_rsrc_t rqa = make_rsrc(qa);
    v4u st[NV];
    auto load_slice = [&](int64_t qrow, int j) {
        const uint32_t vo = (uint32_t)(qrow * K) + spart * (16 * NV);
#pragma unroll
        for (int i = 0; i < NV; ++i)
            st[i] = __builtin_amdgcn_raw_buffer_load_b128(rqa, vo + 16 * i, j * (kMidSlice * G128), 0);
    };
    auto store_slice = [&](int b) {
        v4u *dst = reinterpret_cast<v4u *>(dsm + b * BUF + srow_t * kMidRow + spart * (16 * NV));
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const v4u v = st[i];
            dst[i] = v4u{__builtin_amdgcn_perm(v.y, v.x, 0x06040200u), __builtin_amdgcn_perm(v.y, v.x, 0x07050301u),
                         __builtin_amdgcn_perm(v.w, v.z, 0x06040200u), __builtin_amdgcn_perm(v.w, v.z, 0x07050301u)};
        }
    };

    // ---- weight ring: U groups in flight per wave (cached loads: the other half of each
    // 128-byte line, the next group, is read a few groups later from L2)
    v4u rw0[U], rw1[U];
    uint16_t rs[U] = {}, rz[U];  // (rs stays zero in the debug form)
    auto load_group = [&](int slot, const Unit &x, int64_t g) {
        const int gw = (int)(g * (G128 / 2)), gs2 = (int)(g * N * 2);
        rw0[slot] = __builtin_amdgcn_raw_buffer_load_b128(x.rw, x.vw, gw, 0);
        rw1[slot] = __builtin_amdgcn_raw_buffer_load_b128(x.rw, x.vw + 16, gw, 0);
        if constexpr (!ISUMS) rs[slot] = __builtin_amdgcn_raw_buffer_load_b16(x.rs, x.vs, gs2, 0);
        rz[slot] = __builtin_amdgcn_raw_buffer_load_b16(x.rz, x.vs, gs2, 0);
    };
    // the same without a branch between the two units (the memory-counter waits stay exact)
    auto load_group_sel = [&](int slot, bool here, const Unit &a, const Unit &b, int64_t ga, int64_t gb) {
        const int64_t g = here ? ga : gb;
        const int gw = (int)(g * (G128 / 2)), gs2 = (int)(g * N * 2);
        const __amdgpu_buffer_rsrc_t rw = here ? a.rw : b.rw, rsc = here ? a.rs : b.rs, rzp = here ? a.rz : b.rz;
        const uint32_t vw = here ? a.vw : b.vw, vs = here ? a.vs : b.vs;
        rw0[slot] = __builtin_amdgcn_raw_buffer_load_b128(rw, vw, gw, 0);
        rw1[slot] = __builtin_amdgcn_raw_buffer_load_b128(rw, vw + 16, gw, 0);
        if constexpr (!ISUMS) rs[slot] = __builtin_amdgcn_raw_buffer_load_b16(rsc, vs, gs2, 0);
        rz[slot] = __builtin_amdgcn_raw_buffer_load_b16(rzp, vs, gs2, 0);
    };

    int64_t u = u0;
    Unit cur = unit_of(u);
    int64_t qrow = qa_row(cur, srow_t);
    if (tid < RM) sasc[u & 1][tid] = row_scale(cur, tid);
#pragma unroll
    for (int i = 0; i < U; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        load_group(i, cur, i);
    }
    __builtin_amdgcn_sched_barrier(0);
    load_slice(qrow, 0);
    store_slice(0);
    __syncthreads();
    int q = 0;  // running slice counter: slice q reads buffer q & 1
    for (;;) {
        const bool more = u + 1 < u1;
        const Unit nxt = more ? unit_of(u + 1) : cur;
        const int64_t nqrow = more ? qa_row(nxt, srow_t) : qrow;
        const float nasc = (more && tid < RM) ? row_scale(nxt, tid) : 0.0f;
        // 32-row fragments that hold rows of this expert (wave-uniform)
        const int mt = cur.c > 32 * (MF - 1) ? MF : (int)((cur.c + 31) / 32);
        float acc[MF][16];
#pragma unroll
        for (int f = 0; f < MF; ++f)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[f][i] = 0.0f;
        for (int j = 0; j < nsl; ++j) {
            const bool last = j + 1 == nsl;
            const bool stage_next = !last || more;
            if (stage_next) load_slice(last ? nqrow : qrow, last ? 0 : j + 1);
            const uint8_t *abuf = dsm + (q & 1) * BUF + (lane & 31) * kMidRow + 64 * h;
#pragma unroll
            for (int gs = 0; gs < kMidSlice; ++gs) {
                const int slot = gs % U;
                const int64_t g = (int64_t)j * kMidSlice + gs;
                const uint32_t zadd = zp_add_const(rz[slot]);
                float sc = half_bits_to_float(rs[slot]);
                __asm__ volatile("" : "+v"(sc));
                const uint32_t d8[8] = {rw0[slot].x, rw0[slot].y, rw0[slot].z, rw0[slot].w,
                                        rw1[slot].x, rw1[slot].y, rw1[slot].z, rw1[slot].w};
                v16i dacc[MF];  // (the first step starts from an inline zero: no register clearing)
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const uint32_t a0 = d8[2 * s4], a1 = d8[2 * s4 + 1];
                    const v4i bq = {(int)(((a0 & 0x0F0F0F0Fu) + zadd) ^ 0x80808080u),
                                    (int)((((a0 >> 4) & 0x0F0F0F0Fu) + zadd) ^ 0x80808080u),
                                    (int)(((a1 & 0x0F0F0F0Fu) + zadd) ^ 0x80808080u),
                                    (int)((((a1 >> 4) & 0x0F0F0F0Fu) + zadd) ^ 0x80808080u)};
#pragma unroll
                    for (int f = 0; f < MF; ++f) {
                        if (f >= mt) break;
                        const v4i av = *reinterpret_cast<const v4i *>(abuf + f * 32 * kMidRow + gs * G128 + 16 * s4);
                        dacc[f] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bq, s4 ? dacc[f] : v16i{}, 0, 0, 0);
                    }
                }
#pragma unroll
                for (int f = 0; f < MF; ++f) {
                    if (f >= mt) break;
                    if constexpr (ISUMS) {
                        if (cur.store) {
#pragma unroll
                            for (int i = 0; i < 16; ++i) {
                                const int r = f * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
                                if (sasc[u & 1][r] >= 0.0f)
                                    isums[(g * max_slots + cur.s0 + r) * N + cur.col] = dacc[f][i];
                            }
                        }
                    } else {
#pragma unroll
                        for (int i = 0; i < 16; ++i) acc[f][i] = fmaf(sc, (float)dacc[f][i], acc[f][i]);
                    }
                }
                // refill: group g + U of this unit, else of the next one (the last unit
                // re-reads its own first groups, which nothing consumes)
                const int64_t ga = g + U;
                __builtin_amdgcn_sched_barrier(0);
                load_group_sel(slot, ga < G, cur, nxt, ga, ga - G);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (last && more && tid < RM) sasc[(u + 1) & 1][tid] = nasc;
            if (stage_next) store_slice((q + 1) & 1);
            __syncthreads();
            ++q;
        }
        // outputs of this unit: lane holds column col, rows f*32 + 8*(i/4) + 4*h + i%4
        // (an opaque copy of the lane index keeps the compiler from computing the row
        // addresses before the slice loop, where they would hold registers throughout)
        if (!ISUMS && cur.store) {
            int ln = lane;
            __asm__ volatile("" : "+v"(ln));
            const int h2 = ln >> 5;
            float *ocol = out + cur.s0 * N + cur.col;
#pragma unroll
            for (int f = 0; f < MF; ++f)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    if (f >= mt) break;
                    const int r = f * 32 + 8 * (i >> 2) + 4 * h2 + (i & 3);
                    const float as = sasc[u & 1][r];
                    if (as >= 0.0f) ocol[(int64_t)r * N] = as * acc[f][i];
                }
        }
        if (!more) break;
        ++u;
        cur = nxt;
        qrow = nqrow;
    }
    __builtin_amdgcn_s_waitcnt(0);  // the ring's last (unused) loads
}

template <int WM, int WN, bool ISUMS, int GS = G128>
__global__ __launch_bounds__(64 * WM * WN) void grouped_tiled_kernel(
    const int8_t *__restrict__ qa, const float *__restrict__ a_scale, int64_t R, const int32_t *__restrict__ row_index,
    const int32_t *__restrict__ offsets, int32_t E, int64_t K, const uint8_t *__restrict__ packed,
    const uint16_t *__restrict__ scale, const uint16_t *__restrict__ zp, int64_t N, int64_t max_slots,
    float *__restrict__ out, int32_t *__restrict__ isums, int64_t cmin, int64_t cmax) {
    using S = TileShape<WM, WN>;
    extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
    __shared__ int64_t pfx[kMaxExperts + 1];
    const int64_t ntn = (N + S::BN - 1) / S::BN;
    const int64_t total = expert_prefix(E, pfx, S::THREADS, [&](int e) -> int64_t {
        const int64_t c = clamp_slots(offsets[e + 1], max_slots) - clamp_slots(offsets[e], max_slots);
        return (c > cmin && c <= cmax) ? ((c + S::BM - 1) / S::BM) * ntn : 0;
    });
    // Round r hands each XCD (workgroup b runs on XCD b % 8) a contiguous run of units,
    // row tiles fastest: the workgroups of one XCD then share their experts' weight
    // columns and activation rows in that XCD's L2.
    const int64_t nb = gridDim.x;
    const bool by_xcd = nb % 8 == 0;
    const int64_t lane_u = by_xcd ? (blockIdx.x % 8) * (nb / 8) + blockIdx.x / 8 : blockIdx.x;
    for (int64_t u = lane_u; u < total; u += nb) {
        const int e = find_expert(pfx, E, u);
        const int64_t c = clamp_slots(offsets[e + 1], max_slots) - clamp_slots(offsets[e], max_slots);
        const int64_t mt = (c + S::BM - 1) / S::BM;
        const int64_t local = u - pfx[e];
        const int64_t tm = local % mt, tn = local / mt;
        const int64_t s0 = clamp_slots(offsets[e], max_slots) + tm * S::BM;
        const int rows = (int)((c - tm * S::BM) < S::BM ? (c - tm * S::BM) : S::BM);
        tile2_unit<WM, WN, ISUMS, GS>(dsm, qa, a_scale, row_index, R, TileRows{s0, rows}, K,
                                      packed + (int64_t)e * N * (K / 2),
                                      (ISUMS ? nullptr : scale + (int64_t)e * (K / GS) * N),
                                      zp + (int64_t)e * (K / GS) * N, N, tn * S::BN, out, N, isums, max_slots);
        __syncthreads();  // the next unit reuses the LDS buffers
    }
}

// Experts with more than cmin slots in 256-row tiles of the three-stage loop (the same unit
// order as grouped_tiled_kernel).
// EPI = kEpiSilu: the gate/up product with SiLU * up folded in (N = 2 I weight rows, tiles of
// 64 h columns, out lines of 2 I floats: h, then the per-16-column maxima).
template <bool ISUMS, int EPI = kEpiOut>
__global__ __launch_bounds__(kT3Threads) void grouped_tiled3_kernel(
    const int8_t *__restrict__ qa, const float *__restrict__ a_scale, int64_t R, const int32_t *__restrict__ row_index,
    const int32_t *__restrict__ offsets, int32_t E, int64_t K, const uint8_t *__restrict__ packed,
    const uint16_t *__restrict__ scale, const uint16_t *__restrict__ zp, int64_t N, int64_t max_slots,
    float *__restrict__ out, int32_t *__restrict__ isums, int64_t cmin, T3Epi ep) {
    extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
    __shared__ int64_t pfx[kMaxExperts + 1];
    constexpr int TBN = EPI == kEpiSilu ? kT3BN / 2 : kT3BN;  // output columns per tile
    const int64_t ntn = ((EPI == kEpiSilu ? ep.half : N) + TBN - 1) / TBN;
    const int64_t total = expert_prefix(E, pfx, kT3Threads, [&](int e) -> int64_t {
        const int64_t c = clamp_slots(offsets[e + 1], max_slots) - clamp_slots(offsets[e], max_slots);
        return c > cmin ? ((c + kT3BM - 1) / kT3BM) * ntn : 0;
    });
    const int64_t G = K / G128;
    const int64_t nb = gridDim.x;
    const bool by_xcd = nb % 8 == 0;
    const int64_t lane_u = by_xcd ? (blockIdx.x % 8) * (nb / 8) + blockIdx.x / 8 : blockIdx.x;
    for (int64_t u = lane_u; u < total; u += nb) {
        const int e = find_expert(pfx, E, u);
        const int64_t c = clamp_slots(offsets[e + 1], max_slots) - clamp_slots(offsets[e], max_slots);
        const int64_t mt = (c + kT3BM - 1) / kT3BM;
        const int64_t local = u - pfx[e];
        const int64_t tm = local % mt, tn = local / mt;
        const int64_t s0 = clamp_slots(offsets[e], max_slots) + tm * kT3BM;
        const int rows = (int)((c - tm * kT3BM) < kT3BM ? (c - tm * kT3BM) : kT3BM);
        tile3_unit<ISUMS, EPI, kT3FI>(dsm, qa, a_scale, row_index, R, TileRows{s0, rows}, K,
                               packed + (int64_t)e * N * (K / 2), (ISUMS ? nullptr : scale + (int64_t)e * G * N),
                               zp + (int64_t)e * G * N, N, tn * TBN, out, N, isums, max_slots, ep);
        __syncthreads();  // the next unit reuses the LDS stages and row tables
    }
}

// The same units in 256x256 tiles (tile4_unit: eight 128x64 wave tiles, two LDS stages): half
// as many units as the 256x128 loop, each weight column unpacked once per 256 rows.
// EPI = kEpiSilu: tiles of 128 h columns (256 weight rows: gate and up of each h column).
template <bool ISUMS, int EPI = kEpiOut>
__global__ __launch_bounds__(kT4Threads) void grouped_tiled4_kernel(
    const int8_t *__restrict__ qa, const float *__restrict__ a_scale, int64_t R, const int32_t *__restrict__ row_index,
    const int32_t *__restrict__ offsets, int32_t E, int64_t K, const uint8_t *__restrict__ packed,
    const uint16_t *__restrict__ scale, const uint16_t *__restrict__ zp, int64_t N, int64_t max_slots,
    float *__restrict__ out, int32_t *__restrict__ isums, int64_t cmin, T3Epi ep) {
    extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];
    __shared__ int64_t pfx[kMaxExperts + 1];
    constexpr int TBN = EPI == kEpiSilu ? kT4BN / 2 : kT4BN;  // output columns per tile
    const int64_t ntn = ((EPI == kEpiSilu ? ep.half : N) + TBN - 1) / TBN;
    const int64_t total = expert_prefix(E, pfx, kT4Threads, [&](int e) -> int64_t {
        const int64_t c = clamp_slots(offsets[e + 1], max_slots) - clamp_slots(offsets[e], max_slots);
        return c > cmin ? ((c + kT4BM - 1) / kT4BM) * ntn : 0;
    });
    const int64_t G = K / G128;
    const int64_t nb = gridDim.x;
    const bool by_xcd = nb % 8 == 0;
    const int64_t lane_u = by_xcd ? (blockIdx.x % 8) * (nb / 8) + blockIdx.x / 8 : blockIdx.x;
    for (int64_t u = lane_u; u < total; u += nb) {
        const int e = find_expert(pfx, E, u);
        const int64_t c = clamp_slots(offsets[e + 1], max_slots) - clamp_slots(offsets[e], max_slots);
        const int64_t mt = (c + kT4BM - 1) / kT4BM;
        const int64_t local = u - pfx[e];
        const int64_t tm = local % mt, tn = local / mt;
        const int64_t s0 = clamp_slots(offsets[e], max_slots) + tm * kT4BM;
        const int rows = (int)((c - tm * kT4BM) < kT4BM ? (c - tm * kT4BM) : kT4BM);
        tile4_unit<ISUMS, EPI>(dsm, qa, a_scale, row_index, R, TileRows{s0, rows}, K,
                               packed + (int64_t)e * N * (K / 2), (ISUMS ? nullptr : scale + (int64_t)e * G * N),
                               zp + (int64_t)e * G * N, N, tn * TBN, out, N, isums, max_slots, ep);
        __syncthreads();  // the next unit reuses the LDS stages and row tables
    }
}

template <int MT, int U, int SPLIT>
hipError_t launch_stream2_t(const int8_t *qa, const float *a_scale, int64_t M, int64_t K, const uint8_t *packed,
                            const uint16_t *scale, const uint16_t *zp, int64_t N, float *out, int32_t *isums,
                            hipStream_t stream) {
    const dim3 grid((uint32_t)(N / 16)), block(64 * SPLIT);
    if (isums)
        hipLaunchKernelGGL((gemm_stream2_kernel<MT, U, SPLIT, true>), grid, block, 0, stream, qa, a_scale, M, K, packed,
                           scale, zp, N, out, isums);
    else
        hipLaunchKernelGGL((gemm_stream2_kernel<MT, U, SPLIT, false>), grid, block, 0, stream, qa, a_scale, M, K,
                           packed, scale, zp, N, out, isums);
    return hipGetLastError();
}

template <int MT, int U>
hipError_t launch_stream2_s(int split, const int8_t *qa, const float *a_scale, int64_t M, int64_t K,
                            const uint8_t *packed, const uint16_t *scale, const uint16_t *zp, int64_t N, float *out,
                            int32_t *isums, hipStream_t stream) {
    return split == 2 ? launch_stream2_t<MT, U, 2>(qa, a_scale, M, K, packed, scale, zp, N, out, isums, stream)
                      : launch_stream2_t<MT, U, 1>(qa, a_scale, M, K, packed, scale, zp, N, out, isums, stream);
}

hipError_t launch_stream2(int mt, int u, int split, const int8_t *qa, const float *a_scale, int64_t M, int64_t K,
                          const uint8_t *packed, const uint16_t *scale, const uint16_t *zp, int64_t N, float *out,
                          int32_t *isums, hipStream_t stream) {
    if (mt == 1) {
        if (u >= 2) return launch_stream2_s<1, 2>(split, qa, a_scale, M, K, packed, scale, zp, N, out, isums, stream);
        return launch_stream2_s<1, 1>(split, qa, a_scale, M, K, packed, scale, zp, N, out, isums, stream);
    }
    if (mt == 2) {
        if (u >= 2) return launch_stream2_s<2, 2>(split, qa, a_scale, M, K, packed, scale, zp, N, out, isums, stream);
        return launch_stream2_s<2, 1>(split, qa, a_scale, M, K, packed, scale, zp, N, out, isums, stream);
    }
    return launch_stream2_s<4, 1>(split, qa, a_scale, M, K, packed, scale, zp, N, out, isums, stream);
}

template <int WM, int WN, int GS = G128>
hipError_t launch_tiled(const int8_t *qa, const float *a_scale, int64_t M, int64_t K, const uint8_t *packed,
                        const uint16_t *scale, const uint16_t *zp, int64_t N, float *out, int32_t *isums,
                        hipStream_t stream) {
    using S = TileShape<WM, WN>;
    const int64_t tiles = ((M + S::BM - 1) / S::BM) * ((N + S::BN - 1) / S::BN);
    const size_t lds = 2 * S::LDS_STAGE;
    const dim3 grid((uint32_t)tiles), block(S::THREADS);
    if (isums) {
        if (hipFuncSetAttribute((const void *)gemm_tiled_kernel<WM, WN, true, GS>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
            return hipGetLastError();
        hipLaunchKernelGGL((gemm_tiled_kernel<WM, WN, true, GS>), grid, block, lds, stream, qa, a_scale, M, K, packed,
                           scale, zp, N, out, isums);
    } else {
        if (hipFuncSetAttribute((const void *)gemm_tiled_kernel<WM, WN, false, GS>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
            return hipGetLastError();
        hipLaunchKernelGGL((gemm_tiled_kernel<WM, WN, false, GS>), grid, block, lds, stream, qa, a_scale, M, K, packed,
                           scale, zp, N, out, isums);
    }
    return hipGetLastError();
}

// The three-stage 256x128 loop, when its 32-bit offsets reach every operand.
bool tiled3_fits(int64_t M, int64_t K, int64_t N) {
    return M * K < (1ll << 32) && N * (K / 2) < (1ll << 32) && (K / G128) * N * 2 < (1ll << 31);
}

hipError_t launch_tiled3(const int8_t *qa, const float *a_scale, int64_t M, int64_t K, const uint8_t *packed,
                         const uint16_t *scale, const uint16_t *zp, int64_t N, float *out, int32_t *isums,
                         hipStream_t stream) {
    const int64_t tiles = ((M + kT3BM - 1) / kT3BM) * ((N + kT3BN - 1) / kT3BN);
    const dim3 grid((uint32_t)tiles), block(kT3Threads);
#define W4A8_T3(IS)                                                                                                 \
    do {                                                                                                            \
        if (hipFuncSetAttribute((const void *)gemm_tiled3_kernel<IS>, hipFuncAttributeMaxDynamicSharedMemorySize,   \
                                kT3Lds) != hipSuccess)                                                              \
            return hipGetLastError();                                                                               \
        hipLaunchKernelGGL((gemm_tiled3_kernel<IS>), grid, block, kT3Lds, stream, qa, a_scale, M, K, packed, scale, \
                           zp, N, out, isums, T3Epi{});                                                             \
    } while (0)
    if (isums) W4A8_T3(true);
    else W4A8_T3(false);
#undef W4A8_T3
    return hipGetLastError();
}

// 256x256 tiles when they still give every CU a workgroup (else the 256x128 loop, with twice
// as many tiles).
bool tiled4_pays(int64_t M, int64_t N) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    return ((M + kT4BM - 1) / kT4BM) * ((N + kT4BN - 1) / kT4BN) >= cus;
}

hipError_t launch_tiled4(const int8_t *qa, const float *a_scale, int64_t M, int64_t K, const uint8_t *packed,
                         const uint16_t *scale, const uint16_t *zp, int64_t N, float *out, int32_t *isums,
                         hipStream_t stream) {
    const int64_t tiles = ((M + kT4BM - 1) / kT4BM) * ((N + kT4BN - 1) / kT4BN);
    const dim3 grid((uint32_t)tiles), block(kT4Threads);
#define W4A8_T4(IS)                                                                                                 \
    do {                                                                                                            \
        if (hipFuncSetAttribute((const void *)gemm_tiled4_kernel<IS>, hipFuncAttributeMaxDynamicSharedMemorySize,   \
                                kT4Lds) != hipSuccess)                                                              \
            return hipGetLastError();                                                                               \
        hipLaunchKernelGGL((gemm_tiled4_kernel<IS>), grid, block, kT4Lds, stream, qa, a_scale, M, K, packed, scale, \
                           zp, N, out, isums);                                                                      \
    } while (0)
    if (isums) W4A8_T4(true);
    else W4A8_T4(false);
#undef W4A8_T4
    return hipGetLastError();
}

// tm: `packed` is the tile-major array (scale and zp unused; no isums)
template <int GS = G128>
hipError_t launch_decode(const int8_t *qa, const float *a_scale, int64_t M, int64_t K, const uint8_t *packed,
                         const uint16_t *scale, const uint16_t *zp, int64_t N, float *out, int32_t *isums,
                         bool tm, hipStream_t stream) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return hipGetLastError();
    const int64_t G = K / G128;
    const int64_t ntiles = N / 16;
    int64_t tpw = (ntiles + cus - 1) / cus;
    // K parts per tile: two, or four when a workgroup has at most four tiles (so
    // that all 16 waves stream), as far as the groups divide evenly
    const int split = (G % 8 == 0 && tpw <= 4) ? 4 : ((G % 4 == 0) ? 2 : 1);
    // Tiles per workgroup rounded up to whole rounds of the 16 waves (16 / split tiles a
    // round) when at least 7/8 of the CUs still get a workgroup: every wave then streams
    // (K = 8192, N = 28672: 7 -> 8 tiles, 256 -> 224 workgroups, 22.3 -> 22.1 us).
    {
        const int64_t per_round = kDecWaves / split;
        const int64_t up = (tpw + per_round - 1) / per_round * per_round;
        if (up != tpw && 8 * ((ntiles + up - 1) / up) >= 7 * (int64_t)cus) tpw = up;
    }
    const int64_t nwg = (ntiles + tpw - 1) / tpw;
    const size_t lds = (size_t)(((dec_lds_bytes(M, K) + 15) / 16) * 16 + dec_red_bytes(split));
    const int64_t nwin = G / 2 / split;
    const dim3 grid((uint32_t)nwg), block(kDecThreads);
    // rows staged with one load per thread when they fit, else eight at a time
    const bool one = M * K <= (int64_t)kDecThreads * 16;
#define W4A8_DEC1(UU, SS, IS, SB, TT)                                                                               \
    do {                                                                                                            \
        constexpr int GG = (TT) ? G128 : GS;                                                                        \
        if (hipFuncSetAttribute((const void *)gemm_decode_kernel<UU, SS, IS, SB, TT, GG>,                           \
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)                \
            return hipGetLastError();                                                                               \
        hipLaunchKernelGGL((gemm_decode_kernel<UU, SS, IS, SB, TT, GG>), grid, block, lds, stream, qa, a_scale, M,  \
                           K, packed, scale, zp, N, tpw, out, isums);                                               \
    } while (0)
#define W4A8_DEC(UU, SS)                                                                                            \
    do {                                                                                                            \
        if (isums) W4A8_DEC1(UU, SS, true, 8, false);                                                               \
        else if (one) W4A8_DEC1(UU, SS, false, 1, false);                                                           \
        else W4A8_DEC1(UU, SS, false, 8, false);                                                                    \
    } while (0)
    // tile-major weights: contiguous streams take a deeper ring (four windows in flight);
    // the rows are staged by direct-to-LDS loads, so the staging batch does not apply
#define W4A8_DEC_TM(UU, SS) W4A8_DEC1(UU, SS, false, 1, true)
    if (GS == G128 && tm) {
        if (split == 4) {
            if (nwin % 4 == 0) W4A8_DEC_TM(4, 4);
            else if (nwin % 2 == 0) W4A8_DEC_TM(2, 4);
            else W4A8_DEC_TM(1, 4);
        } else if (split == 2) {
            if (nwin % 4 == 0) W4A8_DEC_TM(4, 2);
            else if (nwin % 2 == 0) W4A8_DEC_TM(2, 2);
            else W4A8_DEC_TM(1, 2);
        } else {
            if (nwin % 4 == 0) W4A8_DEC_TM(4, 1);
            else if (nwin % 2 == 0) W4A8_DEC_TM(2, 1);
            else W4A8_DEC_TM(1, 1);
        }
        return hipGetLastError();
    }
#undef W4A8_DEC_TM
    if (split == 4) {
        if (nwin % 2 == 0) W4A8_DEC(2, 4);
        else W4A8_DEC(1, 4);
    } else if (split == 2) {
        if (nwin % 2 == 0) W4A8_DEC(2, 2);
        else W4A8_DEC(1, 2);
    } else {
        if (nwin % 2 == 0) W4A8_DEC(2, 1);
        else W4A8_DEC(1, 1);
    }
#undef W4A8_DEC
#undef W4A8_DEC1
    return hipGetLastError();
}

}  // namespace

namespace w4a8 {

hipError_t launch_gemm(const int8_t *qa, const float *a_scale, int64_t M, int64_t K, const uint8_t *packed,
                       const uint16_t *scale, const uint16_t *zp, int64_t N, int path, float *out, int32_t *isums,
                       hipStream_t stream) {
    // (the debug entry passes no scale array: its ISUMS forms read none)
    if (path == 1) {
        const int64_t G = K / G128;
        const int mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
        // (the decode loop addresses the packed codes with 32-bit buffer offsets)
        if (G % 2 == 0 && M <= 16 && dec_lds_bytes(M, K) <= kDecLdsMax && N * (K / 2) < kDecCodesMax)
            return launch_decode(qa, a_scale, M, K, packed, scale, zp, N, out, isums, false, stream);
        if (G % 2 == 0) {
            // line-wide loop: two-group windows, K split over two waves when it divides
            const int split = (G % 4 == 0) ? 2 : 1;
            const int64_t nwin = G / 2 / split;
            const int u = ring_depth(nwin, mt == 4 ? 1 : 2);
            return launch_stream2(mt, u, split, qa, a_scale, M, K, packed, scale, zp, N, out, isums, stream);
        }
        const dim3 grid((uint32_t)(N / 16)), block(kStreamThreads);
        const int umax = M <= 16 ? 8 : (M <= 32 ? 4 : 2);
        const int U = ring_depth(G, umax);
#define W4A8_STREAM_U(MT, UU)                                                                                     \
    do {                                                                                                          \
        if (isums)                                                                                                \
            hipLaunchKernelGGL((gemm_stream_kernel<MT, UU, true>), grid, block, 0, stream, qa, a_scale, M, K,     \
                               packed, scale, zp, N, out, isums);                                                 \
        else                                                                                                      \
            hipLaunchKernelGGL((gemm_stream_kernel<MT, UU, false>), grid, block, 0, stream, qa, a_scale, M, K,    \
                               packed, scale, zp, N, out, isums);                                                 \
    } while (0)
#define W4A8_STREAM(MT)                              \
    do {                                             \
        if (U == 8) W4A8_STREAM_U(MT, (MT == 1 ? 8 : 1)); \
        else if (U == 4) W4A8_STREAM_U(MT, (MT <= 2 ? 4 : 1)); \
        else if (U == 2) W4A8_STREAM_U(MT, 2);       \
        else W4A8_STREAM_U(MT, 1);                   \
    } while (0)
        if (M <= 16) W4A8_STREAM(1);
        else if (M <= 32) W4A8_STREAM(2);
        else W4A8_STREAM(4);
#undef W4A8_STREAM
#undef W4A8_STREAM_U
    } else {
        if (tiled3_fits(M, K, N) && (path == 5 || (path == 2 && M > 128 && tiled4_pays(M, N))))
            return launch_tiled4(qa, a_scale, M, K, packed, scale, zp, N, out, isums, stream);
        if (path >= 4 || (path == 2 && M > 128)) {
            if (tiled3_fits(M, K, N))
                return launch_tiled3(qa, a_scale, M, K, packed, scale, zp, N, out, isums, stream);
            return launch_tiled<4, 2>(qa, a_scale, M, K, packed, scale, zp, N, out, isums, stream);
        }
        return launch_tiled<2, 2>(qa, a_scale, M, K, packed, scale, zp, N, out, isums, stream);
    }
    return hipGetLastError();
}

bool decode_group_fits(int64_t M, int64_t K, int64_t N) {
    return M >= 1 && M <= 16 && K % (2 * G128) == 0 && dec_lds_bytes(M, K) <= kDecLdsMax && N * (K / 2) < kDecCodesMax;
}

hipError_t launch_gemm_tiled_group(const int8_t *qa, const float *a_scale, int64_t M, int64_t K, const uint8_t *packed,
                                   const uint16_t *scale, const uint16_t *zp, int64_t N, int group, int path, float *out,
                                   int32_t *isums, hipStream_t stream) {
    if (path == 1) {  // the decode loop (the caller checked decode_group_fits)
        if (group == 64)
            return launch_decode<64>(qa, a_scale, M, K, packed, scale, zp, N, out, isums, false, stream);
        return launch_decode<256>(qa, a_scale, M, K, packed, scale, zp, N, out, isums, false, stream);
    }
    const bool wide = path >= 4 || (path == 2 && M > 128);  // (path 5: the 256x128 loop at these sizes)
    if (group == 64)
        return wide ? launch_tiled<4, 2, 64>(qa, a_scale, M, K, packed, scale, zp, N, out, isums, stream)
                    : launch_tiled<2, 2, 64>(qa, a_scale, M, K, packed, scale, zp, N, out, isums, stream);
    if (group == 256)
        return wide ? launch_tiled<4, 2, 256>(qa, a_scale, M, K, packed, scale, zp, N, out, isums, stream)
                    : launch_tiled<2, 2, 256>(qa, a_scale, M, K, packed, scale, zp, N, out, isums, stream);
    if (wide && tiled3_fits(M, K, N)) return launch_tiled3(qa, a_scale, M, K, packed, scale, zp, N, out, isums, stream);
    return wide ? launch_tiled<4, 2>(qa, a_scale, M, K, packed, scale, zp, N, out, isums, stream)
                : launch_tiled<2, 2>(qa, a_scale, M, K, packed, scale, zp, N, out, isums, stream);
}

int64_t tm_bytes(int64_t N, int64_t K) { return (N / 16) * (K / G128 / 2) * kTmBlock; }

// M <= 16: the decode loop (rows staged in LDS); above: the 256x256 tiled loop (activation
// offsets below 2^32).  Either way the tile-major array must stay below 4 GiB.
bool gemm_tm_supported(int64_t M, int64_t K, int64_t N) {
    if (M < 1 || K % (2 * G128) != 0 || N % 16 != 0 || tm_bytes(N, K) >= kDecCodesMax) return false;
    return M <= 16 ? dec_lds_bytes(M, K) <= kDecLdsMax : M * K < (1ll << 32);
}

hipError_t launch_gemm_tm(const int8_t *qa, const float *a_scale, int64_t M, int64_t K, const uint8_t *tm, int64_t N,
                          float *out, hipStream_t stream) {
    if (M <= 16) return launch_decode(qa, a_scale, M, K, tm, nullptr, nullptr, N, out, nullptr, true, stream);
    const int64_t tiles = ((M + kT4BM - 1) / kT4BM) * ((N + kT4BN - 1) / kT4BN);
    if (hipFuncSetAttribute((const void *)gemm_tiled4_kernel<false, kEpiOut, true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kT4Lds) != hipSuccess)
        return hipGetLastError();
    hipLaunchKernelGGL((gemm_tiled4_kernel<false, kEpiOut, true>), dim3((uint32_t)tiles), dim3(kT4Threads), kT4Lds,
                       stream, qa, a_scale, M, K, tm, (const uint16_t *)nullptr, (const uint16_t *)nullptr, N, out,
                       (int32_t *)nullptr);
    return hipGetLastError();
}

// Standard layout -> tile-major: thread i of workgroup b (b = t * G/2 + w) writes the
// 16 code bytes of lane i & 63 for group 2 w + (i >> 6) (i < 128), or fp16 word
// i - 128 of the block's scale and zero-point area (column (i - 128) / 4).
__global__ __launch_bounds__(192) void weights_to_tm_kernel(const uint8_t *__restrict__ packed,
                                                            const uint16_t *__restrict__ scale,
                                                            const uint16_t *__restrict__ zp, int64_t N, int64_t K,
                                                            uint8_t *__restrict__ tm) {
    const int64_t G = K / G128, W = G / 2;
    const int64_t b = (int64_t)blockIdx.x;
    if (b >= (N / 16) * W) return;
    const int64_t t = b / W, w = b % W;
    uint8_t *dst = tm + b * kTmBlock;
    const int i = threadIdx.x;
    if (i < 128) {
        const int l = i & 63, h = i >> 6;
        const int64_t col = 16 * t + (l & 15);
        const v4u v = *reinterpret_cast<const v4u *>(packed + col * (K / 2) + (2 * w + h) * (G128 / 2) + 16 * (l >> 4));
        // standard bytes hold codes (2j, 2j + 1); re-pair each run of 8 as (b, b + 4)
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t c03, c47;
            spread8(d[j], c03, c47);
            o[j] = c03 | (c47 << 4);
        }
        *reinterpret_cast<v4u *>(dst + h * 1024 + 16 * l) = v4u{o[0], o[1], o[2], o[3]};
    } else {
        const int l = i - 128, c = l >> 2, j = l & 3;
        const int64_t col = 16 * t + c;
        uint16_t word = 0;
        if (j < 2) {
            word = scale[(2 * w + j) * N + col];
        } else if (j == 2) {
            const uint32_t z0 = (uint32_t)(-(int)half_bits_to_float(zp[(2 * w) * N + col])) & 0xFFu;
            const uint32_t z1 = (uint32_t)(-(int)half_bits_to_float(zp[(2 * w + 1) * N + col])) & 0xFFu;
            word = (uint16_t)(z0 | (z1 << 8));
        }
        reinterpret_cast<uint16_t *>(dst + 2048)[l] = word;
    }
}

hipError_t launch_weights_to_tm(const uint8_t *packed, const uint16_t *scale, const uint16_t *zp, int64_t N, int64_t K,
                                uint8_t *tm, hipStream_t stream) {
    const int64_t blocks = (N / 16) * (K / G128 / 2);
    hipLaunchKernelGGL(weights_to_tm_kernel, dim3((uint32_t)blocks), dim3(192), 0, stream, packed, scale, zp, N, K, tm);
    return hipGetLastError();
}

// Experts with more than cmin slots: 128-row tiles up to 128 slots, 256-row tiles
// above (a 256-row tile over a 65..128-slot expert would waste most of its work).
template <int WM, int WN, bool IS, int GS>
static hipError_t launch_grouped_tiled_t(const int8_t *qa, const float *a_scale, int64_t R, const int32_t *row_index,
                                         const int32_t *expert_offsets, int32_t E, int64_t K, const uint8_t *packed,
                                         const uint16_t *scale, const uint16_t *zp, int64_t N, int64_t max_slots,
                                         float *out, int32_t *isums, int64_t cmin, int64_t cmax, int cus,
                                         hipStream_t stream) {
    using S = TileShape<WM, WN>;
    const size_t lds = 2 * S::LDS_STAGE;
    if (hipFuncSetAttribute((const void *)grouped_tiled_kernel<WM, WN, IS, GS>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return hipGetLastError();
    hipLaunchKernelGGL((grouped_tiled_kernel<WM, WN, IS, GS>), dim3((uint32_t)cus), dim3(S::THREADS), lds, stream, qa,
                       a_scale, R, row_index, expert_offsets, E, K, packed, scale, zp, N, max_slots, out, isums, cmin,
                       cmax);
    return hipGetLastError();
}

template <int WM, int WN>
static hipError_t launch_grouped_tiled_s(const int8_t *qa, const float *a_scale, int64_t R, const int32_t *row_index,
                                         const int32_t *expert_offsets, int32_t E, int64_t K, const uint8_t *packed,
                                         const uint16_t *scale, const uint16_t *zp, int64_t N, int64_t max_slots,
                                         float *out, int32_t *isums, int64_t cmin, int64_t cmax, int cus, int gs,
                                         hipStream_t stream) {
#define W4A8_GTS(IS, GG)                                                                                            \
    return launch_grouped_tiled_t<WM, WN, IS, GG>(qa, a_scale, R, row_index, expert_offsets, E, K, packed, scale,   \
                                                  zp, N, max_slots, out, isums, cmin, cmax, cus, stream)
    if (gs == 64) {
        if (isums) W4A8_GTS(true, 64);
        W4A8_GTS(false, 64);
    }
    if (gs == 256) {
        if (isums) W4A8_GTS(true, 256);
        W4A8_GTS(false, 256);
    }
    if (isums) W4A8_GTS(true, G128);
    W4A8_GTS(false, G128);
#undef W4A8_GTS
}

// The expert loop over 256x256 tiles when the slots could fill every CU with such tiles at
// least twice over (an estimate from the slot count: the device-side offsets are not read
// here); else the 256x128 loop, with twice as many units.
static bool grouped_tiled4_pays(int64_t max_slots, int64_t N, int cus) {
    return (max_slots / kT4BM) * ((N + kT4BN - 1) / kT4BN) >= 2 * (int64_t)cus;
}

// experts with more than cmin slots
static hipError_t launch_grouped_tiled(const int8_t *qa, const float *a_scale, int64_t R, const int32_t *row_index,
                                       const int32_t *expert_offsets, int32_t E, int64_t K, const uint8_t *packed,
                                       const uint16_t *scale, const uint16_t *zp, int64_t N, int64_t max_slots,
                                       float *out, int32_t *isums, int64_t cmin, int cus, int gs, hipStream_t stream,
                                       const T3Epi *silu, int64_t *fused_min) {
    if (max_slots <= cmin) return hipSuccess;
    if (cmin < 128) {
        hipError_t err = launch_grouped_tiled_s<2, 2>(qa, a_scale, R, row_index, expert_offsets, E, K, packed, scale,
                                                      zp, N, max_slots, out, isums, cmin, 128, cus, gs, stream);
        if (err != hipSuccess || max_slots <= 128) return err;
    }
    if (gs == G128 && tiled3_fits(R, K, N) && grouped_tiled4_pays(max_slots, N, cus)) {
#define W4A8_GT4(IS, EP, EPA)                                                                                       \
    do {                                                                                                            \
        if (hipFuncSetAttribute((const void *)grouped_tiled4_kernel<IS, EP>,                                        \
                                hipFuncAttributeMaxDynamicSharedMemorySize, kT4Lds) != hipSuccess)                  \
            return hipGetLastError();                                                                               \
        hipLaunchKernelGGL((grouped_tiled4_kernel<IS, EP>), dim3((uint32_t)cus), dim3(kT4Threads), kT4Lds, stream,  \
                           qa, a_scale, R, row_index, expert_offsets, E, K, packed, scale, zp, N, max_slots, out,   \
                           isums, (int64_t)128, EPA);                                                               \
    } while (0)
        if (isums) {
            W4A8_GT4(true, kEpiOut, T3Epi{});
        } else if (silu) {  // the >128-slot experts with SiLU * up folded into the epilogue
            W4A8_GT4(false, kEpiSilu, *silu);
            if (fused_min) *fused_min = 128;
        } else {
            W4A8_GT4(false, kEpiOut, T3Epi{});
        }
#undef W4A8_GT4
        return hipGetLastError();
    }
    if (gs == G128 && tiled3_fits(R, K, N)) {
#define W4A8_GT3(IS)                                                                                                \
    do {                                                                                                            \
        if (hipFuncSetAttribute((const void *)grouped_tiled3_kernel<IS>,                                            \
                                hipFuncAttributeMaxDynamicSharedMemorySize, kT3Lds) != hipSuccess)                  \
            return hipGetLastError();                                                                               \
        hipLaunchKernelGGL((grouped_tiled3_kernel<IS>), dim3((uint32_t)cus), dim3(kT3Threads), kT3Lds, stream, qa,  \
                           a_scale, R, row_index, expert_offsets, E, K, packed, scale, zp, N, max_slots, out, isums,  \
                           (int64_t)128, T3Epi{});                                                                  \
    } while (0)
        if (isums) {
            W4A8_GT3(true);
        } else if (silu) {  // the >128-slot experts with SiLU * up folded into the epilogue
            if (hipFuncSetAttribute((const void *)grouped_tiled3_kernel<false, kEpiSilu>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, kT3Lds) != hipSuccess)
                return hipGetLastError();
            hipLaunchKernelGGL((grouped_tiled3_kernel<false, kEpiSilu>), dim3((uint32_t)cus), dim3(kT3Threads), kT3Lds,
                               stream, qa, a_scale, R, row_index, expert_offsets, E, K, packed, scale, zp, N,
                               max_slots, out, isums, (int64_t)128, *silu);
            if (fused_min) *fused_min = 128;
        } else {
            W4A8_GT3(false);
        }
#undef W4A8_GT3
        return hipGetLastError();
    }
    return launch_grouped_tiled_s<4, 2>(qa, a_scale, R, row_index, expert_offsets, E, K, packed, scale, zp, N,
                                        max_slots, out, isums, 128, INT64_MAX, cus, gs, stream);
}

hipError_t launch_grouped_gemm(const int8_t *qa, const float *a_scale, int64_t R, const int32_t *row_index,
                               const int32_t *expert_offsets, int32_t E, int64_t K, const uint8_t *packed,
                               const uint16_t *scale, const uint16_t *zp, int64_t N, int64_t max_slots,
                               int64_t max_per_expert, float *out, int32_t *isums, int gs, hipStream_t stream,
                               const T3Epi *silu, int64_t *fused_min) {
    if (max_per_expert > max_slots) max_per_expert = max_slots;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return hipGetLastError();
    const int64_t G = K / G128;
    if (gs != G128) {
        // group sizes 64 and 256: the 16-row loop up to 16 slots when its conditions hold,
        // the tiled loop (128- and 256-row tiles) above
        int64_t cmin = 0;
        if (G % 4 == 0 && dec_lds_bytes(16, K) <= kDecLdsMax && N * (K / 2) < kDecCodesMax &&
            (int64_t)R * K < (1ll << 32)) {
            const dim3 dgrid((uint32_t)cus), dblock(kDecThreads);
            const int64_t chunks = std::min<int64_t>(max_slots, (max_slots + 15) / 16 + E);
            const bool four = G % 8 == 0 && chunks * (N / 16) <= 4 * (int64_t)cus;
            const int split = four ? 4 : 2;
            const size_t dlds = (size_t)(((dec_lds_bytes(16, K) + 15) / 16) * 16 + dec_red_bytes(split));
#define W4A8_GDG(UU, SS, IS, GG)                                                                                    \
    do {                                                                                                            \
        if (hipFuncSetAttribute((const void *)grouped_decode_kernel<UU, SS, IS, GG>,                                \
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)dlds) != hipSuccess)               \
            return hipGetLastError();                                                                               \
        hipLaunchKernelGGL((grouped_decode_kernel<UU, SS, IS, GG>), dgrid, dblock, dlds, stream, qa, a_scale, R,    \
                           row_index, expert_offsets, E, K, packed, scale, zp, N, max_slots, out, isums, 16,        \
                           (int64_t)0);                                                                             \
    } while (0)
#define W4A8_GDG2(UU, SS)                                                                                           \
    do {                                                                                                            \
        if (gs == 64) {                                                                                             \
            if (isums) W4A8_GDG(UU, SS, true, 64);                                                                  \
            else W4A8_GDG(UU, SS, false, 64);                                                                       \
        } else {                                                                                                    \
            if (isums) W4A8_GDG(UU, SS, true, 256);                                                                 \
            else W4A8_GDG(UU, SS, false, 256);                                                                      \
        }                                                                                                           \
    } while (0)
            if (four) {
                if ((G / 8) % 2 == 0) W4A8_GDG2(2, 4);
                else W4A8_GDG2(1, 4);
            } else {
                if ((G / 4) % 2 == 0) W4A8_GDG2(2, 2);
                else W4A8_GDG2(1, 2);
            }
#undef W4A8_GDG2
#undef W4A8_GDG
            const hipError_t err = hipGetLastError();
            if (err != hipSuccess) return err;
            cmin = 16;
        }
        if (max_per_expert <= cmin) return hipSuccess;
        return launch_grouped_tiled(qa, a_scale, R, row_index, expert_offsets, E, K, packed, scale, zp, N, max_slots,
                                    out, isums, cmin, cus, gs, stream, silu, fused_min);
    }
    // the decode loop stages gathered rows with 32-bit offsets (row * K) and addresses the
    // codes with 32-bit offsets; larger inputs take the streaming loop (64-bit addresses)
    if (G % 4 == 0 && dec_lds_bytes(16, K) <= kDecLdsMax && N * (K / 2) < kDecCodesMax &&
        (int64_t)R * K < (1ll << 32)) {
        const dim3 dgrid((uint32_t)cus), dblock(kDecThreads);
        // experts with 17..128 slots: one weight pass per 64 rows when the K slicing
        // fits (at least two slices; activation offsets below 2^32)
        const bool mid = G % kMidSlice == 0 && G >= 2 * kMidSlice;
        const int small_max = mid ? kMidMin : (int)kSmallRows;
        // the weight-streaming loop runs if some expert can be in its class; the decode
        // loop takes that class when it has too few units to keep a quarter of the CUs
        // busy (a lone mid-size expert): re-reading it per 16 rows is then cheaper
        const int64_t mid_floor = (mid && max_per_expert > kMidMin) ? cus / 4 : 0;
#define W4A8_GDEC1(UU, SS, IS)                                                                                      \
    do {                                                                                                            \
        const size_t dlds = (size_t)(((dec_lds_bytes(16, K) + 15) / 16) * 16 + dec_red_bytes(SS));                 \
        if (hipFuncSetAttribute((const void *)grouped_decode_kernel<UU, SS, IS>,                                    \
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)dlds) != hipSuccess)               \
            return hipGetLastError();                                                                               \
        hipLaunchKernelGGL((grouped_decode_kernel<UU, SS, IS>), dgrid, dblock, dlds, stream, qa, a_scale, R,        \
                           row_index, expert_offsets, E, K, packed, scale, zp, N, max_slots, out, isums, small_max, \
                           mid_floor);                                                                              \
    } while (0)
#define W4A8_GDEC(UU, SS)                         \
    do {                                          \
        if (isums) W4A8_GDEC1(UU, SS, true);      \
        else W4A8_GDEC1(UU, SS, false);           \
    } while (0)
        // four K parts per tile when no workgroup can get more than four tiles (an upper
        // bound of the work: each expert's last chunk may be partial)
        const int64_t chunks = std::min<int64_t>(max_slots, (max_slots + 15) / 16 + E);
        const bool four = G % 8 == 0 && chunks * (N / 16) <= 4 * (int64_t)cus;
        if (four) {
            if ((G / 8) % 2 == 0) W4A8_GDEC(2, 4);
            else W4A8_GDEC(1, 4);
        } else {
            if ((G / 4) % 2 == 0) W4A8_GDEC(2, 2);
            else W4A8_GDEC(1, 2);
        }
#undef W4A8_GDEC
#undef W4A8_GDEC1
        hipError_t derr = hipGetLastError();
        if (derr != hipSuccess) return derr;
        if (!mid) return max_per_expert <= kSmallRows ? hipSuccess
                                                      : launch_grouped_tiled(qa, a_scale, R, row_index, expert_offsets,
                                                                             E, K, packed, scale, zp, N, max_slots, out,
                                                                             isums, kSmallRows, cus, G128, stream, silu,
                                                                             fused_min);
        // the other loops only when some expert can have that many slots
#define W4A8_GMID1(MF, CMIN, CMAX, IS)                                                                              \
    do {                                                                                                            \
        if (hipFuncSetAttribute((const void *)grouped_mid_kernel<MF, 4, IS>,                                        \
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)mid_lds_bytes(MF)) != hipSuccess)  \
            return hipGetLastError();                                                                               \
        hipLaunchKernelGGL((grouped_mid_kernel<MF, 4, IS>), dim3((uint32_t)cus), dim3(kMidThreads),                \
                           (size_t)mid_lds_bytes(MF), stream, qa, a_scale, R, row_index, expert_offsets, E, K,       \
                           packed, scale, zp, N, max_slots, out, isums, (int64_t)(CMIN), (int64_t)(CMAX),           \
                           mid_floor);                                                                              \
        if ((derr = hipGetLastError()) != hipSuccess) return derr;                                                  \
    } while (0)
        static_assert(kMidRows == 64, "the weight-streaming loop stages 64 rows (MF = 2)");
        if (max_per_expert > kMidMin) {  // 65..128 slots: two row blocks, the weights read twice
            if (isums) W4A8_GMID1(2, kMidMin, kMidMax, true);
            else W4A8_GMID1(2, kMidMin, kMidMax, false);
        }
#undef W4A8_GMID1
        if (max_per_expert <= kMidMax) return hipSuccess;
        return launch_grouped_tiled(qa, a_scale, R, row_index, expert_offsets, E, K, packed, scale, zp, N, max_slots,
                                    out, isums, kMidMax, cus, G128, stream, silu, fused_min);
    }
    const int U = ring_depth(G, 4);
    const dim3 sgrid((uint32_t)(cus * 8)), sblock(kStreamThreads);
#define W4A8_GSTR(UU)                                                                                               \
    do {                                                                                                            \
        if (isums)                                                                                                  \
            hipLaunchKernelGGL((grouped_stream_kernel<UU, true>), sgrid, sblock, 0, stream, qa, a_scale, R,         \
                               row_index, expert_offsets, E, K, packed, scale, zp, N, max_slots, out, isums);       \
        else                                                                                                        \
            hipLaunchKernelGGL((grouped_stream_kernel<UU, false>), sgrid, sblock, 0, stream, qa, a_scale, R,        \
                               row_index, expert_offsets, E, K, packed, scale, zp, N, max_slots, out, isums);       \
    } while (0)
    if (U == 4) W4A8_GSTR(4);
    else if (U == 2) W4A8_GSTR(2);
    else W4A8_GSTR(1);
#undef W4A8_GSTR
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || max_per_expert <= kSmallRows) return err;
    return launch_grouped_tiled(qa, a_scale, R, row_index, expert_offsets, E, K, packed, scale, zp, N, max_slots, out,
                                isums, kSmallRows, cus, G128, stream, silu, fused_min);
}

// The MoE shared expert's down product (T token rows) with the weighted combine folded in.
bool shared_combine_fits(int64_t T, int64_t I, int64_t H, int32_t topk) {
    return T > 128 && topk <= 8 && H % 4 == 0 && tiled3_fits(T, I, H);
}

hipError_t launch_shared_combine(const int8_t *qh, const float *h_scale, int64_t T, int64_t I, const uint8_t *packed,
                                 const uint16_t *scale, const uint16_t *zp, int64_t H, float *y_shared,
                                 const float *y, const int32_t *slot_of_pair, const float *topk_w, int32_t topk,
                                 float *out, hipStream_t stream) {
    const int64_t tiles = ((T + kT3BM - 1) / kT3BM) * ((H + kT3BN - 1) / kT3BN);
    T3Epi ep{};
    ep.y = y;
    ep.sop = slot_of_pair;
    ep.tw = topk_w;
    ep.k = topk;
    ep.fin = out;
    if (hipFuncSetAttribute((const void *)gemm_tiled3_kernel<false, kEpiCombine>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kT3Lds) != hipSuccess)
        return hipGetLastError();
    hipLaunchKernelGGL((gemm_tiled3_kernel<false, kEpiCombine>), dim3((uint32_t)tiles), dim3(kT3Threads), kT3Lds,
                       stream, qh, h_scale, T, I, packed, scale, zp, H, y_shared, (int32_t *)nullptr, ep);
    return hipGetLastError();
}

}  // namespace w4a8
