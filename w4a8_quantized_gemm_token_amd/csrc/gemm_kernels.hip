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
// Two main loops:
//  * streaming (small M, HBM-bound): one wave owns 16 output columns and up to
//    64 rows; it streams its columns' packed bytes with 128-bit loads, prefetched
//    several groups ahead in registers, and feeds v_mfma_i32_16x16x64_i8
//    directly from registers.  Workgroups are ordered so that neighbouring
//    column tiles run on the same XCD (their scale/zp rows share cache lines).
//  * tiled (large M, MFMA-bound): a 256-thread workgroup computes a 128x128
//    tile; each group of 128 k is staged in LDS (double-buffered, padded rows),
//    the weights are unpacked once per workgroup into LDS as INT8, and four
//    waves each run a 64x64 sub-tile with v_mfma_i32_32x32x32_i8.
// Both keep the per-group int32 sum in the MFMA accumulator and fold it into an
// fp32 accumulator with one fma per element per group, groups in increasing g.
#include "w4a8_internal.hpp"

using namespace w4a8dev;

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

// Bijective XCD-aware order: workgroup b runs on XCD b % 8; give each XCD a
// contiguous range of tiles so that neighbouring tiles share that XCD's L2.
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t ntiles) {
    const int64_t q = ntiles / 8, r = ntiles % 8;
    const int64_t x = b % 8, i = b / 8;
    return x * q + (x < r ? x : r) + i;
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
    const int lane = threadIdx.x & 63;
    const int kq = lane >> 4;
    const int64_t col = n0 + (lane & 15);
    const int64_t G = K / G128;

    const v4u *bptr = reinterpret_cast<const v4u *>(wpk + col * (K / 2) + kq * 16);
    const uint16_t *sptr = wsc + col;
    const uint16_t *zptr = wzp + col;

    // activation rows of this lane (row (l & 15) of each 16-row tile)
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
        sq[u] = sptr[g * N];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (avalid[t]) {
                const v4u *ap = reinterpret_cast<const v4u *>(aptr[t] + g * G128);
                aq[u][t][0] = ap[0];
                aq[u][t][1] = ap[1];
            } else {
                aq[u][t][0] = v4u{0u, 0u, 0u, 0u};
                aq[u][t][1] = v4u{0u, 0u, 0u, 0u};
            }
        }
    };

#pragma unroll
    for (int u = 0; u < U; ++u)
        if (u < G) load_group(u, u);

    for (int64_t g0 = 0; g0 < G; g0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t g = g0 + u;
            if (g < G) {
                const v4u b = bq[u];
                const uint16_t zb = zq[u], sb = sq[u];
                v4u a[MT][2];
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    a[t][0] = aq[u][t][0];
                    a[t][1] = aq[u][t][1];
                }
                if (g + U < G) load_group(u, g + U);

                const uint32_t zadd = zp_add_const(zb);
                uint32_t w[8];
                unpack8(b.x, zadd, w[0], w[1]);
                unpack8(b.y, zadd, w[2], w[3]);
                unpack8(b.z, zadd, w[4], w[5]);
                unpack8(b.w, zadd, w[6], w[7]);
                const v4i b0 = {(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
                const v4i b1 = {(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
                const float sc = half_bits_to_float(sb);
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const v4i a0 = {(int)a[t][0].x, (int)a[t][0].y, (int)a[t][0].z, (int)a[t][0].w};
                    const v4i a1 = {(int)a[t][1].x, (int)a[t][1].y, (int)a[t][1].z, (int)a[t][1].w};
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
            }
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
constexpr int kTileThreads = 256;
constexpr int BM = 128, BN = 128;
constexpr int kLdsStride = G128 + 16;  // padded row: 144 bytes, conflict-free 128-bit reads
constexpr int kLdsTile = BM * kLdsStride;

struct TileRows {
    int64_t slot0;
    int rows;  // valid rows in this tile (<= BM)
};

// One workgroup: rows [slot0, slot0 + rows) x columns [n0, n0 + 128), all K.
// Loader mapping (per group): thread t loads A row t/2, bytes (t&1)*64 + [0,64),
// and B column t/2, packed bytes (t&1)*32 + [0,32) (= codes (t&1)*64 + [0,64)).
// Wave w computes rows (w>>1)*64 + [0,64) x columns (w&1)*64 + [0,64) as 2x2
// 32x32 MFMA tiles; lane l of a 32x32 tile feeds A row (l&31) / B column (l&31)
// with k bytes ks*32 + (l>>5)*16 + [0,16), and holds accumulator rows
// 8*(r>>2) + 4*(l>>5) + (r&3), r = 0..15, of column l&31.
template <bool ISUMS>
__device__ __forceinline__ void tile_unit(uint8_t *lds, const int8_t *__restrict__ qa,
                                          const float *__restrict__ a_scale, const int32_t *__restrict__ row_index,
                                          int64_t R, TileRows rows, int64_t K, const uint8_t *__restrict__ wpk,
                                          const uint16_t *__restrict__ wsc, const uint16_t *__restrict__ wzp,
                                          int64_t N, int64_t n0, float *__restrict__ out, int64_t ldo,
                                          int32_t *__restrict__ isums, int64_t M_isums) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t G = K / G128;

    // ---- loader state
    const int lrow = tid >> 1, lpart = tid & 1;
    int64_t arow = -1;
    if (lrow < rows.rows) arow = row_index ? (int64_t)row_index[rows.slot0 + lrow] : rows.slot0 + lrow;
    const bool avalid = arow >= 0 && arow < R;
    const v4u *aglob = reinterpret_cast<const v4u *>(qa + (avalid ? arow : 0) * K + lpart * 64);
    const int64_t bcol = n0 + lrow;
    const bool bvalid = bcol < N;
    const v4u *bglob = reinterpret_cast<const v4u *>(wpk + (bvalid ? bcol : 0) * (K / 2) + lpart * 32);
    const uint16_t *zglob = wzp + (bvalid ? bcol : 0);

    v4u ra[4], rb[2];
    uint16_t rz = 0;
    auto gload = [&](int64_t g) {
        if (avalid) {
#pragma unroll
            for (int i = 0; i < 4; ++i) ra[i] = aglob[g * (G128 / 16) + i];
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) ra[i] = v4u{0u, 0u, 0u, 0u};
        }
        if (bvalid) {
            rb[0] = __builtin_nontemporal_load(bglob + g * (G128 / 2 / 16));
            rb[1] = __builtin_nontemporal_load(bglob + g * (G128 / 2 / 16) + 1);
            rz = zglob[g * N];
        } else {
            rb[0] = rb[1] = v4u{0u, 0u, 0u, 0u};
            rz = 0;
        }
    };
    auto lstore = [&](int buf) {
        uint8_t *A = lds + buf * 2 * kLdsTile;
        uint8_t *B = A + kLdsTile;
        v4u *ad = reinterpret_cast<v4u *>(A + lrow * kLdsStride + lpart * 64);
#pragma unroll
        for (int i = 0; i < 4; ++i) ad[i] = ra[i];
        const uint32_t zadd = zp_add_const(rz);
        uint32_t w[16];
        const uint32_t d[8] = {rb[0].x, rb[0].y, rb[0].z, rb[0].w, rb[1].x, rb[1].y, rb[1].z, rb[1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) unpack8(d[i], zadd, w[2 * i], w[2 * i + 1]);
        if (!bvalid) {
#pragma unroll
            for (int i = 0; i < 16; ++i) w[i] = 0;
        }
        v4u *bd = reinterpret_cast<v4u *>(B + lrow * kLdsStride + lpart * 64);
#pragma unroll
        for (int i = 0; i < 4; ++i) bd[i] = v4u{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
    };

    // ---- compute state
    float acc[2][2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int frow = lane & 31, fk = (lane >> 5) * 16;
    int64_t scol[2];
    bool svalid[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        scol[j] = n0 + wn * 64 + j * 32 + (lane & 31);
        svalid[j] = scol[j] < N;
    }

    gload(0);
    lstore(0);
    __syncthreads();

    for (int64_t g = 0; g < G; ++g) {
        const int buf = (int)(g & 1);
        if (g + 1 < G) gload(g + 1);
        float sc[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) sc[j] = svalid[j] ? half_bits_to_float(wsc[g * N + scol[j]]) : 0.0f;

        const uint8_t *A = lds + buf * 2 * kLdsTile;
        const uint8_t *B = A + kLdsTile;
        v16i d[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) d[i][j][r] = 0;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
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
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    if (ISUMS) {
                        const int m = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                        if (m < rows.rows && svalid[j])
                            isums[(g * M_isums + rows.slot0 + m) * N + scol[j]] = d[i][j][r];
                    } else {
                        acc[i][j][r] = fmaf(sc[j], (float)d[i][j][r], acc[i][j][r]);
                    }
                }
        if (g + 1 < G) lstore(buf ^ 1);
        __syncthreads();
    }

    if (!ISUMS) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m < rows.rows) {
                    const int64_t slot = rows.slot0 + m;
                    const int64_t row = row_index ? (int64_t)row_index[slot] : slot;
                    if (row >= 0 && row < R) {
                        const float as = a_scale[row];
#pragma unroll
                        for (int j = 0; j < 2; ++j)
                            if (svalid[j]) out[slot * ldo + scol[j]] = as * acc[i][j][r];
                    }
                }
            }
    }
}

template <bool ISUMS>
__global__ __launch_bounds__(kTileThreads, 2) void gemm_tiled_kernel(const int8_t *__restrict__ qa,
                                                                     const float *__restrict__ a_scale, int64_t M,
                                                                     int64_t K, const uint8_t *__restrict__ packed,
                                                                     const uint16_t *__restrict__ scale,
                                                                     const uint16_t *__restrict__ zp, int64_t N,
                                                                     float *__restrict__ out,
                                                                     int32_t *__restrict__ isums) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * 2 * kLdsTile];
    const int64_t mt = (M + BM - 1) / BM, nt = (N + BN - 1) / BN;
    const int64_t tile = xcd_tile(blockIdx.x, mt * nt);
    // m fastest inside an XCD's range: concurrently running tiles share weight columns
    const int64_t tm = tile % mt, tn = tile / mt;
    const int64_t m0 = tm * BM;
    const int rows = (int)((M - m0) < BM ? (M - m0) : BM);
    tile_unit<ISUMS>(lds, qa, a_scale, nullptr, M, TileRows{m0, rows}, K, packed, scale, zp, N, tn * BN, out, N, isums,
                     M);
}

// ------------------------------------------------------------------ expert-grouped forms
// Experts with at most kSmallRows slots take the streaming loop (one 64-row
// chunk, MT chosen from the count), larger experts the tiled loop.  Each
// workgroup reads expert_offsets itself and walks a persistent unit list, so
// the slot counts never travel to the host.
constexpr int kSmallRows = 64;
constexpr int kMaxExperts = 1024;

// Exclusive prefix over experts of units(e) into lds_pfx[0..E]; returns the
// total.  Run by the whole workgroup (nthreads = blockDim.x <= 256): thread t
// sums a contiguous run of experts, the runs are scanned with wave shuffles and
// one LDS step, then each thread writes its run's prefixes.
template <typename UnitsFn>
__device__ __forceinline__ int64_t expert_prefix(int32_t E, int64_t *lds_pfx, int nthreads, UnitsFn units) {
    __shared__ int64_t wave_tot[4];
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

__global__ __launch_bounds__(kStreamThreads) void grouped_stream_kernel(
    const int8_t *__restrict__ qa, const float *__restrict__ a_scale, int64_t R, const int32_t *__restrict__ row_index,
    const int32_t *__restrict__ offsets, int32_t E, int64_t K, const uint8_t *__restrict__ packed,
    const uint16_t *__restrict__ scale, const uint16_t *__restrict__ zp, int64_t N, int64_t max_slots,
    float *__restrict__ out) {
    __shared__ int64_t pfx[kMaxExperts + 1];
    const int64_t ntn = N / 16;
    const int64_t total = expert_prefix(E, pfx, kStreamThreads, [&](int e) -> int64_t {
        const int64_t c = clamp_slots(offsets[e + 1], max_slots) - clamp_slots(offsets[e], max_slots);
        return (c > 0 && c <= kSmallRows) ? ntn : 0;
    });
    const int64_t G = K / G128;
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
            stream_unit<1, 4, false>(qa, a_scale, row_index, R, sr, K, wp, ws, wz, N, tn * 16, out, N, nullptr, 0);
        else if (rows <= 32)
            stream_unit<2, 4, false>(qa, a_scale, row_index, R, sr, K, wp, ws, wz, N, tn * 16, out, N, nullptr, 0);
        else
            stream_unit<4, 2, false>(qa, a_scale, row_index, R, sr, K, wp, ws, wz, N, tn * 16, out, N, nullptr, 0);
    }
}

__global__ __launch_bounds__(kTileThreads, 2) void grouped_tiled_kernel(
    const int8_t *__restrict__ qa, const float *__restrict__ a_scale, int64_t R, const int32_t *__restrict__ row_index,
    const int32_t *__restrict__ offsets, int32_t E, int64_t K, const uint8_t *__restrict__ packed,
    const uint16_t *__restrict__ scale, const uint16_t *__restrict__ zp, int64_t N, int64_t max_slots,
    float *__restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * 2 * kLdsTile];
    __shared__ int64_t pfx[kMaxExperts + 1];
    const int64_t ntn = (N + BN - 1) / BN;
    const int64_t total = expert_prefix(E, pfx, kTileThreads, [&](int e) -> int64_t {
        const int64_t c = clamp_slots(offsets[e + 1], max_slots) - clamp_slots(offsets[e], max_slots);
        return c > kSmallRows ? ((c + BM - 1) / BM) * ntn : 0;
    });
    const int64_t G = K / G128;
    for (int64_t u = blockIdx.x; u < total; u += gridDim.x) {
        const int e = find_expert(pfx, E, u);
        const int64_t c = clamp_slots(offsets[e + 1], max_slots) - clamp_slots(offsets[e], max_slots);
        const int64_t mt = (c + BM - 1) / BM;
        const int64_t local = u - pfx[e];
        const int64_t tm = local % mt, tn = local / mt;
        const int64_t s0 = clamp_slots(offsets[e], max_slots) + tm * BM;
        const int rows = (int)((c - tm * BM) < BM ? (c - tm * BM) : BM);
        tile_unit<false>(lds, qa, a_scale, row_index, R, TileRows{s0, rows}, K, packed + (int64_t)e * N * (K / 2),
                         scale + (int64_t)e * G * N, zp + (int64_t)e * G * N, N, tn * BN, out, N, nullptr, 0);
        __syncthreads();  // the next unit reuses the LDS buffers
    }
}

}  // namespace

namespace w4a8 {

hipError_t launch_gemm(const int8_t *qa, const float *a_scale, int64_t M, int64_t K, const uint8_t *packed,
                       const uint16_t *scale, const uint16_t *zp, int64_t N, int path, float *out, int32_t *isums,
                       hipStream_t stream) {
    if (path == 1) {
        const dim3 grid((uint32_t)(N / 16)), block(kStreamThreads);
#define W4A8_STREAM(MT, U)                                                                                        \
    do {                                                                                                          \
        if (isums)                                                                                                \
            hipLaunchKernelGGL((gemm_stream_kernel<MT, U, true>), grid, block, 0, stream, qa, a_scale, M, K,      \
                               packed, scale, zp, N, out, isums);                                                 \
        else                                                                                                      \
            hipLaunchKernelGGL((gemm_stream_kernel<MT, U, false>), grid, block, 0, stream, qa, a_scale, M, K,     \
                               packed, scale, zp, N, out, isums);                                                 \
    } while (0)
        if (M <= 16) W4A8_STREAM(1, 8);
        else if (M <= 32) W4A8_STREAM(2, 4);
        else W4A8_STREAM(4, 2);
#undef W4A8_STREAM
    } else {
        const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
        const dim3 grid((uint32_t)tiles), block(kTileThreads);
        if (isums)
            hipLaunchKernelGGL(gemm_tiled_kernel<true>, grid, block, 0, stream, qa, a_scale, M, K, packed, scale, zp,
                               N, out, isums);
        else
            hipLaunchKernelGGL(gemm_tiled_kernel<false>, grid, block, 0, stream, qa, a_scale, M, K, packed, scale, zp,
                               N, out, isums);
    }
    return hipGetLastError();
}

hipError_t launch_grouped_gemm(const int8_t *qa, const float *a_scale, int64_t R, const int32_t *row_index,
                               const int32_t *expert_offsets, int32_t E, int64_t K, const uint8_t *packed,
                               const uint16_t *scale, const uint16_t *zp, int64_t N, int64_t max_slots, float *out,
                               hipStream_t stream) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return hipGetLastError();
    hipLaunchKernelGGL(grouped_stream_kernel, dim3((uint32_t)(cus * 8)), dim3(kStreamThreads), 0, stream, qa, a_scale,
                       R, row_index, expert_offsets, E, K, packed, scale, zp, N, max_slots, out);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(grouped_tiled_kernel, dim3((uint32_t)(cus * 2)), dim3(kTileThreads), 0, stream, qa, a_scale, R,
                       row_index, expert_offsets, E, K, packed, scale, zp, N, max_slots, out);
    return hipGetLastError();
}

}  // namespace w4a8
