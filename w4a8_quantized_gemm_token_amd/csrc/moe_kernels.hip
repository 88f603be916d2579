// moe_kernels.hip -- routing, expert bucketing and the weighted combine.
//
// [p1 §5.2] (hotelren.com/news/5173946, "Kimi 2.7 MoE: from 4-bit storage to
// INT8 compute"): the router is kept in high precision and decides which
// experts each token visits; [p1 §5.1, §6.3]: unbalanced buckets must not
// degrade into many small matmuls -- the grouped GEMM therefore consumes the
// expert-sorted slot list built here straight from device memory.
// [p4] (feinterview.poetries.top, "MoE deployment: active parameters are not the
// storage bill"): the toy top-1 router over 8 experts.
//
//  * route_topk: one wave per token; each lane keeps E/64 logits in registers,
//    k rounds of a wave-wide (value, -id) arg-max (DPP within rows, scalar reads
//    across them) pick the experts in descending order (ties -> lower id), then a
//    softmax over the k picks, all without divergent branches.
//  * bucket: one workgroup; each wave counts the experts of its contiguous range
//    of pairs (LDS integer atomics), an exclusive scan over experts gives the
//    offsets and each wave's first slot per expert, then every wave places its
//    own pairs in increasing pair index (ballots over the expert id bits rank
//    lanes with the same expert) -- stable, deterministic, no atomics on
//    positions.
//  * route_bucket: both in one launch for batches of at most 16 tokens (the bucketing
//    workgroup's waves route one token each first).
//  * combine: out[t] = sum_j w[t][j] * y[slot(t, j)] + y_shared[t], float4 wide.
#include "w4a8_internal.hpp"

using namespace w4a8dev;

namespace {

constexpr int kMaxE = 1024;
constexpr int kMaxK = 8;
constexpr int kPerLane = kMaxE / kWave;  // 16

constexpr int kRouteThreads = 256;

// (v, i) beats (bv, bi): larger value, then lower id.  A lane with no candidate holds
// (-inf, INT_MAX), which every real candidate beats (non-NaN logits).
__device__ __forceinline__ void better_of(float ov, int oi, float &bv, int &bi) {
    const bool take = (ov > bv) | ((ov == bv) & (oi < bi));
    bv = take ? ov : bv;
    bi = take ? oi : bi;
}
template <int CTRL>
__device__ __forceinline__ void argmax_step(float &bv, int &bi) {
    const float ov = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, bv), CTRL, 0xF,
                                                                           0xF, false));
    const int oi = __builtin_amdgcn_update_dpp(0, bi, CTRL, 0xF, 0xF, false);
    better_of(ov, oi, bv, bi);
}

// One wave per token.  Lane l holds logits l, l + 64, ... (PER of them, PER * 64 >= E) and
// a bitmask of the ones already picked; each of the k rounds takes the lane-local best
// candidate with selects, then a wave-wide arg-max: DPP steps inside each 16-lane row
// (swap neighbours, swap pairs, rotate by 4 and by 8), then the four row winners read
// as scalars -- no LDS round trips, no branches.  Every lane ends up with all k picks;
// lane j writes pick j.
template <int PER>
__device__ __forceinline__ void route_token(const float *__restrict__ logits, int64_t t, int32_t E, int32_t k,
                                            int32_t *__restrict__ ids, float *__restrict__ w) {
    const int lane = threadIdx.x & 63;
    const float *row = logits + t * E;
    float v[PER];
    uint32_t taken = 0;  // bit i: logit i * 64 + lane already picked (or past E)
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = i * kWave + lane;
        const float x = row[e < E ? e : E - 1];
        v[i] = e < E ? x : -INFINITY;
        taken |= (e < E ? 0u : 1u) << i;
    }
    float sel_v[kMaxK];
    int sel_i[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        if (j >= k) break;
        float bv = -INFINITY;
        int bi = 0x7FFFFFFF;  // none yet
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = i * kWave + lane;
            const bool take = !((taken >> i) & 1u) & ((v[i] > bv) | ((v[i] == bv) & (e < bi)));
            bv = take ? v[i] : bv;
            bi = take ? e : bi;
        }
        argmax_step<0xB1>(bv, bi);   // quad_perm [1,0,3,2]
        argmax_step<0x4E>(bv, bi);   // quad_perm [2,3,0,1]
        argmax_step<0x124>(bv, bi);  // row_ror:4
        argmax_step<0x128>(bv, bi);  // row_ror:8
        const int ib = __builtin_bit_cast(int, bv);
        float rv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ib, 0));
        int ri = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
        for (int r = 1; r < 4; ++r)
            better_of(__builtin_bit_cast(float, __builtin_amdgcn_readlane(ib, 16 * r)),
                      __builtin_amdgcn_readlane(bi, 16 * r), rv, ri);
        sel_v[j] = rv;
        sel_i[j] = ri;
        taken |= ((ri & (kWave - 1)) == lane ? 1u : 0u) << ((ri / kWave) & 31);
    }
    // softmax over the picks, in pick order (the same sum on every lane)
    const float top = sel_v[0];
    float ex[kMaxK];
    float denom = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        if (j >= k) break;
        ex[j] = expf(sel_v[j] - top);
        denom += ex[j];
    }
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        if (j >= k) break;
        if (lane == j) {
            ids[t * k + j] = sel_i[j];
            w[t * k + j] = ex[j] / denom;
        }
    }
}

template <int PER>
__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(const float *__restrict__ logits, int64_t T,
                                                                   int32_t E, int32_t k, int32_t *__restrict__ ids,
                                                                   float *__restrict__ w) {
    const int64_t t = (int64_t)blockIdx.x * (kRouteThreads / kWave) + (threadIdx.x >> 6);
    if (t >= T) return;  // whole waves
    route_token<PER>(logits, t, E, k, ids, w);
}

constexpr int kBucketThreads = 1024;
constexpr int kBucketWaves = kBucketThreads / kWave;

// shared_T > 0 appends a shared expert (index E) whose T slots follow the routed
// ones: offsets[E+1] = P + T, and slot P + t reads activation row t.
//
// Wave w owns the contiguous pair range [w C, (w + 1) C), C = ceil(P / 16):
//  1. per-wave expert counts in LDS (integer atomics: the totals are exact);
//  2. offsets[e] = exclusive scan of the totals (wave scans, then the wave totals),
//     and the first slot of wave w's pairs of expert e = offsets[e] + the counts of
//     waves before w;
//  3. each wave walks its range 64 pairs at a time in increasing pair index: lanes
//     holding the same expert are found with ballots over the expert id bits, a lane's
//     slot is its expert's running slot plus its rank among those lanes, and the
//     lowest of them advances the running slot.
// Slots are therefore ordered by expert, then by pair index (stable), with no
// atomics on positions; four barriers in all.
// kBatch 64-pair chunks have their expert ids loaded together (their latencies overlap).
template <int kBatch>
__device__ __forceinline__ void bucket_pairs(const int32_t *__restrict__ ids, int64_t P, int32_t E, int32_t k,
                                             int64_t shared_T, int32_t *__restrict__ offsets,
                                             int32_t *__restrict__ perm, int32_t *__restrict__ slot_row,
                                             int32_t *__restrict__ slot_of_pair) {
    __shared__ int32_t hist[kBucketWaves][kMaxE];  // counts, then each wave's running slot
    __shared__ int32_t wave_sum[kBucketWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t C = (P + kBucketWaves - 1) / kBucketWaves;
    const int64_t p0 = wave * C, p1 = (p0 + C < P) ? p0 + C : P;

    for (int i = tid; i < kBucketWaves * kMaxE; i += kBucketThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
    for (int64_t c0 = p0; c0 < p1; c0 += kBatch * kWave) {
        int e[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int64_t p = c0 + j * kWave + lane;
            e[j] = p < p1 ? ids[p] : -1;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            if (e[j] >= 0) atomicAdd(&hist[wave][e[j]], 1);
    }
    __syncthreads();

    // exclusive scan over experts of the totals (one expert per thread, E <= 1024)
    int32_t total = 0;
    if (tid < E)
        for (int w2 = 0; w2 < kBucketWaves; ++w2) total += hist[w2][tid];
    int32_t incl = total;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int32_t o = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += o;
    }
    if (lane == kWave - 1) wave_sum[wave] = incl;
    __syncthreads();
    int32_t before = 0;
    for (int w2 = 0; w2 < wave; ++w2) before += wave_sum[w2];
    if (tid < E) {
        int32_t run = before + incl - total;  // offsets[tid]
        offsets[tid] = run;
        for (int w2 = 0; w2 < kBucketWaves; ++w2) {
            const int32_t c = hist[w2][tid];
            hist[w2][tid] = run;
            run += c;
        }
    }
    if (tid == kBucketThreads - 1) {
        const int32_t all = before + incl;  // the last thread's inclusive sum covers every expert
        offsets[E] = all;
        if (shared_T > 0) offsets[E + 1] = all + (int32_t)shared_T;
    }
    __syncthreads();

    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int64_t b0 = p0; b0 < p1; b0 += kBatch * kWave) {
        int eb[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int64_t p = b0 + j * kWave + lane;
            eb[j] = p < p1 ? ids[p] : 0;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (b0 + j * kWave >= p1) break;  // wave-uniform: no pairs left in this range
            const int64_t p = b0 + j * kWave + lane;
            const bool valid = p < p1;
            const int e = eb[j];
            uint64_t peers = __ballot(valid);
            for (int b = 0; b < nbits; ++b) {
                const uint64_t bit = __ballot(valid && ((e >> b) & 1));
                peers &= ((e >> b) & 1) ? bit : ~bit;
            }
            const int rank = __popcll(peers & lt_mask);
            const int32_t start = valid ? hist[wave][e] : 0;  // all lanes read before any lane writes
            if (valid) {
                const int32_t slot = start + rank;
                perm[slot] = (int32_t)p;
                slot_of_pair[p] = slot;
                if (slot_row) slot_row[slot] = (int32_t)(p / k);
            }
            if (valid && rank == 0) hist[wave][e] = start + __popcll(peers);
        }
    }
    if (slot_row)
        for (int64_t t = tid; t < shared_T; t += kBucketThreads) slot_row[P + t] = (int32_t)t;
}

template <int kBatch>
__global__ __launch_bounds__(kBucketThreads) void bucket_kernel(const int32_t *__restrict__ ids, int64_t P, int32_t E,
                                                                int32_t k, int64_t shared_T,
                                                                int32_t *__restrict__ offsets,
                                                                int32_t *__restrict__ perm,
                                                                int32_t *__restrict__ slot_row,
                                                                int32_t *__restrict__ slot_of_pair) {
    bucket_pairs<kBatch>(ids, P, E, k, shared_T, offsets, perm, slot_row, slot_of_pair);
}

// Routing and bucketing of a small batch (T <= kFusedRouteT, at most one token per wave) in
// one workgroup: wave w routes token w, and after a barrier -- which also makes the waves'
// writes of ids visible to the whole workgroup -- the same workgroup buckets the pairs.  One
// launch instead of two; the tables are the same bits.  (With four tokens per wave, at T = 64,
// the one CU's serial routing cost more than the launch it saves.)
constexpr int64_t kFusedRouteT = 16;
template <int PER>
__global__ __launch_bounds__(kBucketThreads) void route_bucket_kernel(const float *__restrict__ logits, int64_t T,
                                                                      int32_t E, int32_t k, int32_t *__restrict__ ids,
                                                                      float *__restrict__ w, int64_t shared_T,
                                                                      int32_t *__restrict__ offsets,
                                                                      int32_t *__restrict__ perm,
                                                                      int32_t *__restrict__ slot_row,
                                                                      int32_t *__restrict__ slot_of_pair) {
    for (int64_t t = threadIdx.x >> 6; t < T; t += kBucketWaves) route_token<PER>(logits, t, E, k, ids, w);
    __syncthreads();
    bucket_pairs<1>(ids, T * k, E, k, shared_T, offsets, perm, slot_row, slot_of_pair);
}

constexpr int kCombineThreads = 256;
// grid: (T, ceil(H/4 / 256)); each thread one float4 of one token row
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const float *__restrict__ y,
                                                                  const int32_t *__restrict__ slot_of_pair,
                                                                  const float *__restrict__ topk_w,
                                                                  const float *__restrict__ y_shared, int32_t k,
                                                                  int64_t H, float *__restrict__ out) {
    const int64_t t = blockIdx.x;
    const int64_t c4 = (int64_t)blockIdx.y * kCombineThreads + threadIdx.x;
    if (c4 * 4 >= H) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    // eight routed rows at a time, every load issued before the multiply-adds (in j order)
    for (int j0 = 0; j0 < k; j0 += 8) {
        float4 v[8];
        float wv[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            if (j0 + jj < k) {
                wv[jj] = topk_w[t * k + j0 + jj];
                v[jj] = reinterpret_cast<const float4 *>(y + (int64_t)slot_of_pair[t * k + j0 + jj] * H)[c4];
            }
        }
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            if (j0 + jj < k) {
                acc.x = fmaf(wv[jj], v[jj].x, acc.x);
                acc.y = fmaf(wv[jj], v[jj].y, acc.y);
                acc.z = fmaf(wv[jj], v[jj].z, acc.z);
                acc.w = fmaf(wv[jj], v[jj].w, acc.w);
            }
        }
    }
    if (y_shared) {
        const float4 v = reinterpret_cast<const float4 *>(y_shared + t * H)[c4];
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    reinterpret_cast<float4 *>(out + t * H)[c4] = acc;
}

}  // namespace

namespace w4a8 {

hipError_t launch_moe_route(const float *logits, int64_t T, int32_t E, int32_t topk, int32_t with_shared, int32_t *ids,
                            float *w, int32_t *offsets, int32_t *perm, int32_t *slot_row, int32_t *slot_of_pair,
                            hipStream_t stream) {
    const int64_t shared_f = with_shared ? T : (int64_t)0;
    if (T > 0 && T <= kFusedRouteT && T * topk <= (int64_t)kBucketThreads) {
        const int per = (E + kWave - 1) / kWave;
#define W4A8_RB(PP)                                                                                                 \
    hipLaunchKernelGGL(route_bucket_kernel<PP>, dim3(1), dim3(kBucketThreads), 0, stream, logits, T, E, topk, ids, w, \
                       shared_f, offsets, perm, slot_row, slot_of_pair)
        if (per <= 1) W4A8_RB(1);
        else if (per <= 2) W4A8_RB(2);
        else if (per <= 4) W4A8_RB(4);
        else if (per <= 8) W4A8_RB(8);
        else W4A8_RB(kPerLane);
#undef W4A8_RB
        return hipGetLastError();
    }
    if (T > 0) {
        const dim3 grid((uint32_t)((T + kRouteThreads / kWave - 1) / (kRouteThreads / kWave))), block(kRouteThreads);
        const int per = (E + kWave - 1) / kWave;  // logits per lane, rounded up to a power of two
        if (per <= 1) hipLaunchKernelGGL(route_topk_kernel<1>, grid, block, 0, stream, logits, T, E, topk, ids, w);
        else if (per <= 2) hipLaunchKernelGGL(route_topk_kernel<2>, grid, block, 0, stream, logits, T, E, topk, ids, w);
        else if (per <= 4) hipLaunchKernelGGL(route_topk_kernel<4>, grid, block, 0, stream, logits, T, E, topk, ids, w);
        else if (per <= 8) hipLaunchKernelGGL(route_topk_kernel<8>, grid, block, 0, stream, logits, T, E, topk, ids, w);
        else hipLaunchKernelGGL(route_topk_kernel<kPerLane>, grid, block, 0, stream, logits, T, E, topk, ids, w);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    // one chunk per wave for small batches, eight chunks' ids in flight for large ones
    const int64_t P = T * topk, shared = with_shared ? T : (int64_t)0;
    if (P <= (int64_t)kBucketThreads)
        hipLaunchKernelGGL(bucket_kernel<1>, dim3(1), dim3(kBucketThreads), 0, stream, ids, P, E, topk, shared, offsets,
                           perm, slot_row, slot_of_pair);
    else
        hipLaunchKernelGGL(bucket_kernel<8>, dim3(1), dim3(kBucketThreads), 0, stream, ids, P, E, topk, shared, offsets,
                           perm, slot_row, slot_of_pair);
    return hipGetLastError();
}

hipError_t launch_moe_combine(const float *y, const int32_t *slot_of_pair, const float *topk_w, const float *y_shared,
                              int64_t T, int32_t topk, int64_t H, float *out, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int64_t c4 = H / 4;
    const dim3 grid((uint32_t)T, (uint32_t)((c4 + kCombineThreads - 1) / kCombineThreads));
    hipLaunchKernelGGL(combine_kernel, grid, dim3(kCombineThreads), 0, stream, y, slot_of_pair, topk_w, y_shared, topk,
                       H, out);
    return hipGetLastError();
}

}  // namespace w4a8
