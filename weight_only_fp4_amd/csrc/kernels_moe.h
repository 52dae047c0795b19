// MoE glue around the grouped GEMM: routing (expert offsets and the grouped
// row order), the gated activation between FC1 and FC2, and the top-k
// weighted combine back to token order.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode.h"

namespace nvfp4 {

constexpr int kRouteThreads = 1024;          // one workgroup
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kRouteMaxExperts = 1024;       // LDS: per-wave count table of kRouteWaves x E

// Routing of P = T k (token, slot) pairs, pair p = t k + j choosing expert
// ids[p].  Grouped rows are the pairs sorted by expert, ties kept in pair
// order (a stable sort), so the result does not depend on timing:
//   offsets[e]     = number of pairs with an expert below e (offsets[E] = P),
//   row_token[r]   = token of grouped row r,
//   token_row[p]   = grouped row of pair p.
// One workgroup: the pairs are counted with LDS atomics (a sum, order-free),
// the counts scanned, then the pairs are placed in rounds of 1024: each wave
// ranks its 64 pairs among equal experts with ballots over the expert bits,
// and a wave's pairs follow those of the earlier waves of the round and of
// earlier rounds.  Ids outside [0, E) are clamped for addressing only (the
// result is then meaningless, but every access stays in bounds).
__global__ void __launch_bounds__(kRouteThreads) k_moe_route(const int32_t* __restrict__ ids, int64_t P, int E,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ row_token,
                                                              int32_t* __restrict__ token_row, int k) {
    __shared__ int cnt[kRouteWaves][kRouteMaxExperts];
    __shared__ int running[kRouteMaxExperts + 1];
    __shared__ int wsum[kRouteWaves];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    auto expert = [&](int64_t p) {
        const int e = ids[p];
        return e < 0 ? 0 : (e >= E ? E - 1 : e);
    };

    // ---- counts and their exclusive scan
    for (int e = tid; e < E; e += kRouteThreads) running[e] = 0;
    __syncthreads();
    for (int64_t p = tid; p < P; p += kRouteThreads) atomicAdd(&running[expert(p)], 1);
    __syncthreads();
    {
        // each thread scans a contiguous run of experts, then the runs' totals are scanned
        constexpr int kPer = kRouteMaxExperts / kRouteThreads > 0 ? kRouteMaxExperts / kRouteThreads : 1;
        const int e0 = tid * kPer;
        int local[kPer];
        int sum = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            local[i] = e0 + i < E ? running[e0 + i] : 0;
            sum += local[i];
        }
        // inclusive scan of the per-thread sums: within the wave, then across waves
        int v = sum;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int t = __shfl_up(v, d);
            if (lane >= d) v += t;
        }
        if (lane == 63) wsum[w] = v;
        __syncthreads();
        int before = 0;
        for (int i = 0; i < w; ++i) before += wsum[i];
        int run = before + v - sum;   // exclusive prefix of this thread's run
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            if (e0 + i < E) {
                running[e0 + i] = run;
                offsets[e0 + i] = run;
            }
            run += local[i];
        }
        if (tid == kRouteThreads - 1) offsets[E] = (int)P;
    }
    __syncthreads();

    // ---- stable placement, 1024 pairs per round
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    for (int64_t base = 0; base < P; base += kRouteThreads) {
        for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) cnt[i / E][i % E] = 0;
        __syncthreads();
        const int64_t p = base + tid;
        const bool valid = p < P;
        const int e = valid ? expert(p) : 0;
        uint64_t same = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const uint64_t ones = __ballot(valid && ((e >> b) & 1));
            same &= ((e >> b) & 1) ? ones : ~ones;
        }
        const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
        const int rank = __popcll(same & below);
        if (valid && rank == 0) cnt[w][e] = __popcll(same);   // the lowest lane of each expert group
        __syncthreads();
        if (valid) {
            int row = running[e] + rank;
            for (int ww = 0; ww < w; ++ww) row += cnt[ww][e];
            row_token[row] = (int32_t)(p / k);
            token_row[p] = row;
        }
        __syncthreads();
        for (int ee = tid; ee < E; ee += kRouteThreads) {
            int add = 0;
            for (int ww = 0; ww < kRouteWaves; ++ww) add += cnt[ww][ee];
            running[ee] += add;
        }
        __syncthreads();
    }
}

// Gated SiLU: a[r, i] = RNE_bf16(silu(gate) * up) with gate = h[r, i] and
// up = h[r, I + i], silu(v) = v / (1 + e^-v), in fp32.  Thread: 8 columns.
__global__ void k_moe_silu_mul(const uint16_t* __restrict__ h, int64_t ld_h, int64_t R, int64_t I,
                               uint16_t* __restrict__ a, int64_t ld_a) {
    const int64_t per_row = (I + 7) / 8;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= R * per_row) return;
    const int64_t r = idx / per_row, i0 = (idx % per_row) * 8;
    const uint16_t* hr = h + r * ld_h;
    uint16_t* ar = a + r * ld_a;
    for (int e = 0; e < 8 && i0 + e < I; ++e) {
        const float g = bf16_to_f32(hr[i0 + e]), u = bf16_to_f32(hr[I + i0 + e]);
        const float sg = g / (1.0f + expf(-g));
        ar[i0 + e] = (uint16_t)f32_to_bf16_rne(sg * u);
    }
}

// Top-k weighted combine: out[t, c] = RNE_bf16(sum_j wt[t, j] * y[token_row[t k + j], c]),
// summed in fp32 in slot order j = 0 .. k - 1.  Thread: 8 columns.
__global__ void k_moe_combine(const uint16_t* __restrict__ y, int64_t ld_y, const int32_t* __restrict__ token_row,
                              const float* __restrict__ wt, int64_t T, int k, int64_t H, uint16_t* __restrict__ out,
                              int64_t ld_o) {
    const int64_t per_row = (H + 7) / 8;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= T * per_row) return;
    const int64_t t = idx / per_row, c0 = (idx % per_row) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
        const float wj = wt[t * k + j];
        const uint16_t* yr = y + (int64_t)token_row[t * k + j] * ld_y;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (c0 + e < H) acc[e] = __builtin_fmaf(wj, bf16_to_f32(yr[c0 + e]), acc[e]);
    }
    uint16_t* orow = out + t * ld_o;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (c0 + e < H) orow[c0 + e] = (uint16_t)f32_to_bf16_rne(acc[e]);
}

}  // namespace nvfp4
