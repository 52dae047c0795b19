// MoE glue around the grouped GEMM: routing (expert offsets and the grouped
// row order), the gated activation between FC1 and FC2, and the top-k
// weighted combine back to token order.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode.h"

namespace nvfp4 {

constexpr int kRouteThreads = 1024;                 // pairs per workgroup
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kRouteMaxExperts = kRouteThreads;     // one expert per thread in the scans

// Routing of P = T k (token, slot) pairs, pair p = t k + j choosing expert
// ids[p].  Grouped rows are the pairs sorted by expert, ties kept in pair
// order (a stable sort), so the result does not depend on timing:
//   offsets[e]     = number of pairs with an expert below e (offsets[E] = P),
//   row_token[r]   = token of grouped row r,
//   token_row[p]   = grouped row of pair p.
// Launches over blocks of kRouteThreads pairs (block b: pairs
// 1024 b .. 1024 b + 1023, wave w of its workgroup: 64 of them; one block
// is one launch of place alone, up to kRouteRawBlocks blocks count + place
// with the scan done inside place):
//   count  - per block and expert, the number of pairs (hist[b][e]);
//   scan   - offsets, and each block's first row per expert
//            (hist[b][e] = offsets[e] + the pairs of e in blocks before b);
//   place  - a pair's row is its block's first row for its expert, plus the
//            pairs of that expert in the earlier waves of the block, plus its
//            rank among the equal-expert lanes of its wave.
// A wave finds the lanes holding the same expert as each lane with one
// ballot per expert bit; the lowest such lane speaks for the group.  Ids
// outside [0, E) are clamped for addressing only (the result is then
// meaningless, but every access stays in bounds).
struct RouteMatch {
    int e;           // the lane's expert (clamped; 0 past the end)
    uint64_t same;   // lanes of the wave with the same expert (0 past the end)
    int rank;        // lanes of the group below this one
};

__device__ __forceinline__ RouteMatch route_match(const int32_t* __restrict__ ids, int64_t p, int64_t P, int E) {
    const int lane = threadIdx.x & 63;
    const bool valid = p < P;
    const int v = valid ? ids[p] : 0;
    RouteMatch m;
    m.e = v < 0 ? 0 : (v >= E ? E - 1 : v);
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const uint64_t ones = __ballot(valid && ((m.e >> b) & 1));
        same &= ((m.e >> b) & 1) ? ones : ~ones;
    }
    m.same = valid ? same : 0ull;
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    m.rank = __popcll(m.same & below);
    return m;
}

__global__ void __launch_bounds__(kRouteThreads) k_moe_route_count(const int32_t* __restrict__ ids, int64_t P, int E,
                                                                    int32_t* __restrict__ hist) {
    __shared__ int cnt[kRouteMaxExperts];
    const int tid = threadIdx.x;
    if (tid < E) cnt[tid] = 0;
    __syncthreads();
    const RouteMatch m = route_match(ids, (int64_t)blockIdx.x * kRouteThreads + tid, P, E);
    if (m.same != 0 && m.rank == 0) atomicAdd(&cnt[m.e], __popcll(m.same));   // a sum: order-free
    __syncthreads();
    if (tid < E) hist[(int64_t)blockIdx.x * E + tid] = cnt[tid];
}

// Exclusive scan over the experts of a per-expert value held by thread e
// (e < E <= kRouteThreads), for the whole workgroup.
__device__ __forceinline__ int route_block_scan(int v_in, int* wsum) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int v = v_in;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(v, d);
        if (lane >= d) v += t;
    }
    if (lane == 63) wsum[w] = v;
    __syncthreads();
    int before = 0;
    for (int i = 0; i < w; ++i) before += wsum[i];
    return before + v - v_in;
}

__global__ void __launch_bounds__(kRouteThreads) k_moe_route_scan(int32_t* __restrict__ hist, int64_t blocks, int E,
                                                                   int64_t P, int32_t* __restrict__ offsets) {
    __shared__ int wsum[kRouteWaves];
    const int tid = threadIdx.x;
    // expert tid: the pairs of blocks before b, in place (16 blocks' loads in
    // flight at a time); then its total
    constexpr int kBatch = 16;
    int total = 0;
    if (tid < E) {
        for (int64_t b0 = 0; b0 < blocks; b0 += kBatch) {
            int c[kBatch];
#pragma unroll
            for (int i = 0; i < kBatch; ++i) c[i] = b0 + i < blocks ? hist[(b0 + i) * E + tid] : 0;
#pragma unroll
            for (int i = 0; i < kBatch; ++i) {
                if (b0 + i < blocks) hist[(b0 + i) * E + tid] = total;
                total += c[i];
            }
        }
    }
    const int first = route_block_scan(total, wsum);
    if (tid < E) {
        offsets[tid] = first;
        for (int64_t b = 0; b < blocks; ++b) hist[b * E + tid] += first;
    }
    if (tid == 0) offsets[E] = (int)P;
}

// hist == NULL: a single block (P <= kRouteThreads) that also derives the
// offsets from its own counts, so routing takes one launch.  raw_blocks > 0:
// hist holds the raw per-block counts of the raw_blocks blocks (no scan
// launch); every workgroup sums them per expert itself (at most
// kRouteRawBlocks loads per expert thread), scans the totals into the
// offsets (workgroup 0 stores them) and adds the counts of the blocks before
// its own.  Otherwise hist holds each block's first row per expert.
constexpr int kRouteRawBlocks = 32;
__global__ void __launch_bounds__(kRouteThreads) k_moe_route_place(const int32_t* __restrict__ ids, int64_t P, int E,
                                                                    const int32_t* __restrict__ hist,
                                                                    int32_t* __restrict__ row_token,
                                                                    int32_t* __restrict__ token_row, int k,
                                                                    int32_t* __restrict__ offsets,
                                                                    int raw_blocks = 0) {
    __shared__ int cnt[kRouteWaves * kRouteMaxExperts];   // [wave][expert], row stride E
    __shared__ int wsum[kRouteWaves];
    const int tid = threadIdx.x, w = tid >> 6;
    for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) cnt[i] = 0;
    __syncthreads();
    const int64_t p = (int64_t)blockIdx.x * kRouteThreads + tid;
    const RouteMatch m = route_match(ids, p, P, E);
    if (m.same != 0 && m.rank == 0) cnt[w * E + m.e] = __popcll(m.same);   // the lowest lane of each group
    __syncthreads();
    // expert tid: each wave's first row, in place
    int c[kRouteWaves];
    int total = 0;
    if (tid < E) {
#pragma unroll
        for (int ww = 0; ww < kRouteWaves; ++ww) {
            c[ww] = cnt[ww * E + tid];
            total += c[ww];
        }
    }
    int first = 0;
    if (hist == nullptr) {   // single block: the offsets are the scan of its own counts
        first = route_block_scan(tid < E ? total : 0, wsum);
        if (tid < E) offsets[tid] = first;
        if (tid == 0) offsets[E] = (int)P;
    } else if (raw_blocks > 0) {
        // expert tid: its total over all blocks and over the blocks before this one
        int all = 0, before = 0;
        if (tid < E) {
            int c2[kRouteRawBlocks];
#pragma unroll
            for (int b = 0; b < kRouteRawBlocks; ++b) c2[b] = b < raw_blocks ? hist[(int64_t)b * E + tid] : 0;
#pragma unroll
            for (int b = 0; b < kRouteRawBlocks; ++b) {
                all += c2[b];
                before += b < (int)blockIdx.x ? c2[b] : 0;
            }
        }
        const int off_e = route_block_scan(tid < E ? all : 0, wsum);
        if (blockIdx.x == 0) {
            if (tid < E) offsets[tid] = off_e;
            if (tid == 0) offsets[E] = (int)P;
        }
        first = off_e + before;
    }
    if (tid < E) {
        int run = (hist && raw_blocks == 0) ? hist[(int64_t)blockIdx.x * E + tid] : first;
#pragma unroll
        for (int ww = 0; ww < kRouteWaves; ++ww) {
            cnt[ww * E + tid] = run;
            run += c[ww];
        }
    }
    __syncthreads();
    if (m.same != 0) {
        const int row = cnt[w * E + m.e] + m.rank;
        row_token[row] = (int32_t)((int)p / k);
        token_row[p] = row;
    }
}

// The elementwise steps take bf16, or fp16 with F16 (inputs and output).
//
// Gated SiLU: a[r, i] = RNE_bf16(silu(gate) * up) with gate = h[r, i] and
// up = h[r, I + i], silu(v) = v / (1 + e^-v), in fp32.  Thread: 8 columns,
// moved with 16-byte loads and stores when VEC (the host checks that every
// row start and I keep 16-byte alignment).
template <bool F16>
__device__ __forceinline__ uint32_t silu_mul_pair(uint32_t g2, uint32_t u2) {
    const float g0 = act_to_f32<F16>(g2 & 0xFFFFu), g1 = act_to_f32<F16>(g2 >> 16);
    const float u0 = act_to_f32<F16>(u2 & 0xFFFFu), u1 = act_to_f32<F16>(u2 >> 16);
    return round_out<F16>(silu_times(g0, u0)) | (round_out<F16>(silu_times(g1, u1)) << 16);
}

template <bool VEC, bool F16 = false>
__global__ void k_moe_silu_mul(const uint16_t* __restrict__ h, int64_t ld_h, int64_t R, int64_t I,
                               uint16_t* __restrict__ a, int64_t ld_a) {
    const int64_t per_row = (I + 7) / 8;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= R * per_row) return;
    const int64_t r = idx / per_row, i0 = (idx % per_row) * 8;
    const uint16_t* hr = h + r * ld_h;
    uint16_t* ar = a + r * ld_a;
    if (VEC && i0 + 8 <= I) {
        const uint4 g = *reinterpret_cast<const uint4*>(hr + i0), u = *reinterpret_cast<const uint4*>(hr + I + i0);
        *reinterpret_cast<uint4*>(ar + i0) =
            make_uint4(silu_mul_pair<F16>(g.x, u.x), silu_mul_pair<F16>(g.y, u.y), silu_mul_pair<F16>(g.z, u.z),
                       silu_mul_pair<F16>(g.w, u.w));
        return;
    }
    for (int e = 0; e < 8 && i0 + e < I; ++e)
        ar[i0 + e] = (uint16_t)(silu_mul_pair<F16>(hr[i0 + e], hr[I + i0 + e]) & 0xFFFFu);
}

// Non-gated squared ReLU: a[r, i] = RNE_bf16(max(h[r, i], 0)^2) in fp32.
// Thread: 8 columns, 16-byte loads and stores when VEC.
template <bool F16>
__device__ __forceinline__ uint32_t relu2_pair(uint32_t h2) {
    return round_out<F16>(relu_squared(act_to_f32<F16>(h2 & 0xFFFFu))) |
           (round_out<F16>(relu_squared(act_to_f32<F16>(h2 >> 16))) << 16);
}

template <bool VEC, bool F16 = false>
__global__ void k_moe_relu2(const uint16_t* __restrict__ h, int64_t ld_h, int64_t R, int64_t I,
                            uint16_t* __restrict__ a, int64_t ld_a) {
    const int64_t per_row = (I + 7) / 8;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= R * per_row) return;
    const int64_t r = idx / per_row, i0 = (idx % per_row) * 8;
    const uint16_t* hr = h + r * ld_h;
    uint16_t* ar = a + r * ld_a;
    if (VEC && i0 + 8 <= I) {
        const uint4 v = *reinterpret_cast<const uint4*>(hr + i0);
        *reinterpret_cast<uint4*>(ar + i0) =
            make_uint4(relu2_pair<F16>(v.x), relu2_pair<F16>(v.y), relu2_pair<F16>(v.z), relu2_pair<F16>(v.w));
        return;
    }
    for (int e = 0; e < 8 && i0 + e < I; ++e) ar[i0 + e] = (uint16_t)(relu2_pair<F16>(hr[i0 + e]) & 0xFFFFu);
}

// Slot order of the top-k combine: acc[c] = fma(w_j, y_j[c], acc[c]) for
// j = 0 .. k - 1 from 0, over 8 columns.  The slots are taken 8 at a time:
// their rows and weights are loaded first, then every row's 8 values (LOAD8
// returns them as 4 words, two values each), so that a chunk costs two
// memory latencies instead of two per slot.
template <bool F16, typename Load8>
__device__ __forceinline__ void combine_slots(const int32_t* token_row, const float* wt, int64_t pair0, int k,
                                              Load8 load8, float (&acc)[8]) {
    for (int j0 = 0; j0 < k; j0 += 8) {
        int row[8];
        float wj[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bool v = j0 + i < k;
            row[i] = v ? token_row[pair0 + j0 + i] : 0;
            wj[i] = v ? wt[pair0 + j0 + i] : 0.f;
        }
        uint4 d[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (j0 + i < k) d[i] = load8(row[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (j0 + i >= k) break;
            const uint32_t w4[4] = {d[i].x, d[i].y, d[i].z, d[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] = __builtin_fmaf(wj[i], act_to_f32<F16>(w4[e] & 0xFFFFu), acc[2 * e]);
                acc[2 * e + 1] = __builtin_fmaf(wj[i], act_to_f32<F16>(w4[e] >> 16), acc[2 * e + 1]);
            }
        }
    }
}

// 8 combined values to out (16-byte store when aligned and whole).
template <bool F16>
__device__ __forceinline__ void combine_store(uint16_t* o, int64_t n, int64_t N, const float (&acc)[8]) {
    if (n + 8 <= N && (reinterpret_cast<uintptr_t>(o) & 15) == 0) {
        uint32_t p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            p[e] = round_out<F16>(fp32_value(acc[2 * e])) | (round_out<F16>(fp32_value(acc[2 * e + 1])) << 16);
        *reinterpret_cast<uint4*>(o) = make_uint4(p[0], p[1], p[2], p[3]);
        return;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (n + e < N) o[e] = (uint16_t)round_out<F16>(fp32_value(acc[e]));
}

// Top-k weighted combine: out[t, c] = RNE_bf16(sum_j wt[t, j] * y[token_row[t k + j], c]),
// summed in fp32 in slot order j = 0 .. k - 1.  Thread: 8 columns, 16-byte
// loads and stores when VEC.
template <bool VEC, bool F16 = false>
__global__ void k_moe_combine(const uint16_t* __restrict__ y, int64_t ld_y, const int32_t* __restrict__ token_row,
                              const float* __restrict__ wt, int64_t T, int k, int64_t H, uint16_t* __restrict__ out,
                              int64_t ld_o) {
    const int64_t per_row = (H + 7) / 8;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= T * per_row) return;
    const int64_t t = idx / per_row, c0 = (idx % per_row) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (VEC && c0 + 8 <= H) {
        combine_slots<F16>(token_row, wt, t * k, k, [&](int row) {
            return *reinterpret_cast<const uint4*>(y + (int64_t)row * ld_y + c0);
        }, acc);
    } else {
        combine_slots<F16>(token_row, wt, t * k, k, [&](int row) {
            const uint16_t* yr = y + (int64_t)row * ld_y + c0;
            uint32_t v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = c0 + e < H ? yr[e] : 0u;
            return make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16));
        }, acc);
    }
    combine_store<F16>(out + t * ld_o + c0, c0, H, acc);
}

}  // namespace nvfp4
