// The top-k combine's slot-order sum, shared by the standalone combine
// kernel and the combine in the grouped GEMM's epilogue, so that both give
// the same bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode.h"

namespace nvfp4 {

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

}  // namespace nvfp4
