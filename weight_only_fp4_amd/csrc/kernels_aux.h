// Repack and dequantise (test export) kernels.
#pragma once
#include "decode.h"
#include "layout.h"

namespace nvfp4 {

// One thread per (expert, row unit, K chunk, lane): gathers the 16 canonical
// code bytes and the 2 scale bytes the lane owns in the repacked layout and
// writes them with one 128-bit and one 16-bit store.  Positions past N or K
// are written as zero.  mx: the scales are E8M0 bytes, one per 32 K (ld_s >=
// K / 32); the lane's 32-wide K group is one MXFP4 group and both of its
// scale bytes take that group's byte.
// gate_I > 0: a gated FC1 weight (N = 2 gate_I rows, gate_I a multiple of 16)
// is laid out with its 16-row units alternating gate / up for the gated
// epilogue: blob row 32 j + c (c < 16) is gate row 16 j + c and blob row
// 32 j + 16 + c the matching up row.  In the canonical input the gate rows
// come first (rows [0, I)) unless up_first, which puts the up rows there.
__global__ void __launch_bounds__(256) k_repack(const uint8_t* __restrict__ w, int64_t ld_w,
                                                const uint8_t* __restrict__ s, int64_t ld_s,
                                                int64_t N, int64_t K, int64_t NU, int64_t KC, int64_t total_lanes,
                                                BlobView v, uint8_t* __restrict__ codes_out,
                                                uint8_t* __restrict__ scales_out, int mx, int64_t gate_I,
                                                int up_first) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= total_lanes) return;
    const int lane = (int)(t & 63);
    const int64_t idx = t >> 6;              // (e * NU + u) * KC + c
    const int64_t c = idx % KC;
    const int64_t eu = idx / KC;
    const int64_t u = eu % NU;
    const int64_t e = eu / NU;
    const int64_t blk = v.block(e, u, c);
    const int64_t n = u * kUnitN + (lane & 15);
    const int64_t kbyte0 = c * (kChunkK / 2) + (lane >> 4) * 16;   // canonical byte of the lane's first code
    const int64_t kbytes = K / 2;
    uint32_t q[4] = {0u, 0u, 0u, 0u};
    uint32_t sc = 0u;
    if (n < N) {
        // canonical row of blob row n
        const int64_t half = (n >> 4) & 1;                           // 0: gate unit, 1: up unit
        const int64_t src = gate_I > 0 ? (half ^ (int64_t)up_first) * gate_I + (n >> 5) * kUnitN + (n & 15) : n;
        const uint8_t* row = w + (e * N + src) * ld_w;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t j = kbyte0 + i;
            const uint32_t b = (j < kbytes) ? (uint32_t)row[j] : 0u;
            q[i >> 2] |= b << (8 * (i & 3));
        }
        const uint8_t* srow = s + (e * N + src) * ld_s;
        if (mx) {
            const int64_t sb = c * (kChunkK / 32) + (lane >> 4);
            const uint32_t s0 = (sb < K / 32) ? (uint32_t)srow[sb] : 0u;
            sc = s0 | (s0 << 8);
        } else {
            const int64_t sb0 = c * (kChunkK / 16) + (lane >> 4) * 2;
            const int64_t nblk = K / 16;
            const uint32_t s0 = (sb0 < nblk) ? (uint32_t)srow[sb0] : 0u;
            const uint32_t s1 = (sb0 + 1 < nblk) ? (uint32_t)srow[sb0 + 1] : 0u;
            sc = s0 | (s1 << 8);
        }
    }
    *reinterpret_cast<uint4*>(codes_out + blk * kCodeBlock + lane * 16) = make_uint4(q[0], q[1], q[2], q[3]);
    *reinterpret_cast<uint16_t*>(scales_out + blk * kScaleBlock + lane * 2) = (uint16_t)sc;
}

// Decode a repacked blob to bf16 [E][N][ld_out] with the GEMM kernels' decode
// (decode8_bf16; E4M3 or, with v.mx, E8M0 scales).  One thread per (expert, row unit, K chunk, lane).
__global__ void __launch_bounds__(256) k_dequant(BlobView v, int64_t N, int64_t K, int64_t NU, int64_t KC,
                                                 int64_t total_lanes, uint16_t* __restrict__ out, int64_t ld_out) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= total_lanes) return;
    const int lane = (int)(t & 63);
    const int64_t idx = t >> 6;
    const int64_t c = idx % KC;
    const int64_t eu = idx / KC;
    const int64_t u = eu % NU;
    const int64_t e = eu / NU;
    const int64_t blk = v.block(e, u, c);
    const int64_t n = u * kUnitN + (lane & 15);
    if (n >= N) return;
    const uint4 q = *reinterpret_cast<const uint4*>(v.codes + blk * kCodeBlock + lane * 16);
    const uint32_t sc = *reinterpret_cast<const uint16_t*>(v.scales + blk * kScaleBlock + lane * 2);
    const float s0 = v.mx ? e8m0_to_f32(sc) : e4m3_to_f32(sc & 0xFFu);
    const float s1 = v.mx ? e8m0_to_f32(sc >> 8) : e4m3_to_f32(sc >> 8);
    const uint32_t qd[4] = {q.x, q.y, q.z, q.w};
    const int64_t k0 = c * kChunkK + (lane >> 4) * 32;
    uint16_t* row = out + (e * N + n) * ld_out;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint4 dv = decode8_bf16(qd[d], d < 2 ? s0 : s1);
        const uint32_t vd[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t k = k0 + d * 8 + i;
            if (k < K) row[k] = (uint16_t)((vd[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
        }
    }
}

// Plain read of n16 16-byte words, the bandwidth reference the GEMMs are
// measured against: workgroup b reads its contiguous share of the buffer with
// non-temporal 16-byte loads, U per thread in flight, and folds them into one
// dword per thread; a store that depends on every loaded word (taken only if
// the fold hits a fixed value) keeps the loads from being dropped.
template <int U>
__global__ void __launch_bounds__(256) k_stream_read(const uint8_t* __restrict__ p, int64_t n16,
                                                     uint32_t* __restrict__ out) {
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t b0 = (int64_t)blockIdx.x * per;
    const int64_t b1 = b0 + per < n16 ? b0 + per : n16;
    uint32_t acc = 0u;
    for (int64_t i = b0 + threadIdx.x; i < b1; i += 256 * U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = i + u * 256;
            v[u] = j < b1 ? load_stream_u4(p + j * 16) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) out[blockIdx.x] = acc;
}

}  // namespace nvfp4
