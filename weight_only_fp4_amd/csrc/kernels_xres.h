// Decode-sized GEMM with the activation held in registers (rows <= 16).
//
//   Each of the W waves of a workgroup owns one contiguous K slice of CH
//   chunks (128 k each).  A wave loads the activation rows of its slice once:
//   coalesced 16-byte loads (each load instruction covers four rows x 256
//   bytes, whole cache lines) go through a small private LDS area and come
//   back in the register layout of the v_mfma_f32_16x16x32_bf16 A operand,
//   where they stay for the whole kernel; the weight ring goes out right
//   after them.  The workgroup then walks U
//   consecutive 16-row units of W: every wave streams its slice of each unit
//   through a D-deep register ring (one 128-bit code load and one scale
//   dword per lane and chunk), decodes the codes into exact bf16 fragments
//   and accumulates a 16 x 16 fp32 tile per unit.  The loop has no barrier,
//   so each wave computes as soon as its own weights arrive instead of
//   waiting for the slowest wave of the workgroup at every step.
//
//   Reduction, in a fixed order (bitwise reproducible): wave w + W/2 adds its
//   tiles into wave w's through LDS, then the W/2 sums are added in wave
//   order, scaled by the global scale and rounded to bf16 (fp16 with F16).
//   K beyond 16 waves x CH chunks is split S ways across workgroups (grid
//   y): each split publishes its partial tile and the last arrival adds the
//   S partials in split order (SplitK); the publish / count / reload round
//   trip costs about 2 us, so shapes whose K fits one workgroup never split.
//
//   K slots of an MFMA step map to k = 32 g + 8 t + e (lane group g, step t,
//   element e) on both operands, as in the tile kernel, so a weight lane reads
//   one 32-wide K group of the repacked layout.  With PRE the pre-quant
//   scale is applied to each activation piece (prescale8) as the slice is
//   staged, once per wave.  Activation rows past `rows`
//   and K pieces past K are zero (never loaded); units past NU read unit
//   NU - 1 and store nothing.  FULL (K == 128 S W CH: every wave owns CH whole
//   chunks) compiles without any per-chunk condition; otherwise chunks past
//   K re-read the last chunk with a zero scale, so they add exact zeros
//   whatever that chunk holds (no branch in the loop).
#pragma once
#include "decode.h"
#include "kernels_gemm.h"
#include "layout.h"

namespace nvfp4 {

constexpr int kXresRowBytes = 256 + 16;                // one row of a staged chunk, padded
constexpr int kXresWaveBytes = 16 * kXresRowBytes;     // a wave's staging area

template <int CH, int U, int W, int D, bool FULL, bool F16 = false, bool PRE = false, bool MX = false>
__global__ void __launch_bounds__(W * 64) k_gemm_xres(const uint16_t* __restrict__ x, int64_t ld_x, BlobView bv,
                                                      int NU, int KC, int K, int N, const float* __restrict__ gscale,
                                                      int g_is_div, uint16_t* __restrict__ y, int64_t ld_y, int rows,
                                                      SplitK sk, const uint16_t* __restrict__ pre) {
    constexpr int NI = U * CH;          // ring items of a wave: (unit, chunk), unit-major
    constexpr int H = W / 2;            // waves after the first reduction stage
    constexpr int TILE = U * 256;       // fp32 outputs of the workgroup (16 rows x 16 U columns)
    static_assert(D >= 1, "ring depth");
    constexpr int DR = D < NI ? D : NI;   // ring slots in use
    static_assert(W % 2 == 0, "the first reduction stage pairs waves w and w + W/2");
    __shared__ __attribute__((aligned(16))) uint8_t xs[W * kXresWaveBytes];
    __shared__ int s_flag;
    __shared__ __attribute__((aligned(16))) float red[H * TILE];

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int s = (int)blockIdx.y, S = sk.S;                              // K split of this workgroup
    const int c0 = (s * W + w) * CH;                                      // first chunk of this wave's slice
    const int nch = KC - c0 < CH ? (KC - c0 > 0 ? KC - c0 : 0) : CH;      // chunks that exist (wave-uniform)
    const int u0 = (int)blockIdx.x * U;

    // ---- weight ring
    const int64_t cstr = bv.chunk_stride * kCodeBlock;
    auto blk_of = [&](int it) {
        // chunks past this wave's range re-read the last chunk of the matrix (never used)
        const int u = u0 + it / CH, c = c0 + it % CH < KC ? c0 + it % CH : KC - 1;
        return bv.block(0, u < NU ? u : NU - 1, 0) * kCodeBlock + (int64_t)c * cstr;   // code byte offset
    };
    uint4 cw[DR];
    uint32_t sw[DR];
    auto load_item = [&](int it, int slot) {
        const int64_t off = blk_of(it);
        cw[slot] = load_stream_u4(bv.codes + off + lane * 16);
        sw[slot] = load_scale_dword(bv.scales + (off >> 3), lane);
    };

    // ---- activation chunk c of the slice, coalesced: load i takes rows
    // 4 i + (lane >> 4), bytes 16 (lane & 15) of the chunk's 256 per row
    uint4 xa[CH][4];
    uint4 pa[CH];   // pre-quant scale piece of the lane's k (PRE only; the same for its four rows)
    auto load_x = [&](int c) {
        const int k = (c0 + c) * kChunkK + (lane & 15) * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * i + (lane >> 4);
            xa[c][i] = (row < rows && (FULL || k < K)) ? *reinterpret_cast<const uint4*>(x + (int64_t)row * ld_x + k)
                                                       : make_uint4(0u, 0u, 0u, 0u);
        }
        if constexpr (PRE) pa[c] = *reinterpret_cast<const uint4*>(pre + (FULL || k < K ? k : 0));
    };
    // through this wave's LDS area into the A-operand layout: lane (r, g)
    // takes X[r][128 c + 32 g + 8 t + 0..7] (row stride = 16 mod 256 bytes:
    // the 16 lanes of a lane group hit distinct banks).  LDS operations of a
    // wave complete in order, so one area serves every chunk.
    uint8_t* mine = xs + w * kXresWaveBytes;
    uint4 xr[CH][4];
    auto stage_x = [&](int c) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<uint4*>(mine + (4 * i + (lane >> 4)) * kXresRowBytes + (lane & 15) * 16) =
                PRE ? prescale8<F16>(xa[c][i], pa[c]) : xa[c][i];
#pragma unroll
        for (int t = 0; t < 4; ++t)
            xr[c][t] = *reinterpret_cast<const uint4*>(mine + r * kXresRowBytes + g * 64 + t * 16);
    };

    // prologue: the whole activation slice, then the weight ring; the slice
    // is staged into registers once its loads land.  Counters retire in issue
    // order, so loading the activation first lets that wait leave the whole
    // ring in flight (measured faster than a weight item first).
#pragma unroll
    for (int c = 0; c < CH; ++c) load_x(c);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < DR; ++d) {
        load_item(d, d);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) stage_x(c);

    f32x4 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int it = 0; it < NI; ++it) {
        const int slot = it % DR, u = it / CH, c = it % CH;
        const uint4 cv = cw[slot];
        const uint32_t sv = sw[slot];
        if (it + DR < NI) {
            load_item(it + DR, slot);
            __builtin_amdgcn_sched_barrier(0);
        }
        f32x2 sc = scale_pair_f32<MX>(scale_pair(sv, lane));
        if (!FULL) {
            const bool have = c < nch;
            sc.x = have ? sc.x : 0.f;
            sc.y = have ? sc.y : 0.f;
        }
        if constexpr (F16 && !MX) {
            // fp16 with E4M3 scales: the scale's power of two in the conversion, its significand by fp16 pairs
            const HalfScale h0 = half_scale(sc.x), h1 = half_scale(sc.y);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t d = t == 0 ? cv.x : t == 1 ? cv.y : t == 2 ? cv.z : cv.w;
                acc[u] = mma16<F16>(xr[c][t], decode8_f16_split(d, t < 2 ? h0 : h1), acc[u]);
            }
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t d = t == 0 ? cv.x : t == 1 ? cv.y : t == 2 ? cv.z : cv.w;
                acc[u] = mma16<F16>(xr[c][t], decode8_fmt<F16, MX>(d, t < 2 ? sc.x : sc.y), acc[u]);
            }
        }
    }

    // ---- reduce the W wave tiles: lane (r, g) holds rows 4 g + i of column 16 u + r
    if (w >= H) {
#pragma unroll
        for (int u = 0; u < U; ++u) *reinterpret_cast<f32x4*>(&red[((w - H) * U + u) * 256 + lane * 4]) = acc[u];
    }
    __syncthreads();
    if (w < H) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            f32x4* p = reinterpret_cast<f32x4*>(&red[(w * U + u) * 256 + lane * 4]);
            *p = acc[u] + *p;
        }
    }
    __syncthreads();
    constexpr int PER = (TILE + W * 64 - 1) / (W * 64);   // outputs per thread
    float v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        // o = (u, m, n): consecutive threads take consecutive columns of one row
        const int o = tid + j * W * 64, oc = o < TILE ? o : 0, m = (oc >> 4) & 15;
        const int src = (oc >> 8) * 256 + ((m >> 2) * 16 + (oc & 15)) * 4 + (m & 3);
        float a = red[src];
#pragma unroll
        for (int ww = 1; ww < H; ++ww) a += red[ww * TILE + src];
        v[j] = a;
    }
    if (S > 1) {
        // K splits: publish this split's partial tile; the last arrival adds
        // the S partials in split order 0..S-1, whichever arrived last
        const int64_t tile = blockIdx.x, tiles = gridDim.x;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int o = tid + j * W * 64;
            if (o < TILE) store_partial(sk.partials + ((int64_t)s * tiles + tile) * TILE + o, v[j]);
        }
        if (!split_arrive(sk.counters, tile, S, &s_flag)) return;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int o = tid + j * W * 64;
            if (o >= TILE) continue;
            float a = 0.f;
            for (int ss = 0; ss < S; ++ss) {
                const float p = ss == s ? v[j] : load_partial(sk.partials + ((int64_t)ss * tiles + tile) * TILE + o);
                a = ss == 0 ? p : a + p;
            }
            v[j] = a;
        }
    }
    const float gv = global_scale_at(gscale, 0, g_is_div);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int o = tid + j * W * 64, m = (o >> 4) & 15;
        const int64_t col = (int64_t)(u0 + (o >> 8)) * kUnitN + (o & 15);
        if (o < TILE && m < rows && col < N) y[(int64_t)m * ld_y + col] = (uint16_t)round_out<F16>(scale_acc(gv, v[j]));
    }
}

}  // namespace nvfp4
