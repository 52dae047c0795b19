// Tile GEMM for rows > 8: a BM x (16 NT W) output tile per workgroup.
//
//   BM = 16 MS rows.  The activation chunk (BM rows x 128 k) is staged once
//   per workgroup in a double-buffered LDS ring and shared by all W waves;
//   its global loads ride in the same D-deep register ring as the weights,
//   so no chunk waits on a load issued in its own iteration;
//   wave w owns NT consecutive 16-row units of W, decodes their codes straight
//   into exact bf16 v_mfma_f32_16x16x32_bf16 fragments and accumulates MS x NT
//   16x16 sub-tiles in fp32.  The 32 K slots of an MFMA step map to
//   k = 32 g + 8 t + e (lane group g, step t, element e) on both operands, so
//   each weight lane reads a whole 32-wide K group of the repacked layout.
//
//   K may be split S ways across workgroups (grid z).  Each split writes its
//   fp32 partial tile to the workspace, then bumps the tile's counter; the
//   workgroup that arrives last adds the S partials in split order (0..S-1,
//   independent of arrival order, so the result is bitwise reproducible),
//   applies the epilogue and resets the counter to zero for the next call.
//
//   Grouped (MoE) form: grid y has R/BM + E row-tile slots, mapped to
//   (expert, tile) by a wave-wide prefix scan of the per-expert tile counts
//   read from expert_offsets; surplus slots exit before touching weights.
#pragma once
#include "decode.h"
#include "kernels_gemm.h"
#include "layout.h"

namespace nvfp4 {

constexpr int kTileLDA = 136;   // bf16 per LDS row of the activation stage (128 + 8 pad)

struct SplitK {
    int S;              // K splits (grid z)
    float* partials;    // [S][tiles][BM * units * 16] fp32 in lane order, used when S > 1
    int* counters;      // [row tiles][unit groups], zero between calls
};

template <int MS, int NT, int W, int D, bool GROUPED, bool KFULL>
__global__ void __launch_bounds__(W * 64) k_gemm_tile(const uint16_t* __restrict__ x, int64_t ld_x, BlobView bv,
                                                      int NU, int KC, int K, int N,
                                                      const float* __restrict__ gscale, int g_is_div,
                                                      uint16_t* __restrict__ y, int64_t ld_y, int64_t rows_dense,
                                                      const int32_t* __restrict__ offsets, int E, SplitK sk) {
    constexpr int BM = 16 * MS;
    constexpr int UG = NT * W;                                     // units per workgroup
    constexpr int APIECES = BM * 16;                               // 16-byte pieces per activation chunk
    constexpr int APT = (APIECES + W * 64 - 1) / (W * 64);         // pieces per thread
    static_assert(D >= 2, "the ring stages chunk c + 1 from another slot while refilling chunk c's");
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * kTileLDA];
    __shared__ float2 lut[256];
    __shared__ int s_map[3];

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

    // ---- which rows: dense m-tile, or (expert, m-tile) of the grouped form
    int e = 0;
    int64_t row0, rows;
    if (GROUPED) {
        if (tid == 0) s_map[0] = -1;
        __syncthreads();
        if (w == 0) {
            const int by = (int)blockIdx.y;
            int carry = 0;
            for (int base = 0; base < E; base += 64) {
                const int ex = base + lane;
                const int cnt = ex < E ? (offsets[ex + 1] - offsets[ex]) : 0;
                const int tiles = (cnt + BM - 1) / BM;
                int v = tiles;
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    const int t = __shfl_up(v, d);
                    if (lane >= d) v += t;
                }
                const int incl = carry + v, excl = incl - tiles;
                if (tiles > 0 && by >= excl && by < incl) {
                    s_map[0] = ex;
                    s_map[1] = by - excl;
                }
                carry += __shfl(v, 63);
            }
        }
        __syncthreads();
        e = s_map[0];
        if (e < 0) return;   // uniform: a slot past the last active tile
        row0 = (int64_t)offsets[e] + (int64_t)s_map[1] * BM;
        rows = (int64_t)offsets[e + 1] - row0;
    } else {
        row0 = (int64_t)blockIdx.y * BM;
        rows = rows_dense - row0;
    }
    if (rows > BM) rows = BM;
    build_scale_table(lut);

    const int S = sk.S, s = (int)blockIdx.z;
    const int c0 = (int)((int64_t)KC * s / S), c1 = (int)((int64_t)KC * (s + 1) / S);
    const int u_w = (int)blockIdx.x * UG + w * NT;                 // this wave's first unit
    const int64_t cstr = bv.chunk_stride * kCodeBlock;
    const uint8_t* cb[NT];
    const uint8_t* sb[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        // units past NU read unit 0 (their columns are never stored)
        const int64_t blk = bv.block(e, (u_w + j) < NU ? u_w + j : 0, 0);
        cb[j] = bv.codes + blk * kCodeBlock;
        sb[j] = bv.scales + blk * kScaleBlock;
    }

    // ---- per-wave ring of D chunks: NT code blocks + scale pairs, and this
    // thread's share of the activation chunk (staged to LDS one chunk ahead
    // of its use, so its load is issued D - 1 chunks before it is needed).
    // Activation piece p = thread + i * threads: row p >> 4, k piece p & 15.
    struct Slot {
        uint4 cw[NT];
        uint32_t sw[NT];
        uint4 a[APT];
    };
    const uint16_t* xbase = x + row0 * ld_x;
    const int c_last = c1 - 1;
    auto load_slot = [&](Slot& b, int c_req) {
        const int c = c_req < c_last ? c_req : c_last;
        const int64_t boff = (int64_t)c * cstr;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            b.cw[j] = load_stream_u4(cb[j] + boff + (uint32_t)(lane * 16));
            b.sw[j] = load_stream_u16(sb[j] + (boff >> 3) + (uint32_t)(lane * 2));
        }
#pragma unroll
        for (int i = 0; i < APT; ++i) {
            const int p = tid + i * W * 64;
            const int pr = (p >> 4) < BM ? (p >> 4) : 0, pk = p & 15;
            const int k = c * kChunkK + pk * 8;
            // rows past `rows` read row 0 (outputs never stored); pieces past K are zeroed at store
            b.a[i] = *reinterpret_cast<const uint4*>(xbase + (int64_t)(pr < rows ? pr : 0) * ld_x + (k < K ? k : 0));
        }
    };
    auto store_a = [&](int buf, const Slot& b, int c) {
#pragma unroll
        for (int i = 0; i < APT; ++i) {
            const int p = tid + i * W * 64;
            if (APIECES % (W * 64) != 0 && p >= APIECES) break;
            const int pr = p >> 4, pk = p & 15;
            const bool kin = KFULL || (c * kChunkK + pk * 8 < K);
            const uint4 v = b.a[i];
            *reinterpret_cast<uint4*>(&As[buf][pr * kTileLDA + pk * 8]) =
                make_uint4(kin ? v.x : 0u, kin ? v.y : 0u, kin ? v.z : 0u, kin ? v.w : 0u);
        }
    };

    f32x4 acc[MS][NT];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[ms][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const Slot& b, int buf) {
        const uint16_t* abase = &As[buf][r * kTileLDA + g * 32];
        float sc[NT][2];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const float2 l0 = lut[b.sw[j] & 0xFFu], l1 = lut[(b.sw[j] >> 8) & 0xFFu];
            sc[j][0] = __uint_as_float(__float_as_uint(l0.x) & 0x7F800000u) * l0.y;
            sc[j][1] = __uint_as_float(__float_as_uint(l1.x) & 0x7F800000u) * l1.y;
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            bf16x8 bf[NT];
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const uint32_t d = t == 0 ? b.cw[j].x : t == 1 ? b.cw[j].y : t == 2 ? b.cw[j].z : b.cw[j].w;
                bf[j] = uint4_to_bf16x8(decode8_bf16(d, sc[j][t >> 1]));
            }
#pragma unroll
            for (int ms = 0; ms < MS; ++ms) {
                const bf16x8 af = uint4_to_bf16x8(*reinterpret_cast<const uint4*>(abase + ms * 16 * kTileLDA + t * 8));
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    acc[ms][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[j], acc[ms][j], 0, 0, 0);
            }
        }
    };

    if (c0 < c1) {
        Slot ring[D];
#pragma unroll
        for (int d = 0; d < D; ++d) load_slot(ring[d], c0 + d);
        store_a(0, ring[0], c0);
        __syncthreads();   // scale table and first activation chunk ready
        // Iteration for chunk cc (ring slot d, LDS buffer (cc - c0) & 1):
        // stage chunk cc + 1 into the other buffer, refill slot d with chunk
        // cc + D, contract chunk cc, then one barrier.
        int c = c0;
        for (; c + D <= c1; c += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int cc = c + d;
                if (cc + 1 < c1) store_a((cc + 1 - c0) & 1, ring[(d + 1) % D], cc + 1);
                const Slot cur = ring[d];
                load_slot(ring[d], cc + D);
                compute(cur, (cc - c0) & 1);
                __syncthreads();
            }
        }
#pragma unroll
        for (int d = 0; d < D - 1; ++d) {
            const int cc = c + d;
            if (cc < c1) {
                if (cc + 1 < c1) store_a((cc + 1 - c0) & 1, ring[d + 1], cc + 1);
                compute(ring[d], (cc - c0) & 1);
                __syncthreads();
            }
        }
    } else {
        __syncthreads();
    }

    const float gv = effective_global_scale(gscale[e], g_is_div);
    // lane (r, g) holds rows 16 ms + 4 g + i of column 16 (u_w + j) + r
    if (S == 1) {
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int64_t n = (int64_t)(u_w + j) * kUnitN + r;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = ms * 16 + g * 4 + i;
                    if (m < rows && n < N) y[(row0 + m) * ld_y + n] = (uint16_t)f32_to_bf16_rne(gv * acc[ms][j][i]);
                }
            }
        return;
    }

    // ---- split K: publish this split's partial tile, the last arrival reduces.
    // Partials are stored and loaded with device-scope (sc1) accesses, which
    // are coherent across the XCDs' separate L2 caches; an agent-scope fence
    // would instead write back and invalidate the whole L2 of the XCD.  Each
    // wave waits for its stores to be acknowledged before the barrier that
    // precedes the counter bump, so every split's partial is visible on the
    // device before the counter can return S - 1.
    const int64_t tile = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    const int64_t tiles = (int64_t)gridDim.x * gridDim.y;
    constexpr int64_t kTilePairs = (int64_t)MS * NT * W * 64 * 2;   // float pairs per partial tile
    uint64_t* parts = reinterpret_cast<uint64_t*>(sk.partials);
    auto pidx = [&](int ms, int j, int h) { return (((ms * NT + j) * W + w) * 64 + lane) * 2 + h; };
    uint64_t* my_part = parts + ((int64_t)s * tiles + tile) * kTilePairs;
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint64_t v = (uint64_t)__float_as_uint(acc[ms][j][2 * h]) |
                                   ((uint64_t)__float_as_uint(acc[ms][j][2 * h + 1]) << 32);
                __hip_atomic_store(my_part + pidx(ms, j, h), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);   // all of this wave's partial stores acknowledged
    __syncthreads();
    if (tid == 0) s_map[2] = atomicAdd(&sk.counters[tile], 1);
    __syncthreads();
    if (s_map[2] != S - 1) return;   // uniform: not the last split of this tile
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float v0 = 0.f, v1 = 0.f;   // splits added in order 0..S-1 whichever arrived last
                for (int ss = 0; ss < S; ++ss) {
                    float a0 = acc[ms][j][2 * h], a1 = acc[ms][j][2 * h + 1];
                    if (ss != s) {
                        const uint64_t pv = __hip_atomic_load(parts + ((int64_t)ss * tiles + tile) * kTilePairs +
                                                                  pidx(ms, j, h),
                                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        a0 = __uint_as_float((uint32_t)pv);
                        a1 = __uint_as_float((uint32_t)(pv >> 32));
                    }
                    v0 += a0;
                    v1 += a1;
                }
                acc[ms][j][2 * h] = v0;
                acc[ms][j][2 * h + 1] = v1;
            }
    if (tid == 0) __hip_atomic_store(&sk.counters[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int64_t n = (int64_t)(u_w + j) * kUnitN + r;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = ms * 16 + g * 4 + i;
                if (m < rows && n < N) y[(row0 + m) * ld_y + n] = (uint16_t)f32_to_bf16_rne(gv * acc[ms][j][i]);
            }
        }
}

}  // namespace nvfp4
