// W4A16 NVFP4 GEMM kernels for gfx950.
//
//   Y[m,n] = RNE_bf16(g * sum_k X'[m,k] * e2m1(code(n,k)) * e4m3(S[n,k/16]))
//
// X' is the activation (already multiplied by the pre-quant scale when one
// is given).  Two kernels, chosen by the number of rows:
//
// small-M (rows <= 16 per pass; HBM-bound): one workgroup per 16-row unit
//   of W, its W waves splitting K.  Each wave streams its K range of the
//   unit with one 128-bit load per lane per 128-wide chunk and contracts it
//   with v_mfma_f32_4x4x4bf16_1k in the 16-block form: block b of the
//   instruction handles rows 4(b&3)..+3 of the unit and the 32-wide K group
//   b>>2, so every lane holds the codes of one weight row and one K group.
//   Only the power of two of each E4M3 scale is applied in the code
//   conversion; the remaining significand factor multiplies the fp32
//   partial sum of its 16-wide block (four MFMA steps), which costs one FMA
//   per output row and block instead of one multiply per weight.  The
//   activation operand is broadcast within each group of four blocks
//   (cbsz = 2) from the block that holds the current step's K slice, so
//   every lane loads one distinct 16-byte piece per four rows.  Partial sums are reduced across K
//   groups with lane shuffles and across waves through LDS in a fixed order.
//
// large-M (MFMA-bound): 128 x 256 output tile per workgroup of four waves.
//   The activation tile (128 rows x 128 k) is staged through LDS with double
//   buffering; each wave owns 64 output columns, decodes its weight
//   fragments straight into registers (exact bf16) and runs
//   v_mfma_f32_16x16x32_bf16 over 8 x 4 sub-tiles with fp32 accumulators.
//   The 32 K slots of one MFMA step map to k = 32 g + 8 t + e for lane group
//   g, step t, element e, on both operands, so the weight lanes read whole
//   32-wide K groups from the repacked layout.
//
// Both kernels exist in a dense and a grouped (MoE) form.  The grouped form
// reads expert_offsets on the device: the small-M grid has one slice per
// expert and slices of experts without rows exit at once; the large-M grid
// has an upper bound of (R / 128 + E) row tiles, mapped to (expert, tile) by
// a wave-wide prefix scan of the per-expert tile counts, extra tiles exit.
// Experts without rows therefore read no weight bytes.
#pragma once
#include "decode.h"
#include "layout.h"

namespace nvfp4 {

constexpr int kSmallRows = 16;      // rows per pass of the small-M kernel
constexpr int kLargeBM = 128;       // rows per tile of the large-M kernel
constexpr int kLargeUnits = 16;     // 16-row units of W per large-M tile (256 columns)
constexpr int kLargeLDA = 136;      // bf16 per LDS row of the activation tile (128 + 8 pad)
constexpr int kMaxExperts = 4096;

// ----------------------------------------------------------------- small-M --

template <int MG>
__device__ __forceinline__ void small_m_pass(const uint16_t* __restrict__ xrow0, int64_t ld_x, int rows,
                                             const uint8_t* __restrict__ cp, const uint8_t* __restrict__ sp,
                                             int c0, int c1, int K, float (*red_w)[16], int lane) {
    // Lane l = 16 g + 4 q + i holds rows 4 mg + i of the activation at
    // k = 128 c + 32 g + 8 q .. +7 (one 16-byte piece per m-group).  MFMA
    // step t (k = 32 g + 4 t .. +3) broadcasts A from block q = t >> 1 of
    // each group of four blocks (cbsz = 2, abid = t >> 1).
    const int g = lane >> 4, q = (lane >> 2) & 3, ai = lane & 3;
    f32x4 acc[MG];
    const uint16_t* xr[MG];
    bool xv[MG];
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) {
        acc[mg] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int m = 4 * mg + ai;
        xv[mg] = m < rows;
        xr[mg] = xrow0 + (int64_t)(xv[mg] ? m : 0) * ld_x + g * 32 + q * 8;
    }

    uint4 cw_n = make_uint4(0u, 0u, 0u, 0u);
    uint32_t sw_n = 0u;
    uint4 xa_n[MG];

    auto load = [&](int c) {
        cw_n = *reinterpret_cast<const uint4*>(cp + (int64_t)c * kCodeBlock);
        sw_n = *reinterpret_cast<const uint16_t*>(sp + (int64_t)c * kScaleBlock);
        const bool kin = c * kChunkK + g * 32 + q * 8 < K;
#pragma unroll
        for (int mg = 0; mg < MG; ++mg)
            xa_n[mg] = (xv[mg] && kin) ? *reinterpret_cast<const uint4*>(xr[mg] + (int64_t)c * kChunkK)
                                       : make_uint4(0u, 0u, 0u, 0u);
    };

    if (c0 < c1) load(c0);
    for (int c = c0; c < c1; ++c) {
        const uint4 cw = cw_n;
        const uint32_t sw = sw_n;
        uint4 xa[MG];
#pragma unroll
        for (int mg = 0; mg < MG; ++mg) xa[mg] = xa_n[mg];
        if (c + 1 < c1) load(c + 1);

        float cs0, f0, cs1, f1;
        split_scale(e4m3_to_f32(sw & 0xFFu), cs0, f0);
        split_scale(e4m3_to_f32(sw >> 8), cs1, f1);
        const s16x4 b0 = decode4_bf16_pow2<0>(cw.x, cs0), b1 = decode4_bf16_pow2<2>(cw.x, cs0);
        const s16x4 b2 = decode4_bf16_pow2<0>(cw.y, cs0), b3 = decode4_bf16_pow2<2>(cw.y, cs0);
        const s16x4 b4 = decode4_bf16_pow2<0>(cw.z, cs1), b5 = decode4_bf16_pow2<2>(cw.z, cs1);
        const s16x4 b6 = decode4_bf16_pow2<0>(cw.w, cs1), b7 = decode4_bf16_pow2<2>(cw.w, cs1);
#pragma unroll
        for (int mg = 0; mg < MG; ++mg) {
            const s16x4 alo = dwords_to_s16x4(xa[mg].x, xa[mg].y), ahi = dwords_to_s16x4(xa[mg].z, xa[mg].w);
            f32x4 p = {0.f, 0.f, 0.f, 0.f};
            p = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(alo, b0, p, 2, 0, 0);
            p = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ahi, b1, p, 2, 0, 0);
            p = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(alo, b2, p, 2, 1, 0);
            p = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ahi, b3, p, 2, 1, 0);
            f32x4 r = {0.f, 0.f, 0.f, 0.f};
            r = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(alo, b4, r, 2, 2, 0);
            r = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ahi, b5, r, 2, 2, 0);
            r = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(alo, b6, r, 2, 3, 0);
            r = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ahi, b7, r, 2, 3, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mg][i] = __builtin_fmaf(f1, r[i], __builtin_fmaf(f0, p[i], acc[mg][i]));
        }
    }

    // Sum the four K groups: lanes l, l^16, l^32, l^48 hold the same outputs.
#pragma unroll
    for (int mg = 0; mg < MG; ++mg)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v = acc[mg][i];
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            if (lane < 16) red_w[4 * mg + i][lane] = v;   // lane < 16: column lane, row 4 mg + i
        }
}

template <int W, bool GROUPED>
__global__ void __launch_bounds__(W * 64) k_gemm_small_m(const uint16_t* __restrict__ x, int64_t ld_x,
                                                         const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales, int NU, int KC, int K,
                                                         int N, const float* __restrict__ gscale, int g_is_div,
                                                         uint16_t* __restrict__ y, int64_t ld_y, int64_t rows_dense,
                                                         const int32_t* __restrict__ offsets) {
    __shared__ float red[W][kSmallRows][16];
    const int u = blockIdx.x;
    const int e = GROUPED ? (int)blockIdx.y : 0;
    int64_t row0 = 0, count = rows_dense;
    if (GROUPED) {
        row0 = offsets[e];
        count = (int64_t)offsets[e + 1] - row0;
    }
    if (count <= 0 || u >= NU) return;   // uniform over the workgroup

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c0 = (int)((int64_t)KC * w / W), c1 = (int)((int64_t)KC * (w + 1) / W);
    const int64_t blk0 = ((int64_t)e * NU + u) * KC;
    const uint8_t* cp = codes + blk0 * kCodeBlock + lane * 16;
    const uint8_t* sp = scales + blk0 * kScaleBlock + lane * 2;
    const float gv = effective_global_scale(gscale[e], g_is_div);

    for (int64_t p0 = 0; p0 < count; p0 += kSmallRows) {
        const int rows = (int)((count - p0) < kSmallRows ? (count - p0) : kSmallRows);
        const uint16_t* xrow0 = x + (row0 + p0) * ld_x;
        switch ((rows + 3) >> 2) {
            case 1: small_m_pass<1>(xrow0, ld_x, rows, cp, sp, c0, c1, K, red[w], lane); break;
            case 2: small_m_pass<2>(xrow0, ld_x, rows, cp, sp, c0, c1, K, red[w], lane); break;
            case 3: small_m_pass<3>(xrow0, ld_x, rows, cp, sp, c0, c1, K, red[w], lane); break;
            default: small_m_pass<4>(xrow0, ld_x, rows, cp, sp, c0, c1, K, red[w], lane); break;
        }
        __syncthreads();
        for (int t = threadIdx.x; t < rows * 16; t += W * 64) {
            const int r = t >> 4, col = t & 15;
            float s = 0.f;
#pragma unroll
            for (int ww = 0; ww < W; ++ww) s += red[ww][r][col];
            const int64_t n = (int64_t)u * kUnitN + col;
            if (n < N) y[(row0 + p0 + r) * ld_y + n] = (uint16_t)f32_to_bf16_rne(gv * s);
        }
        __syncthreads();
    }
}

// ----------------------------------------------------------------- large-M --

template <bool GROUPED>
__global__ void __launch_bounds__(256, 1) k_gemm_large_m(const uint16_t* __restrict__ x, int64_t ld_x,
                                                         const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales, int NU, int KC, int K,
                                                         int N, const float* __restrict__ gscale, int g_is_div,
                                                         uint16_t* __restrict__ y, int64_t ld_y, int64_t rows_dense,
                                                         const int32_t* __restrict__ offsets, int E) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kLargeBM * kLargeLDA];
    __shared__ int s_map[2];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4;

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
                const int tiles = (cnt + kLargeBM - 1) / kLargeBM;
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
        row0 = (int64_t)offsets[e] + (int64_t)s_map[1] * kLargeBM;
        rows = (int64_t)offsets[e + 1] - row0;
    } else {
        row0 = (int64_t)blockIdx.y * kLargeBM;
        rows = rows_dense - row0;
    }
    if (rows > kLargeBM) rows = kLargeBM;

    // This wave's four 16-row units of W (64 output columns).
    const int u_base = (int)blockIdx.x * kLargeUnits + w * 4;
    const uint8_t* cpj[4];
    const uint8_t* spj[4];
    bool okj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        okj[j] = (u_base + j) < NU;
        const int64_t blk = ((int64_t)e * NU + (okj[j] ? u_base + j : 0)) * KC;
        cpj[j] = codes + blk * kCodeBlock + lane * 16;
        spj[j] = scales + blk * kScaleBlock + lane * 2;
    }

    // Activation tile loader: 128 rows x 16 pieces of 8 bf16; thread -> 8 pieces.
    const int a_piece = tid & 15, a_row0 = tid >> 4;
    const uint16_t* xbase = x + row0 * ld_x;
    uint4 areg[8];
    auto load_a = [&](int c) {
        const int k = c * kChunkK + a_piece * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = a_row0 + 16 * i;
            const bool ok = (r < rows) && (k < K);
            areg[i] = ok ? *reinterpret_cast<const uint4*>(xbase + (int64_t)r * ld_x + k) : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<uint4*>(&As[buf][(a_row0 + 16 * i) * kLargeLDA + a_piece * 8]) = areg[i];
    };
    uint4 bc[4], bc_n[4];
    uint32_t bs[4], bs_n[4];
    auto load_b = [&](int c) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bc_n[j] = okj[j] ? *reinterpret_cast<const uint4*>(cpj[j] + (int64_t)c * kCodeBlock) : make_uint4(0u, 0u, 0u, 0u);
            bs_n[j] = okj[j] ? (uint32_t)*reinterpret_cast<const uint16_t*>(spj[j] + (int64_t)c * kScaleBlock) : 0u;
        }
    };

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    load_a(0);
    load_b(0);
    store_a(0);
    __syncthreads();

    for (int c = 0; c < KC; ++c) {
        const int buf = c & 1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bc[j] = bc_n[j];
            bs[j] = bs_n[j];
        }
        const bool more = (c + 1) < KC;
        if (more) {
            load_a(c + 1);
            load_b(c + 1);
        }
        float slo[4], shi[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            slo[j] = e4m3_to_f32(bs[j] & 0xFFu);
            shi[j] = e4m3_to_f32(bs[j] >> 8);
        }
        const uint16_t* abase = &As[buf][(lane & 15) * kLargeLDA + g * 32];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            bf16x8 bf[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t d = t == 0 ? bc[j].x : t == 1 ? bc[j].y : t == 2 ? bc[j].z : bc[j].w;
                bf[j] = uint4_to_bf16x8(decode8_bf16(d, t < 2 ? slo[j] : shi[j]));
            }
#pragma unroll
            for (int ms = 0; ms < 8; ++ms) {
                const bf16x8 af = uint4_to_bf16x8(*reinterpret_cast<const uint4*>(abase + ms * 16 * kLargeLDA + t * 8));
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[ms][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[j], acc[ms][j], 0, 0, 0);
            }
        }
        if (more) store_a(buf ^ 1);
        __syncthreads();
    }

    const float gv = effective_global_scale(gscale[e], g_is_div);
#pragma unroll
    for (int ms = 0; ms < 8; ++ms)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = (int64_t)(u_base + j) * kUnitN + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = ms * 16 + g * 4 + i;
                if (m < rows && n < N) y[(row0 + m) * ld_y + n] = (uint16_t)f32_to_bf16_rne(gv * acc[ms][j][i]);
            }
        }
}

}  // namespace nvfp4
