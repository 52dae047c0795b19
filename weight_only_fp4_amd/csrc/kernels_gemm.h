// W4A16 NVFP4 GEMM kernels for gfx950.
//
//   Y[m,n] = RNE_bf16(g * sum_k X'[m,k] * e2m1(code(n,k)) * e4m3(S[n,k/16]))
//
// X' is the activation (already multiplied by the pre-quant scale when one
// is given).  This file holds the small-M kernel, used for up to 4 rows
// (the host planner's choice; a pass covers up to 16 rows):
//
// small-M (HBM-bound): one workgroup per 16-row unit
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
// Rows above 4 go to the tile kernel (kernels_tile.h).  The small-M grouped
// form reads expert_offsets on the device: one grid slice per expert, and
// slices of experts without rows exit at once, so they read no weight bytes.
#pragma once
#include "decode.h"
#include "layout.h"

namespace nvfp4 {

constexpr int kSmallRows = 16;      // rows per pass of the small-M kernel
constexpr int kMaxExperts = 4096;

// ----------------------------------------------------------------- small-M --

// One chunk's operands for one wave: NT weight code blocks, their scale pairs,
// and MG activation pieces.
template <int MG, int NT>
struct SmallSlot {
    uint4 cw[NT];
    uint32_t sw[NT];
    uint4 xa[MG];
};

// Scale table in LDS: entry b = {operand for the exponent-only conversion,
// remaining fp32 factor} of E4M3 byte b (split_scale).  Two LDS reads per
// lane and chunk replace the bit decoding of its two scales.
__device__ __forceinline__ void build_scale_table(float2* lut) {
    for (int b = threadIdx.x; b < 256; b += blockDim.x) {
        float cs, f;
        split_scale(e4m3_to_f32((uint32_t)b), cs, f);
        lut[b] = make_float2(cs, f);
    }
}

// Contract one 128-wide K chunk of NT units against MG row groups.  kin: the
// lane's activation piece lies below K; when KFULL (K a multiple of 128) it
// always does.  Pieces past K are zeroed here, at use, so that data read
// from the clamped address cannot reach the sums (the weights there are zero
// padding, but the activation might not be finite).
template <int MG, int NT, bool KFULL>
__device__ __forceinline__ void small_m_chunk(const SmallSlot<MG, NT>& s, bool kin, const float2* lut,
                                              f32x4 (&acc)[NT][MG]) {
    s16x4 alo[MG], ahi[MG];
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) {
        const uint4 v = s.xa[mg];
        if (KFULL) {
            alo[mg] = dwords_to_s16x4(v.x, v.y);
            ahi[mg] = dwords_to_s16x4(v.z, v.w);
        } else {
            alo[mg] = dwords_to_s16x4(kin ? v.x : 0u, kin ? v.y : 0u);
            ahi[mg] = dwords_to_s16x4(kin ? v.z : 0u, kin ? v.w : 0u);
        }
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const float2 s0 = lut[s.sw[j] & 0xFFu], s1 = lut[(s.sw[j] >> 8) & 0xFFu];
        const uint4 cw = s.cw[j];
        const s16x4 b0 = decode4_bf16_pow2<0>(cw.x, s0.x), b1 = decode4_bf16_pow2<2>(cw.x, s0.x);
        const s16x4 b2 = decode4_bf16_pow2<0>(cw.y, s0.x), b3 = decode4_bf16_pow2<2>(cw.y, s0.x);
        const s16x4 b4 = decode4_bf16_pow2<0>(cw.z, s1.x), b5 = decode4_bf16_pow2<2>(cw.z, s1.x);
        const s16x4 b6 = decode4_bf16_pow2<0>(cw.w, s1.x), b7 = decode4_bf16_pow2<2>(cw.w, s1.x);
#pragma unroll
        for (int mg = 0; mg < MG; ++mg) {
            f32x4 p = {0.f, 0.f, 0.f, 0.f};
            p = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(alo[mg], b0, p, 2, 0, 0);
            p = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ahi[mg], b1, p, 2, 0, 0);
            p = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(alo[mg], b2, p, 2, 1, 0);
            p = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ahi[mg], b3, p, 2, 1, 0);
            f32x4 r = {0.f, 0.f, 0.f, 0.f};
            r = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(alo[mg], b4, r, 2, 2, 0);
            r = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ahi[mg], b5, r, 2, 2, 0);
            r = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(alo[mg], b6, r, 2, 3, 0);
            r = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ahi[mg], b7, r, 2, 3, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[j][mg][i] = __builtin_fmaf(s1.y, r[i], __builtin_fmaf(s0.y, p[i], acc[j][mg][i]));
        }
    }
}

// One wave's share of a pass: rows [0, rows) (rows <= 4 MG) of the activation
// block starting at xrow0, NT consecutive units whose code / scale blocks
// start at the wave-uniform cbase / sbase (unit j, chunk c at + j * ustr +
// c * cstr code bytes, an eighth of that in scale bytes), K chunks [c0, c1).  Operands of the next D chunks are kept in flight in a
// register ring.  Lane l = 16 g + 4 q + i holds rows 4 mg + i of the
// activation at k = 128 c + 32 g + 8 q .. +7; MFMA step t (k = 32 g + 4 t ..
// +3) broadcasts A from block q = t >> 1 of each group of four blocks
// (cbsz = 2, abid = t >> 1).  On return the wave's partial sums, reduced over
// its four K groups, are in red_w[row * red_ld + col] for rows < 4 MG and
// cols < 16 NT.
template <int MG, int NT, int D, bool KFULL>
__device__ __forceinline__ void small_m_pass(const uint16_t* __restrict__ xrow0, int64_t ld_x, int rows,
                                             const uint8_t* __restrict__ cbase, const uint8_t* __restrict__ sbase,
                                             int64_t ustr, int64_t cstr, int nt_valid, int c0, int c1, int K,
                                             const float2* lut, float* red_w, int red_ld, int lane) {
    const int g = lane >> 4, q = (lane >> 2) & 3, ai = lane & 3;
    f32x4 acc[NT][MG];
    uint32_t xoff[MG];   // byte offset of the lane's activation piece in chunk 0
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) {
        const int m = 4 * mg + ai;
        xoff[mg] = (uint32_t)(((int64_t)(m < rows ? m : 0) * ld_x + g * 32 + q * 8) * 2);
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j][mg] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (c0 >= c1) {
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int mg = 0; mg < MG; ++mg)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (lane < 16) red_w[(4 * mg + i) * red_ld + j * 16 + lane] = 0.f;
        return;
    }

    // Loads are issued unconditionally from clamped, in-bounds addresses and
    // never masked at load time: a load under a lane-divergent branch, or a
    // select right after it, makes the compiler wait for the load there,
    // which would serialise the prefetch ring.  Rows past `rows` and units
    // past nt_valid read valid but unrelated data; they only feed output
    // rows / columns that are never stored.  Addresses are a wave-uniform
    // base plus a 32-bit lane offset.
    const int c_last = c1 - 1;
    const int kpiece = g * 32 + q * 8;
    const uint8_t* xb = reinterpret_cast<const uint8_t*>(xrow0);
    auto load = [&](SmallSlot<MG, NT>& s, int c_req) {
        const int c = c_req < c_last ? c_req : c_last;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int64_t jj = j < nt_valid ? j : 0;
            const int64_t boff = jj * ustr + (int64_t)c * cstr;   // wave-uniform
            s.cw[j] = load_stream_u4(cbase + boff + (uint32_t)(lane * 16));
            s.sw[j] = load_stream_u16(sbase + (boff >> 3) + (uint32_t)(lane * 2));
        }
        const uint32_t kb = (KFULL || c * kChunkK + kpiece < K) ? (uint32_t)(c * kChunkK * 2) : 0u;
#pragma unroll
        for (int mg = 0; mg < MG; ++mg) s.xa[mg] = *reinterpret_cast<const uint4*>(xb + (xoff[mg] + kb));
    };
    auto kin = [&](int c) { return KFULL || (c * kChunkK + kpiece < K); };

    // Straight-line main loop over D chunks (each slot is refilled D chunks
    // ahead as soon as it has been read), then a load-free tail for the last
    // (c1 - c0) % D chunks, which are already in the ring.
    SmallSlot<MG, NT> ring[D];
#pragma unroll
    for (int d = 0; d < D; ++d) load(ring[d], c0 + d);
    int c = c0;
    for (; c + D <= c1; c += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const SmallSlot<MG, NT> cur = ring[d];
            load(ring[d], c + D + d);
            small_m_chunk<MG, NT, KFULL>(cur, kin(c + d), lut, acc);
        }
    }
#pragma unroll
    for (int d = 0; d < D - 1; ++d)
        if (c + d < c1) small_m_chunk<MG, NT, KFULL>(ring[d], kin(c + d), lut, acc);

    // Sum the four K groups: lanes l, l^16, l^32, l^48 hold the same outputs;
    // lane l < 16 then holds column l of each unit, rows 4 mg + i.
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int mg = 0; mg < MG; ++mg)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = acc[j][mg][i];
                v += __shfl_xor(v, 16);
                v += __shfl_xor(v, 32);
                if (lane < 16) red_w[(4 * mg + i) * red_ld + j * 16 + lane] = v;
            }
}

// Rows 9..16 of a pass: v_mfma_f32_16x16x32_bf16 on fully scaled bf16
// weight fragments (decode8_bf16), 4 MFMAs per unit and chunk instead of the
// 32 the 4x4x4 form needs for 16 rows.  Lane l = 16 g + r holds activation
// row r at k = 128 c + 32 g + 8 t .. +7 for MFMA step t (four 16-byte pieces
// per chunk) and the codes of weight row 16 u + r at the same k; the MFMA
// sums over the four lane groups, so no K-group reduction is needed.  On
// return red_w[row * red_ld + col] holds the wave's partial sums for rows <
// 16 and cols < 16 NT.
template <int NT>
struct Slot16 {
    uint4 cw[NT];
    uint32_t sw[NT];
    uint4 xa[4];
};

template <int NT, int D, bool KFULL>
__device__ __forceinline__ void small_m_pass16(const uint16_t* __restrict__ xrow0, int64_t ld_x, int rows,
                                               const uint8_t* __restrict__ cbase, const uint8_t* __restrict__ sbase,
                                               int64_t ustr, int64_t cstr, int nt_valid, int c0, int c1, int K,
                                               const float2* lut, float* red_w, int red_ld, int lane) {
    const int g = lane >> 4, r = lane & 15;
    f32x4 acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t xoff = (uint32_t)(((int64_t)(r < rows ? r : 0) * ld_x + g * 32) * 2);
    if (c0 < c1) {
        const int c_last = c1 - 1;
        const uint8_t* xb = reinterpret_cast<const uint8_t*>(xrow0);
        auto load = [&](Slot16<NT>& s, int c_req) {
            const int c = c_req < c_last ? c_req : c_last;
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int64_t jj = j < nt_valid ? j : 0;
                const int64_t boff = jj * ustr + (int64_t)c * cstr;   // wave-uniform
                s.cw[j] = load_stream_u4(cbase + boff + (uint32_t)(lane * 16));
                s.sw[j] = load_stream_u16(sbase + (boff >> 3) + (uint32_t)(lane * 2));
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bool kin = KFULL || (c * kChunkK + g * 32 + t * 8 < K);
                s.xa[t] = *reinterpret_cast<const uint4*>(xb + xoff + (kin ? (uint32_t)((c * kChunkK + t * 8) * 2)
                                                                         : 0u));
            }
        };
        auto chunk = [&](const Slot16<NT>& s, int c) {
            bf16x8 a[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bool kin = KFULL || (c * kChunkK + g * 32 + t * 8 < K);
                const uint4 v = s.xa[t];
                a[t] = uint4_to_bf16x8(kin ? v : make_uint4(0u, 0u, 0u, 0u));
            }
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const float2 l0 = lut[s.sw[j] & 0xFFu], l1 = lut[(s.sw[j] >> 8) & 0xFFu];
                // the full scale: 2^exponent(conversion operand) times the factor, exact
                const float s0 = __uint_as_float(__float_as_uint(l0.x) & 0x7F800000u) * l0.y;
                const float s1 = __uint_as_float(__float_as_uint(l1.x) & 0x7F800000u) * l1.y;
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], uint4_to_bf16x8(decode8_bf16(s.cw[j].x, s0)), acc[j], 0, 0, 0);
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], uint4_to_bf16x8(decode8_bf16(s.cw[j].y, s0)), acc[j], 0, 0, 0);
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[2], uint4_to_bf16x8(decode8_bf16(s.cw[j].z, s1)), acc[j], 0, 0, 0);
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[3], uint4_to_bf16x8(decode8_bf16(s.cw[j].w, s1)), acc[j], 0, 0, 0);
            }
        };
        Slot16<NT> ring[D];
#pragma unroll
        for (int d = 0; d < D; ++d) load(ring[d], c0 + d);
        int c = c0;
        for (; c + D <= c1; c += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const Slot16<NT> cur = ring[d];
                load(ring[d], c + D + d);
                chunk(cur, c + d);
            }
        }
#pragma unroll
        for (int d = 0; d < D - 1; ++d)
            if (c + d < c1) chunk(ring[d], c + d);
    }
    // lane l holds rows 4 (l >> 4) + i of column l & 15 of each unit
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) red_w[(4 * g + i) * red_ld + j * 16 + r] = acc[j][i];
}

// Small-M GEMM: one workgroup per NT consecutive 16-row units of W (and per
// expert in the grouped form); its W waves split K into contiguous chunk
// ranges, and the per-wave partial sums are added in wave order through LDS.
// MG in 1..4: every pass uses MG row groups of the 4x4x4 form (rows <= 4 MG).
// MG == 16: every pass uses the 16x16x32 form (rows <= 16).
// MG == 0: each pass of up to 16 rows picks one or four row groups (grouped).
template <int MG, int NT, int W, int D, bool GROUPED, bool KFULL>
__global__ void __launch_bounds__(W * 64) k_gemm_small_m(const uint16_t* __restrict__ x, int64_t ld_x, BlobView bv,
                                                         int NU, int KC, int K,
                                                         int N, const float* __restrict__ gscale, int g_is_div,
                                                         uint16_t* __restrict__ y, int64_t ld_y, int64_t rows_dense,
                                                         const int32_t* __restrict__ offsets) {
    constexpr int RLD = NT * 16;
    __shared__ float red[W][kSmallRows * RLD];
    __shared__ float2 lut[256];
    const int u0 = blockIdx.x * NT;
    const int e = GROUPED ? (int)blockIdx.y : 0;
    int64_t row0 = 0, count = rows_dense;
    if (GROUPED) {
        row0 = offsets[e];
        count = (int64_t)offsets[e + 1] - row0;
    }
    if (count <= 0 || u0 >= NU) return;   // uniform over the workgroup
    build_scale_table(lut);

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: keeps the chunk loop scalar
    const int c0 = (int)((int64_t)KC * w / W), c1 = (int)((int64_t)KC * (w + 1) / W);
    const int nt_valid = (NU - u0) < NT ? (NU - u0) : NT;
    const int64_t blk0 = bv.block(e, u0, 0);
    const uint8_t* cbase = bv.codes + blk0 * kCodeBlock;
    const uint8_t* sbase = bv.scales + blk0 * kScaleBlock;
    const int64_t ustr = bv.unit_stride * kCodeBlock, cstr = bv.chunk_stride * kCodeBlock;
    const float gv = effective_global_scale(gscale[e], g_is_div);
    __syncthreads();   // scale table ready

    for (int64_t p0 = 0; p0 < count; p0 += kSmallRows) {
        const int rows = (int)((count - p0) < kSmallRows ? (count - p0) : kSmallRows);
        const uint16_t* xrow0 = x + (row0 + p0) * ld_x;
        if constexpr (MG == 16) {
            small_m_pass16<NT, D, KFULL>(xrow0, ld_x, rows, cbase, sbase, ustr, cstr, nt_valid, c0, c1, K, lut, red[w],
                                         RLD, lane);
        } else if constexpr (MG > 0) {
            small_m_pass<MG, NT, D, KFULL>(xrow0, ld_x, rows, cbase, sbase, ustr, cstr, nt_valid, c0, c1, K, lut,
                                           red[w], RLD, lane);
        } else {
            if (rows <= 4)
                small_m_pass<1, NT, D, KFULL>(xrow0, ld_x, rows, cbase, sbase, ustr, cstr, nt_valid, c0, c1, K, lut,
                                              red[w], RLD, lane);
            else
                small_m_pass<4, NT, (D > 2 ? 2 : D), KFULL>(xrow0, ld_x, rows, cbase, sbase, ustr, cstr, nt_valid, c0,
                                                           c1, K, lut, red[w], RLD, lane);
        }
        __syncthreads();
        for (int t = threadIdx.x; t < rows * RLD; t += W * 64) {
            const int r = t / RLD, col = t % RLD;
            float acc = 0.f;
#pragma unroll
            for (int ww = 0; ww < W; ++ww) acc += red[ww][r * RLD + col];
            const int64_t n = (int64_t)u0 * kUnitN + col;
            if (n < N) y[(row0 + p0 + r) * ld_y + n] = (uint16_t)f32_to_bf16_rne(gv * acc);
        }
        __syncthreads();
    }
}

}  // namespace nvfp4
