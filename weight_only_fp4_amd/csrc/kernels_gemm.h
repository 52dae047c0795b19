// W4A16 NVFP4 GEMM kernels for gfx950.
//
//   Y[m,n] = RNE(g * sum_k X'[m,k] * e2m1(code(n,k)) * e4m3(S[n,k/16]))
//
// X and Y are bf16, or fp16 with F16 (the same kernels; weights decode exactly
// to either type, MFMAs of that type, RNE to it in the epilogue).
//
// X' is the activation, multiplied by the pre-quant scale where each piece
// is loaded when one is given (PRE; prescale8: RNE(X * s), never written
// back to memory).  This file holds the small-M kernel, used for up to 4
// rows (the host planner's choice; a pass covers up to 16 rows):
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

// K split across workgroups (grid z).  Each split publishes its fp32 partial
// tile to the workspace and bumps the tile's counter; the workgroup that
// arrives last adds the S partials in split order 0..S-1 (independent of the
// arrival order, so results are bitwise reproducible), applies the epilogue
// and resets the counter to zero for the next call.  Partials are stored and
// loaded with device-scope (sc1) accesses, which are coherent across the
// XCDs' separate L2 caches; an agent-scope fence would instead write back and
// invalidate the whole L2 of the XCD.
struct SplitK {
    int S;              // K splits (grid z)
    float* partials;    // [S][tiles][tile floats], used when S > 1
    int* counters;      // [tiles], zero between calls
};

__device__ __forceinline__ void store_partial(float* p, float v) {
    __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_partial(const float* p) {
    return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT));
}

// Called by every thread of a workgroup after it has stored its split's
// partial with store_partial: waits until the stores are acknowledged, then
// bumps the counter of `tile`.  Returns true in the workgroup that arrived
// last (the one that must reduce); that workgroup also resets the counter.
__device__ __forceinline__ bool split_arrive(int* counters, int64_t tile, int S, int* s_flag) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);   // all of this wave's partial stores acknowledged
    __syncthreads();
    if (threadIdx.x == 0) {
        const int prev = atomicAdd(&counters[tile], 1);
        *s_flag = prev;
        if (prev == S - 1) __hip_atomic_store(&counters[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    return *s_flag == S - 1;
}

// ----------------------------------------------------------------- small-M --

// One chunk's operands for one wave: NT weight code blocks, their scale pairs,
// MG activation pieces and the pre-quant scale piece of their k (used with
// PRE only).
template <int MG, int NT>
struct SmallSlot {
    uint4 cw[NT];
    uint32_t sw[NT];
    uint4 xa[MG];
    uint4 pa;
};

// Scale table in LDS: entry b = {operand for the exponent-only conversion,
// remaining fp32 factor} of scale byte b (split_scale), an E4M3 byte or, with
// mx, an E8M0 byte (a power of two: the conversion applies all of it and the
// factor is 1, except 2^-127, an fp32 denormal, carried by the factor, and
// NaN).  Two LDS reads per lane and chunk replace the bit decoding of its two
// scales.
__device__ __forceinline__ void build_scale_table(float2* lut, int mx) {
    for (int b = threadIdx.x; b < 256; b += blockDim.x) {
        float cs, f;
        if (mx) {
            const bool special = b == 0 || b == 255;
            cs = special ? 1.0f : e8m0_to_f32((uint32_t)b);
            f = special ? e8m0_to_f32((uint32_t)b) : 1.0f;
        } else {
            split_scale(e4m3_to_f32((uint32_t)b), cs, f);
        }
        lut[b] = make_float2(cs, f);
    }
}

// Contract one 128-wide K chunk of NT units against MG row groups.  kin: the
// lane's activation piece lies below K; when KFULL (K a multiple of 128) it
// always does.  Pieces past K are zeroed here, at use, so that data read
// from the clamped address cannot reach the sums (the weights there are zero
// padding, but the activation might not be finite).
template <int MG, int NT, bool KFULL, bool F16, bool PRE>
__device__ __forceinline__ void small_m_chunk(const SmallSlot<MG, NT>& s, bool kin, const float2* lut, int lane,
                                              f32x4 (&acc)[NT][MG]) {
    s16x4 alo[MG], ahi[MG];
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) {
        const uint4 v = PRE ? prescale8<F16>(s.xa[mg], s.pa) : s.xa[mg];
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
        const uint32_t sp = scale_pair(s.sw[j], lane);
        const float2 s0 = lut[sp & 0xFFu], s1 = lut[(sp >> 8) & 0xFFu];
        const uint4 cw = s.cw[j];
        const s16x4 b0 = decode4_pow2<F16, 0>(cw.x, s0.x), b1 = decode4_pow2<F16, 2>(cw.x, s0.x);
        const s16x4 b2 = decode4_pow2<F16, 0>(cw.y, s0.x), b3 = decode4_pow2<F16, 2>(cw.y, s0.x);
        const s16x4 b4 = decode4_pow2<F16, 0>(cw.z, s1.x), b5 = decode4_pow2<F16, 2>(cw.z, s1.x);
        const s16x4 b6 = decode4_pow2<F16, 0>(cw.w, s1.x), b7 = decode4_pow2<F16, 2>(cw.w, s1.x);
#pragma unroll
        for (int mg = 0; mg < MG; ++mg) {
            f32x4 p = {0.f, 0.f, 0.f, 0.f};
            p = mma4<F16, 2, 0>(alo[mg], b0, p);
            p = mma4<F16, 2, 0>(ahi[mg], b1, p);
            p = mma4<F16, 2, 1>(alo[mg], b2, p);
            p = mma4<F16, 2, 1>(ahi[mg], b3, p);
            f32x4 r = {0.f, 0.f, 0.f, 0.f};
            r = mma4<F16, 2, 2>(alo[mg], b4, r);
            r = mma4<F16, 2, 2>(ahi[mg], b5, r);
            r = mma4<F16, 2, 3>(alo[mg], b6, r);
            r = mma4<F16, 2, 3>(ahi[mg], b7, r);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[j][mg][i] = __builtin_fmaf(s1.y, r[i], __builtin_fmaf(s0.y, p[i], acc[j][mg][i]));
        }
    }
}

// Prefetch ring over n chunks (indices 0..n-1) of one wave: D slots, each
// consumed and then refilled with the chunk D ahead.  Scheduling barriers pin
// the issue order, so the wait before a slot's use only covers loads issued
// D - 1 slots earlier (left to itself the scheduler sinks refills to the end
// of the unrolled body and drains the ring every D chunks).  The steady loop
// runs only while every refill is in range, so its wait counts are static
// and no chunk is loaded twice; the last < 2D chunks drain with guarded
// refills.  `mid` runs once, after the first D loads are issued (the caller
// builds its LDS tables and synchronises there, under the load latency).
// Every wave must call this (mid may hold a barrier).  The first D loads are
// unconditional (a conditional prologue leaves the compiler unable to count
// them at the loop head), so load(slot, 0) must be in bounds even when
// n == 0; chunks past n - 1 repeat chunk n - 1 (short waves only).
template <int D, typename Slot, typename LoadF, typename UseF, typename MidF>
__device__ __forceinline__ void run_ring(int n, LoadF&& load, UseF&& use, MidF&& mid) {
    Slot ring[D];
    const int last = n > 1 ? n - 1 : 0;
#pragma unroll
    for (int d = 0; d < D; ++d) {
        load(ring[d], d < last ? d : last);
        __builtin_amdgcn_sched_barrier(0);
    }
    mid();
    if (n <= 0) return;
    int i = 0;
    for (; i + 2 * D <= n; i += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            use(ring[d], i + d);
            __builtin_amdgcn_sched_barrier(0);
            load(ring[d], i + D + d);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
        if (i + d < n) use(ring[d], i + d);
        if (i + D + d < n) load(ring[d], i + D + d);
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
        if (i + D + d < n) use(ring[d], i + D + d);
}

// Weight-side addressing of one wave: NT consecutive units whose code / scale
// blocks start at the wave-uniform cbase / sbase (unit j, chunk c at
// + j * ustr + c * cstr code bytes, an eighth of that in scale bytes).  Units
// past nt_valid re-read unit 0 (their columns are never stored).
struct WaveWeights {
    const uint8_t* cbase;
    const uint8_t* sbase;
    int64_t ustr, cstr;
    int nt_valid;
    template <int NT>
    __device__ __forceinline__ void load(uint4 (&cw)[NT], uint32_t (&sw)[NT], int c, int lane) const {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int64_t jj = j < nt_valid ? j : 0;
            const int64_t boff = jj * ustr + (int64_t)c * cstr;   // wave-uniform
            cw[j] = load_stream_u4(cbase + boff + (uint32_t)(lane * 16));
            sw[j] = load_scale_dword(sbase + (boff >> 3), lane);
        }
    }
};

// One wave's share of a pass in the 4x4x4 form: rows [0, rows) (rows <= 4 MG)
// of the activation block starting at xrow0, NT units, chunks [c0, c1).  Lane
// l = 16 g + 4 q + i holds rows 4 mg + i of the activation at k = 128 c +
// 32 g + 8 q .. +7 (for each row group, the 16 lanes of a row read its 256
// contiguous bytes of the chunk); MFMA step t (k = 32 g + 4 t .. +3)
// broadcasts A from block q = t >> 1 of each group of four blocks (cbsz = 2,
// abid = t >> 1).  On return the wave's partial sums, reduced over its four K
// groups, are in red_w[row * red_ld + col] for rows < 4 MG, cols < 16 NT.
template <int MG, int NT, int D, bool KFULL, bool F16, bool PRE, typename MidF>
__device__ __forceinline__ void small_m_pass(const uint16_t* __restrict__ xrow0, int64_t ld_x, int rows,
                                             const uint16_t* __restrict__ pre, const WaveWeights& ww, int c0,
                                             int c1, int K, const float2* lut, float* red_w, int red_ld, int lane,
                                             MidF&& mid, const int32_t* __restrict__ rix = nullptr) {
    const int g = lane >> 4, q = (lane >> 2) & 3, ai = lane & 3;
    f32x4 acc[NT][MG];
    uint32_t xoff[MG];   // byte offset of the lane's activation row (row rix[m] of xrow0 when gathering)
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) {
        const int m = 4 * mg + ai, mm = m < rows ? m : 0;
        xoff[mg] = (uint32_t)((int64_t)(rix ? rix[mm] : mm) * ld_x * 2);
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j][mg] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // Loads are issued unconditionally from in-bounds addresses and masked
    // only at use: a load under a lane-divergent branch, or a select right
    // after it, makes the compiler wait for the load there.  Rows past
    // `rows` read row 0 and only feed output rows that are never stored;
    // activation pieces past K read k = 0..7 of their row (valid: K >= 16)
    // and are zeroed at use.
    const int kpiece = g * 32 + q * 8;
    const uint8_t* xb = reinterpret_cast<const uint8_t*>(xrow0);
    auto kin = [&](int c) { return KFULL || (c * kChunkK + kpiece < K); };
    auto load = [&](SmallSlot<MG, NT>& s, int i) {
        const int c = c0 + i;
        ww.load<NT>(s.cw, s.sw, c, lane);
        const uint32_t kb = kin(c) ? (uint32_t)((c * kChunkK + kpiece) * 2) : 0u;
#pragma unroll
        for (int mg = 0; mg < MG; ++mg) s.xa[mg] = *reinterpret_cast<const uint4*>(xb + (xoff[mg] + kb));
        if constexpr (PRE) s.pa = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(pre) + kb);
    };
    auto use = [&](const SmallSlot<MG, NT>& s, int i) {
        small_m_chunk<MG, NT, KFULL, F16, PRE>(s, kin(c0 + i), lut, lane, acc);
    };
    run_ring<D, SmallSlot<MG, NT>>(c1 - c0, load, use, mid);

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

// One wave's share of a pass in the 16x16x32 form (rows <= 16):
// v_mfma_f32_16x16x32_bf16 on fully scaled bf16 weight fragments
// (decode8_bf16), 4 MFMAs per unit and chunk.  Lane l = 16 g + r holds
// activation row r at k = 128 c + 32 g + 8 t .. +7 for MFMA step t (four
// 16-byte pieces per chunk) and the codes of weight row 16 u + r at the same
// k; the MFMA sums over the four lane groups.  On return red_w[row * red_ld
// + col] holds the wave's partial sums for rows < 16 and cols < 16 NT.
template <int NT>
struct Slot16 {
    uint4 cw[NT];
    uint32_t sw[NT];
    uint4 xa[4];
    uint4 pa[4];   // pre-quant scale pieces (PRE only)
};

template <int NT, int D, bool KFULL, bool F16, bool PRE, typename MidF>
__device__ __forceinline__ void small_m_pass16(const uint16_t* __restrict__ xrow0, int64_t ld_x, int rows,
                                               const uint16_t* __restrict__ pre, const WaveWeights& ww, int c0,
                                               int c1, int K, const float2* lut, float* red_w, int red_ld, int lane,
                                               MidF&& mid) {
    const int g = lane >> 4, r = lane & 15;
    f32x4 acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t xoff = (uint32_t)((int64_t)(r < rows ? r : 0) * ld_x * 2);   // the lane's activation row
    const uint8_t* xb = reinterpret_cast<const uint8_t*>(xrow0);
    auto kin = [&](int c, int t) { return KFULL || (c * kChunkK + g * 32 + t * 8 < K); };
    auto load = [&](Slot16<NT>& s, int i) {
        const int c = c0 + i;
        ww.load<NT>(s.cw, s.sw, c, lane);
        // pieces past K read k = 0..7 of the row (valid: K >= 16) and are zeroed at use
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t kb = kin(c, t) ? (uint32_t)((c * kChunkK + g * 32 + t * 8) * 2) : 0u;
            s.xa[t] = *reinterpret_cast<const uint4*>(xb + xoff + kb);
            if constexpr (PRE) s.pa[t] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(pre) + kb);
        }
    };
    auto use = [&](const Slot16<NT>& s, int i) {
        const int c = c0 + i;
        uint4 a[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint4 v = PRE ? prescale8<F16>(s.xa[t], s.pa[t]) : s.xa[t];
            a[t] = kin(c, t) ? v : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const uint32_t sp = scale_pair(s.sw[j], lane);
            const float2 l0 = lut[sp & 0xFFu], l1 = lut[(sp >> 8) & 0xFFu];
            if constexpr (F16) {
                // the table's split as is: exponent in the conversion, the factor
                // (exact in fp16, or 0 / NaN for the special bytes) by fp16 pairs
                const _Float16 f0 = (_Float16)l0.y, f1 = (_Float16)l1.y;
                const HalfScale h0{l0.x, f16x2v{f0, f0}}, h1{l1.x, f16x2v{f1, f1}};
                acc[j] = mma16<F16>(a[0], decode8_f16_split(s.cw[j].x, h0), acc[j]);
                acc[j] = mma16<F16>(a[1], decode8_f16_split(s.cw[j].y, h0), acc[j]);
                acc[j] = mma16<F16>(a[2], decode8_f16_split(s.cw[j].z, h1), acc[j]);
                acc[j] = mma16<F16>(a[3], decode8_f16_split(s.cw[j].w, h1), acc[j]);
            } else {
                // the full scale: 2^exponent(conversion operand) times the factor, exact
                const float s0 = __uint_as_float(__float_as_uint(l0.x) & 0x7F800000u) * l0.y;
                const float s1 = __uint_as_float(__float_as_uint(l1.x) & 0x7F800000u) * l1.y;
                acc[j] = mma16<F16>(a[0], decode8<F16>(s.cw[j].x, s0), acc[j]);
                acc[j] = mma16<F16>(a[1], decode8<F16>(s.cw[j].y, s0), acc[j]);
                acc[j] = mma16<F16>(a[2], decode8<F16>(s.cw[j].z, s1), acc[j]);
                acc[j] = mma16<F16>(a[3], decode8<F16>(s.cw[j].w, s1), acc[j]);
            }
        }
    };
    run_ring<D, Slot16<NT>>(c1 - c0, load, use, mid);
    // lane l holds rows 4 (l >> 4) + i of column l & 15 of each unit
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) red_w[(4 * g + i) * red_ld + j * 16 + r] = acc[j][i];
}

// Small-M GEMM: one workgroup per NT consecutive 16-row units of W (and per
// expert in the grouped form); its W waves split the workgroup's K range into
// contiguous chunk ranges, and the per-wave partial sums are added in wave
// order through LDS.  The dense form may also split K across S workgroups
// (grid z, SplitK).
// MG in 1, 2, 4: every pass uses MG row groups of the 4x4x4 form (rows <= 4 MG).
// MG == 16: every pass uses the 16x16x32 form (rows <= 16).
// MG == 0: each pass of up to 16 rows picks one or four row groups (grouped).
// The first weight loads of a wave are issued before the scale table is
// built, so the table build and its barrier run under the load latency.
// ACT (grouped form): the MoE activation the epilogue applies (kActNone,
// kActSiluGlu with NT even: each workgroup holds gate / up unit pairs and
// writes N / 2 columns, kActRelu2).
template <int MG, int NT, int W, int D, bool GROUPED, bool KFULL, bool F16 = false, bool PRE = false,
          int ACT = kActNone>
__global__ void __launch_bounds__(W * 64) k_gemm_small_m(const uint16_t* __restrict__ x, int64_t ld_x, BlobView bv,
                                                         int NU, int KC, int K,
                                                         int N, const float* __restrict__ gscale, int g_is_div,
                                                         uint16_t* __restrict__ y, int64_t ld_y, int64_t rows_dense,
                                                         const int32_t* __restrict__ offsets, SplitK sk,
                                                         const int32_t* __restrict__ row_index,
                                                         const uint16_t* __restrict__ pre) {
    constexpr int RLD = NT * 16;
    constexpr int kTileFloats = kSmallRows * RLD;
    constexpr int kPer = (kTileFloats + W * 64 - 1) / (W * 64);   // partial-tile floats per thread
    __shared__ float red[W][kTileFloats];
    __shared__ float2 lut[256];
    __shared__ int s_flag;
    const int u0 = blockIdx.x * NT;
    const int e = GROUPED ? (int)blockIdx.y : 0;
    int64_t row0 = 0, count = rows_dense;
    if (GROUPED) {
        row0 = offsets[e];
        count = (int64_t)offsets[e + 1] - row0;
    }
    if (count <= 0 || u0 >= NU) return;   // uniform over the workgroup

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: keeps the chunk loop scalar
    // this split's chunks [C0, C0 + span), this wave's [c0, c1); c0 <= KC - 1
    // even for an empty range, so the ring's unconditional first loads stay
    // in bounds
    const int S = GROUPED ? 1 : sk.S, s = GROUPED ? 0 : (int)blockIdx.z;
    const int C0 = (int)((int64_t)KC * s / S), span = (int)((int64_t)KC * (s + 1) / S) - C0;
    const int c0 = C0 + (int)((int64_t)span * w / W), c1 = C0 + (int)((int64_t)span * (w + 1) / W);
    const int64_t blk0 = bv.block(e, u0, 0);
    const WaveWeights ww{bv.codes + blk0 * kCodeBlock, bv.scales + blk0 * kScaleBlock,
                         bv.unit_stride * kCodeBlock, bv.chunk_stride * kCodeBlock,
                         (NU - u0) < NT ? (NU - u0) : NT};
    bool first = true;
    auto mid = [&]() {
        if (first) {
            build_scale_table(lut, bv.mx);
            // scale table ready.  Only LDS writes need to be visible, so the
            // barrier waits for lgkmcnt alone: the compiler's own barrier
            // would wait for every outstanding load (the ring's first slots)
            // whenever copies into LDS are in flight.
            wait_lgkmcnt0();
            asm volatile("s_barrier" ::: "memory");
            first = false;
        }
    };

    // rows per pass: 16 for the dynamic form (MG = 0) and the 16-row form, 4 MG otherwise (a grouped
    // expert with more rows takes several passes, each streaming its weights again)
    constexpr int kPass = MG == 0 || MG == 16 ? kSmallRows : 4 * MG;
    for (int64_t p0 = 0; p0 < count; p0 += kPass) {
        const int rows = (int)((count - p0) < kPass ? (count - p0) : kPass);
        // grouped row r reads activation row row_index[r] when gathering
        const int32_t* rix = GROUPED && row_index ? row_index + row0 + p0 : nullptr;
        const uint16_t* xrow0 = rix ? x : x + (row0 + p0) * ld_x;
        if constexpr (MG == 16) {
            small_m_pass16<NT, D, KFULL, F16, PRE>(xrow0, ld_x, rows, pre, ww, c0, c1, K, lut, red[w], RLD, lane, mid);
        } else if constexpr (MG > 0) {
            small_m_pass<MG, NT, D, KFULL, F16, PRE>(xrow0, ld_x, rows, pre, ww, c0, c1, K, lut, red[w], RLD, lane,
                                                     mid, rix);
        } else {
            if (rows <= 4)
                small_m_pass<1, NT, D, KFULL, F16, PRE>(xrow0, ld_x, rows, pre, ww, c0, c1, K, lut, red[w], RLD, lane,
                                                        mid, rix);
            else
                small_m_pass<4, NT, (D > 2 ? 2 : D), KFULL, F16, PRE>(xrow0, ld_x, rows, pre, ww, c0, c1, K, lut, red[w],
                                                                      RLD, lane, mid, rix);
        }
        __syncthreads();
        const float gv = global_scale_at(gscale, e, g_is_div);
        auto store_y = [&](int t, float acc) {
            const int r = t / RLD, col = t % RLD;
            const int64_t n = (int64_t)u0 * kUnitN + col;
            uint32_t v = round_out<F16>(scale_acc(gv, acc));
            if constexpr (ACT == kActRelu2) v = round_out<F16>(relu_squared(act_to_f32<F16>(v)));
            if (n < N) y[(row0 + p0 + r) * ld_y + n] = (uint16_t)v;
        };
        if (S == 1) {
            if constexpr (ACT == kActSiluGlu) {
                // unit 2 j + 1 of the pair holds the up projection of unit 2 j's
                // columns; output column 16 (u0 / 2 + j) + c, N / 2 columns
                static_assert(NT % 2 == 0, "gate / up units come in pairs");
                constexpr int kHalf = RLD / 2;
                for (int t = threadIdx.x; t < rows * kHalf; t += W * 64) {
                    const int r = t / kHalf, pj = (t % kHalf) >> 4, c = t & 15;
                    const int tg = r * RLD + pj * 2 * kUnitN + c;
                    float ag = 0.f, au = 0.f;
#pragma unroll
                    for (int wi = 0; wi < W; ++wi) {
                        ag += red[wi][tg];
                        au += red[wi][tg + kUnitN];
                    }
                    const int64_t n = ((int64_t)u0 / 2 + pj) * kUnitN + c;
                    const float hg = act_to_f32<F16>(round_out<F16>(scale_acc(gv, ag)));
                    const float hu = act_to_f32<F16>(round_out<F16>(scale_acc(gv, au)));
                    if (n < N / 2) y[(row0 + p0 + r) * ld_y + n] = (uint16_t)round_out<F16>(silu_times(hg, hu));
                }
            } else {
                for (int t = threadIdx.x; t < rows * RLD; t += W * 64) {
                    float acc = 0.f;
#pragma unroll
                    for (int wi = 0; wi < W; ++wi) acc += red[wi][t];
                    store_y(t, acc);
                }
            }
            __syncthreads();
            continue;
        }
        // split K (dense form, one pass): publish, the last arrival reduces
        const int64_t tile = blockIdx.x, tiles = gridDim.x;
        float part[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int t = threadIdx.x + i * W * 64;
            part[i] = 0.f;
            if (t < rows * RLD) {
#pragma unroll
                for (int wi = 0; wi < W; ++wi) part[i] += red[wi][t];
                store_partial(sk.partials + ((int64_t)s * tiles + tile) * kTileFloats + t, part[i]);
            }
        }
        if (!split_arrive(sk.counters, tile, S, &s_flag)) return;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int t = threadIdx.x + i * W * 64;
            if (t < rows * RLD) {
                float acc = 0.f;   // splits added in order 0..S-1 whichever arrived last
                for (int ss = 0; ss < S; ++ss)
                    acc += ss == s ? part[i] : load_partial(sk.partials + ((int64_t)ss * tiles + tile) * kTileFloats + t);
                store_y(t, acc);
            }
        }
        return;
    }
}

}  // namespace nvfp4
