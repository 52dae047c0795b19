// Dense GEMM for many rows (prefill-sized M): MFMA-bound.
//
//   Workgroup tile 128 rows x 16 NT WN columns: WN waves side by side, each
//   owning all 128 rows and NT units (16 NT columns) as 8 x NT tiles of
//   16 x 16 (v_mfma_f32_16x16x32_bf16, fp32 accumulators in AGPRs).  The
//   tile is wide in N because an activation byte costs 2 B per element and a
//   weight byte 0.5625: with 512 columns per workgroup each staged activation
//   chunk feeds 8 waves.  K advances one 128-wide chunk at a time:
//     - the activation chunk (128 rows x 256 bytes = 32 KB) is copied to LDS
//       with global_load_lds_dwordx4 (1 KB per copy: four rows), double
//       buffered, in the XOR-swizzled layout of the other kernels (slot q of
//       a 256-byte row holds piece q ^ (row & 15)), so every fragment read is
//       a conflict-free ds_read_b128;
//     - each wave loads its NT units' code blocks and scale pairs into
//       registers (one 128-bit and one 32-bit load per unit and lane) and
//       decodes them into exact bf16 B fragments (decode8_bf16);
//     - the loads of chunk c + 1 are issued before chunk c is contracted, so
//       the one barrier per chunk finds them landed.
//   The 32 K slots of an MFMA step map to k = 32 g + 8 t + e (lane group g,
//   step t, element e) on both operands, as in the tile kernel.
#pragma once
#include "decode.h"
#include "kernels_gemm.h"
#include "layout.h"

namespace nvfp4 {

constexpr int kMfmaBM = 128;                   // rows per workgroup tile
constexpr int kMfmaStage = kMfmaBM * 256;      // LDS bytes of one staged activation chunk

// LDS address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Asynchronous copy global -> LDS: lane l moves the 16 (4) bytes at
// base + voff (base wave-uniform) to LDS address lds + 16 l (4 l).  Written
// as inline assembly so that the compiler, which cannot tell which LDS bytes
// such a copy writes, does not wait for every copy in flight before each LDS
// read; the kernel waits for its own copies (vmcnt) before the barrier that
// publishes them.  M0 carries the LDS base and needs one wait state.
__device__ __forceinline__ void lds_copy16(uint32_t lds, const uint8_t* base, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(base)
                 : "memory", "m0");
}
__device__ __forceinline__ void lds_copy4(uint32_t lds, const uint8_t* base, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds), "v"(voff), "s"(base)
                 : "memory", "m0");
}

template <int NT, int WN, bool KFULL>
__global__ void __launch_bounds__(WN * 64) k_gemm_mfma(const uint16_t* __restrict__ x, int64_t ld_x, BlobView bv, int NU,
                                                   int KC, int K, int N, const float* __restrict__ gscale,
                                                   int g_is_div, uint16_t* __restrict__ y, int64_t ld_y, int M) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[2][kMfmaStage];            // activations
    __shared__ __attribute__((aligned(16))) uint8_t wcodes[2][WN][NT * kCodeBlock];   // per-wave weights
    __shared__ __attribute__((aligned(16))) uint8_t wscale[2][WN][NT * kScaleBlock];
    __shared__ float2 lut[256];
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr int kCopies = kMfmaBM / 4;                  // 1 KB activation copies per chunk
    constexpr int kCopiesPerWave = (kCopies + WN - 1) / WN;
    const int m0 = (int)blockIdx.y * kMfmaBM;
    const int u_w = (int)blockIdx.x * NT * WN + NT * w;   // this wave's first unit

    build_scale_table(lut);

    // ---- activation copies: copy i (0 .. kCopies - 1) of a chunk moves rows
    // 4 i .. 4 i + 3; wave w issues copies w, w + WN, ..; lane l takes row
    // 4 i + (l >> 4) and the piece stored in slot l & 15.  Rows past M read
    // row M - 1 (never stored); copies past kCopies repeat copy w.
    const int q = lane & 15;
    uint32_t a_src[kCopiesPerWave];   // byte offset of the lane's piece in chunk 0, per copy
#pragma unroll
    for (int k = 0; k < kCopiesPerWave; ++k) {
        const int i = (w + WN * k) < kCopies ? w + WN * k : w, row = 4 * i + (lane >> 4);
        const int grow = m0 + row < M ? m0 + row : M - 1;
        a_src[k] = (uint32_t)(((int64_t)grow * ld_x + (q ^ (row & 15)) * 8) * 2);
    }
    const uint8_t* xb = uniform_ptr(reinterpret_cast<const uint8_t*>(x));
    auto copy_a = [&](int c, int buf) {
        const uint32_t dst = lds_addr(stage[buf]);
#pragma unroll
        for (int k = 0; k < kCopiesPerWave; ++k) {
            const int i = (w + WN * k) < kCopies ? w + WN * k : w, row = 4 * i + (lane >> 4);
            uint32_t off = a_src[k] + (uint32_t)(c * kChunkK * 2);
            if (!KFULL && c * kChunkK + (q ^ (row & 15)) * 8 >= K) off = a_src[k] - (q ^ (row & 15)) * 16;   // k = 0 of the row
            lds_copy16(dst + i * 1024, xb, off);
        }
    };
    // zero the staged pieces of the last chunk that lie at k >= K (their
    // copies read k = 0 of the row)
    auto zero_tail = [&](uint8_t* dst) {
        const int c = KC - 1;
        for (int t = tid; t < kMfmaBM * 16; t += WN * 64) {
            const int row = t >> 4, slot = t & 15;
            if (c * kChunkK + (slot ^ (row & 15)) * 8 >= K)
                *reinterpret_cast<uint4*>(dst + row * 256 + slot * 16) = make_uint4(0u, 0u, 0u, 0u);
        }
    };

    // ---- weight blocks of this wave's NT units (units past NU read unit 0, never stored)
    const uint8_t* cb[NT];   // wave-uniform block bases; the lane offset is added at the load
    const uint8_t* sb[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int64_t blk = bv.block(0, (u_w + j) < NU ? u_w + j : 0, 0);
        cb[j] = bv.codes + blk * kCodeBlock;
        sb[j] = bv.scales + blk * kScaleBlock;
    }
    const int64_t cstr = bv.chunk_stride * kCodeBlock;
    // Weight copies of a chunk go to the wave's own LDS slice (no other wave
    // reads it, so only this wave's copies have to be waited for): NT code
    // blocks of 1 KB (lane l moves bytes 16 l .. 16 l + 15) and NT / 2 scale
    // copies of 256 B (lanes 0..31 move unit 2 p's 128-byte block, lanes
    // 32..63 unit 2 p + 1's).
    static_assert(NT % 2 == 0, "scale copies move two units");
    const uint32_t lane16 = (uint32_t)(lane * 16);
    // scale copy p: uniform base = the lower of the two blocks, per-lane
    // 32-bit offsets (so the copies use scalar-base addressing)
    const uint8_t* s_base[NT / 2];
    uint32_t s_off[NT / 2];
#pragma unroll
    for (int p = 0; p < NT / 2; ++p) {
        const uint8_t* lo = sb[2 * p] < sb[2 * p + 1] ? sb[2 * p] : sb[2 * p + 1];
        s_base[p] = lo;
        s_off[p] = (uint32_t)((lane < 32 ? sb[2 * p] : sb[2 * p + 1]) - lo) + (uint32_t)((lane & 31) * 4);
    }
    auto copy_b = [&](int c, int buf) {
        const int64_t co = (int64_t)c * cstr;
        const uint32_t codes = lds_addr(wcodes[buf][w]), scl = lds_addr(wscale[buf][w]);
#pragma unroll
        for (int j = 0; j < NT; ++j) lds_copy16(codes + j * kCodeBlock, uniform_ptr(cb[j] + co), lane16);
#pragma unroll
        for (int p = 0; p < NT / 2; ++p) lds_copy4(scl + p * 2 * kScaleBlock, uniform_ptr(s_base[p] + (co >> 3)), s_off[p]);
    };

    // ---- contraction of one chunk as 32 issue groups f = 8 t + ms (MFMA
    // step t, row block ms).  Group f issues the LDS read of activation
    // fragment f + 2 (three-slot ring), the NT MFMAs of fragment f against
    // the B fragments of step t, and a slice of the VALU work for step t + 1:
    // in steps 0..2 half a unit's decode (8 VALU per 4 MFMAs); in step 3 the
    // next chunk's code blocks and scales are read from LDS and its step-0
    // fragments decoded.  A scheduling fence closes every group, so each
    // MFMA has VALU work beside it and each LDS read two groups of lead.
    static_assert(NT == 4, "the issue groups spread 4 units' decode over 8 row blocks");
    uint4 cw[NT];             // the lane's 16 code bytes of each unit, this chunk
    float s0[NT], s1[NT];     // full scales of the lane's two 16-k blocks, per unit
    uint4 bfa[NT], bfb[NT];   // B fragments: even steps in bfa, odd steps in bfb
    uint32_t sp[NT];
    float2 l0[NT], l1[NT];

    auto read_b = [&](int buf) {   // code blocks and scale pairs of a staged chunk
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            cw[j] = *reinterpret_cast<const uint4*>(wcodes[buf][w] + j * kCodeBlock + lane16);
            sp[j] = *reinterpret_cast<const uint16_t*>(wscale[buf][w] + j * kScaleBlock + lane * 2);
        }
    };
    auto lut_b = [&]() {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            l0[j] = lut[sp[j] & 0xFFu];
            l1[j] = lut[sp[j] >> 8];
        }
    };
    auto scales_b = [&]() {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            s0[j] = __uint_as_float(__float_as_uint(l0[j].x) & 0x7F800000u) * l0[j].y;
            s1[j] = __uint_as_float(__float_as_uint(l1[j].x) & 0x7F800000u) * l1[j].y;
        }
    };
    // half h (elements 4 h .. 4 h + 3) of unit j's B fragment for step t
    auto decode_half = [&](int t, int j, int h, uint4& out) {
        const uint32_t d = t == 0 ? cw[j].x : t == 1 ? cw[j].y : t == 2 ? cw[j].z : cw[j].w;
        const float sc = t < 2 ? s0[j] : s1[j];
        const f32x2 p = h == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0)
                               : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
        const f32x2 q = h == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1)
                               : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
        const uint32_t lo = pack_hi_halves(p.x * sc, p.y * sc), hi = pack_hi_halves(q.x * sc, q.y * sc);
        if (h == 0) {
            out.x = lo;
            out.y = hi;
        } else {
            out.z = lo;
            out.w = hi;
        }
    };
    auto decode_full = [&](int t, int j, uint4& out) {
        decode_half(t, j, 0, out);
        decode_half(t, j, 1, out);
    };

    f32x4 acc[8][NT];
#pragma unroll
    for (int ms = 0; ms < 8; ++ms)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[ms][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto frag = [&](const uint8_t* a, int f) {   // activation fragment f = 8 t + ms
        const int t = f >> 3, ms = f & 7;
        return *reinterpret_cast<const uint4*>(a + (16 * ms + r) * 256 + (((4 * g + t) ^ r) << 4));
    };
    auto chunk = [&](int c, int buf) {
        const uint8_t* a = stage[buf];
        uint4 af[3];
        af[0] = frag(a, 0);
        af[1] = frag(a, 1);
#pragma unroll
        for (int f = 0; f < 32; ++f) {
            const int t = f >> 3, ms = f & 7;
            if (f + 2 < 32) af[(f + 2) % 3] = frag(a, f + 2);
            const uint4* bf = (t & 1) ? bfb : bfa;
            uint4* nb = (t & 1) ? bfa : bfb;   // step t + 1's fragments
#pragma unroll
            for (int j = 0; j < NT; ++j)
                acc[ms][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(uint4_to_bf16x8(af[f % 3]), uint4_to_bf16x8(bf[j]),
                                                                    acc[ms][j], 0, 0, 0);
            if (t < 3) {
                decode_half(t + 1, ms >> 1, ms & 1, nb[ms >> 1]);
            } else if (ms == 0) {
                // this wave's copies of chunk c + 1 landed.  In the last
                // chunk the other stage holds chunk c - 1: the reads and
                // decodes below run anyway (their results are not used), so
                // that none of their registers has to live across chunks.
                __builtin_amdgcn_s_waitcnt(0);
                read_b(buf ^ 1);
            } else if (ms == 1) {
                lut_b();
            } else if (ms == 2) {
                scales_b();
            } else if (ms < 7) {
                decode_full(0, ms - 3, nb[ms - 3]);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // VALU
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- chunk pipeline.  Chunk c is contracted from stage c & 1; the copies
    // of chunk c + 1 into the other stage are issued first and waited for in
    // the last MFMA step.  One barrier per chunk.
    copy_a(0, 0);
    copy_b(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    if (!KFULL && KC == 1) zero_tail(stage[0]);
    __syncthreads();
    read_b(0);
    lut_b();
    scales_b();
#pragma unroll
    for (int j = 0; j < NT; ++j) decode_full(0, j, bfa[j]);
    for (int c = 0; c < KC; ++c) {
        const int buf = c & 1;
        if (c + 1 < KC) {
            copy_a(c + 1, buf ^ 1);
            copy_b(c + 1, buf ^ 1);
        }
        chunk(c, buf);
        if (!KFULL && c + 1 == KC - 1) zero_tail(stage[buf ^ 1]);
        // every wave is done with stage `buf`, and the activation copies into
        // the other stage (waited for above by each wave) are published
        wait_lgkmcnt0();
        asm volatile("s_barrier" ::: "memory");
    }

    // ---- epilogue: lane (r, g) holds rows 16 ms + 4 g + i of column 16 (u_w + j) + r
    const float gv = effective_global_scale(gscale[0], g_is_div);
#pragma unroll
    for (int ms = 0; ms < 8; ++ms)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int64_t n = (int64_t)(u_w + j) * kUnitN + r;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + 16 * ms + 4 * g + i;
                if (m < M && n < N) y[(int64_t)m * ld_y + n] = (uint16_t)f32_to_bf16_rne(gv * acc[ms][j][i]);
            }
        }
}

}  // namespace nvfp4
