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
constexpr int kMfmaLds = 2 * kMfmaStage;       // double buffer

template <int NT, int WN, bool KFULL>
__global__ void __launch_bounds__(WN * 64) k_gemm_mfma(const uint16_t* __restrict__ x, int64_t ld_x, BlobView bv, int NU,
                                                   int KC, int K, int N, const float* __restrict__ gscale,
                                                   int g_is_div, uint16_t* __restrict__ y, int64_t ld_y, int M) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
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
    const uint8_t* xb = reinterpret_cast<const uint8_t*>(x);
    auto copy_a = [&](int c, int buf) {
#pragma unroll
        for (int k = 0; k < kCopiesPerWave; ++k) {
            const int i = (w + WN * k) < kCopies ? w + WN * k : w, row = 4 * i + (lane >> 4);
            uint32_t off = a_src[k] + (uint32_t)(c * kChunkK * 2);
            if (!KFULL && c * kChunkK + (q ^ (row & 15)) * 8 >= K) off = a_src[k] - (q ^ (row & 15)) * 16;   // k = 0 of the row
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(xb + off),
                                             (__attribute__((address_space(3))) void*)(smem + buf * kMfmaStage + i * 1024),
                                             16, 0, 0);
        }
    };
    // zero the staged pieces of the last chunk that lie at k >= K (their
    // copies read k = 0 of the row)
    auto zero_tail = [&](int buf) {
        const int c = KC - 1;
        for (int t = tid; t < kMfmaBM * 16; t += WN * 64) {
            const int row = t >> 4, slot = t & 15;
            if (c * kChunkK + (slot ^ (row & 15)) * 8 >= K)
                *reinterpret_cast<uint4*>(smem + buf * kMfmaStage + row * 256 + slot * 16) = make_uint4(0u, 0u, 0u, 0u);
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
    const uint32_t lane16 = (uint32_t)(lane * 16);
    struct BRegs {
        uint4 cw[NT];
        uint32_t sw[NT];
    };
    auto load_b = [&](BRegs& b, int c) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            b.cw[j] = load_stream_u4(cb[j] + (int64_t)c * cstr + lane16);
            b.sw[j] = load_scale_dword(sb[j] + (((int64_t)c * cstr) >> 3), lane);
        }
    };

    f32x4 acc[8][NT];
#pragma unroll
    for (int ms = 0; ms < 8; ++ms)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[ms][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One chunk: four MFMA steps; per step the B fragments of the wave's NT
    // units are decoded, then 8 x NT MFMAs run.  Two waves share each SIMD,
    // so one wave's decode overlaps the other's MFMAs.
    auto compute = [&](const BRegs& b, int buf) {
        float s0[NT], s1[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const uint32_t sp = scale_pair(b.sw[j], lane);
            const float2 l0 = lut[sp & 0xFFu], l1 = lut[(sp >> 8) & 0xFFu];
            s0[j] = __uint_as_float(__float_as_uint(l0.x) & 0x7F800000u) * l0.y;
            s1[j] = __uint_as_float(__float_as_uint(l1.x) & 0x7F800000u) * l1.y;
        }
        const uint8_t* abase = smem + buf * kMfmaStage + r * 256;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            bf16x8 bf[NT];
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const uint32_t d = t == 0 ? b.cw[j].x : t == 1 ? b.cw[j].y : t == 2 ? b.cw[j].z : b.cw[j].w;
                bf[j] = uint4_to_bf16x8(decode8_bf16(d, t < 2 ? s0[j] : s1[j]));
            }
#pragma unroll
            for (int ms = 0; ms < 8; ++ms) {
                const bf16x8 af = uint4_to_bf16x8(
                    *reinterpret_cast<const uint4*>(abase + ms * 16 * 256 + (((4 * g + t) ^ r) << 4)));
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    acc[ms][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[j], acc[ms][j], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);   // keep each step's fragments local (register pressure)
        }
    };

    // ---- chunk pipeline: one loop body per chunk, so the accumulators keep
    // one register assignment (an unrolled pair of bodies made the compiler
    // shuffle them between register files); the next chunk's weight
    // registers are copied into place once they have landed
    BRegs bc, bn;
    copy_a(0, 0);
    load_b(bc, 0);
    __builtin_amdgcn_s_waitcnt(0);
    if (!KFULL && KC == 1) zero_tail(0);
    __syncthreads();
    for (int c = 0; c < KC; ++c) {
        const int buf = c & 1;
        if (c + 1 < KC) {
            copy_a(c + 1, buf ^ 1);
            load_b(bn, c + 1);
        }
        compute(bc, buf);
        __builtin_amdgcn_s_waitcnt(0);   // chunk c + 1 landed (issued before chunk c was contracted)
        if (!KFULL && c + 1 == KC - 1) zero_tail(buf ^ 1);
        __syncthreads();                 // every wave is done with this buffer and sees the next
        bc = bn;
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
