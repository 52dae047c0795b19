// Dense GEMM for many rows (prefill-sized M): MFMA-bound.
//
//   One wave per SIMD, four per workgroup.  A wave owns 16 MS rows x 64
//   columns (NT = 4 units) as MS x 4 tiles of 16 x 16, contracted with
//   v_mfma_f32_16x16x32_bf16; a workgroup owns 16 MS rows x 256 columns.
//   The cost that bounds this kernel beside the MFMAs is decoding the weights
//   (about two VALU per decoded element); a decoded B fragment feeds MS
//   MFMAs, so the tall wave tile (MS = 16: 256 rows, 256 accumulators, which
//   needs the register file of a wave that has its SIMD to itself) halves the
//   decode per MFMA of a 128-row tile.
//
//   K advances one 128-wide chunk at a time:
//     - the activation chunk (16 MS rows x 256 bytes) is copied into LDS with
//       asynchronous global -> LDS copies, double buffered, in the
//       XOR-swizzled layout (slot q of a 256-byte row holds piece q ^ (row &
//       15)), so every fragment read is a conflict-free ds_read_b128;
//     - each wave copies its four units' code and scale blocks into its own
//       LDS slice a chunk ahead, reads them into registers when the chunk's
//       first decode is due, and decodes them into exact bf16 fragments;
//     - the chunk is issued as 4 MS groups (MFMA step t, row block ms): the
//       LDS read of the fragment three groups ahead, the four MFMAs of the
//       group, and a slice of the next step's decode, closed by a
//       scheduling fence, so that every MFMA has independent work beside it.
//   The MFMA takes the weights as its first operand, so the accumulators hold
//   the transposed tile: a lane ends with four adjacent output columns of one
//   row (one 8-byte store).  The 32 K slots of a step map to k = 32 g + 8 t +
//   e (lane group g, step t, element e) on both operands.
#pragma once
#include <type_traits>

#include "decode.h"
#include "kernels_gemm.h"
#include "layout.h"

namespace nvfp4 {

constexpr int kMfmaNT = 4;                                 // units per wave
constexpr int kMfmaWN = 4;                                 // waves per workgroup, one per SIMD
constexpr int kMfmaUnits = kMfmaNT * kMfmaWN;              // units per workgroup tile (256 columns)
constexpr int kMfmaTileRows = 256;                         // rows of a whole tile (MS = 16)

// LDS address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Asynchronous copy global -> LDS: lane l moves the 16 (lds_copy4: 4) bytes
// at base + voff (base wave-uniform) to LDS address lds + 16 l (4 l).  Written as inline assembly
// so that the compiler, which cannot tell which LDS bytes such a copy
// writes, does not wait for every copy in flight before each LDS read; the
// kernel waits for its own copies (vmcnt) before the barrier that publishes
// them.  The compiler inserts no wait states around the statement, so it
// carries its own: M0 (the LDS base) needs one after it is written, and the
// base address is first copied by a scalar move into a scratch pair that the
// load reads, because a vector instruction writing the base (as the compiler
// does when it restores a spilled scalar with v_readlane) needs five wait
// states before a memory instruction reads it, while a scalar read of it is
// interlocked.  The move is also M0's wait state.
__device__ __forceinline__ void lds_copy16(uint32_t lds, const uint8_t* base, uint32_t voff) {
    uint64_t tmp;
    asm volatile("s_mov_b32 m0, %1\n\ts_mov_b64 %0, %3\n\tglobal_load_lds_dwordx4 %2, %0"
                 : "=&s"(tmp)
                 : "s"(lds), "v"(voff), "s"(base)
                 : "memory", "m0");
}

// acc += A . B for one 16 x 16 x 32 bf16 step, accumulating in place in
// accumulation registers.  Written as inline assembly because the compiler,
// left to itself, renames most accumulators of a 256-accumulator tile in
// every chunk and copies them back through VGPRs at the loop edge.
//
// The compiler inserts no wait states around an MFMA it cannot see.  CDNA3
// and CDNA4 need two between a VALU write of a VGPR and an MFMA reading it as
// a source; the issue groups below produce every operand at least one group
// ahead, which the scheduler keeps apart in every form built, but only the
// generated code can show it: the library build checks the assembly of every
// form of this kernel (isa_check.py) and refuses to link one in which an
// operand is written fewer than two wait states before its MFMA (a stale
// operand read then depends on how the waves of the compute unit happen to
// issue).  A fixed s_nop here would cost about a tenth of the prefill rate,
// the loop being bound by instruction issue.  The accumulators are only ever
// written by these statements (same size, full overlap: no wait needed
// between them) and read after the drain in mfma_drain.
template <bool F16>
__device__ __forceinline__ void mfma_acc(f32x4& acc, const uint4& a, const uint4& b) {
    if constexpr (F16)
        asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0"
            : "+a"(acc)
            : "v"(__builtin_bit_cast(u32x4v, a)), "v"(__builtin_bit_cast(u32x4v, b)));
    else
        asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
            : "+a"(acc)
            : "v"(__builtin_bit_cast(u32x4v, a)), "v"(__builtin_bit_cast(u32x4v, b)));
}
// Wait states after the last MFMA before its accumulators are read (more
// than the longest MFMA pipeline).
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// Exchange rows of 16 lanes between two registers: odd rows of a with even
// rows of b (lane_swap16), rows 2-3 of a with rows 0-1 of b (lane_swap32).
__device__ __forceinline__ void lane_swap16(uint32_t& a, uint32_t& b) {
    const auto v = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = v[0];
    b = v[1];
}
__device__ __forceinline__ void lane_swap32(uint32_t& a, uint32_t& b) {
    const auto v = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = v[0];
    b = v[1];
}

// Calls f(std::integral_constant<int, i>) for i = I .. N - 1: a loop whose
// index is a compile-time constant in every iteration (register arrays
// indexed by it stay in registers however large the body).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

__device__ __forceinline__ void lds_copy4(uint32_t lds, const uint8_t* base, uint32_t voff) {
    uint64_t tmp;
    asm volatile("s_mov_b32 m0, %1\n\ts_mov_b64 %0, %3\n\tglobal_load_lds_dword %2, %0"
                 : "=&s"(tmp)
                 : "s"(lds), "v"(voff), "s"(base)
                 : "memory", "m0");
}

// Output tile (mt, nt) at position t of the tile order, which walks four
// tile rows at a time across all tile columns (the workgroups running
// together then share activation rows and weight columns in the caches).
__device__ __forceinline__ void mfma_tile(int t, int MT, int NTn, int& mt, int& nt) {
    constexpr int kGroupRows = 4;
    const int grp = t / (kGroupRows * NTn), in = t % (kGroupRows * NTn);
    const int rows = MT - grp * kGroupRows < kGroupRows ? MT - grp * kGroupRows : kGroupRows;
    mt = grp * kGroupRows + in % rows;
    nt = in / rows;
}

// Work item p (the workgroup id after the XCD remap below) covers part p % P
// (P = 16 / MS row parts of 16 MS rows) of tile t0 + p / P of the tile order
// (whole tiles are 256 rows x 256 columns).
//
// Synchronisation of the asynchronous copies.  Every copy a wave issues is
// counted by its own vmcnt, in issue order; the wave waits on exact counts
// derived from the fixed issue schedule of a chunk (below), so nothing it
// reads from LDS, and nothing another wave reads after the chunk's barrier,
// can still be in flight, whatever the relative speed of the waves and of
// other workgroups on the compute unit.  Per chunk c a wave issues, in order:
// [PRE: the pre-scale chunk of c + 1], its kCopiesPerWave activation copies
// of chunk c + 1 (groups 0, 2, ..), then the kWCopies weight copies of chunk
// c + 2 (groups kReadB + 1, kReadB + 2, after the wait at kReadB that retires
// the weight copies of chunk c + 1).  The barrier wait must retire the
// activation copies of chunk c + 1: it may leave the weight copies of c + 2
// in flight only when they were issued before it (tall tiles); with 64-row
// tiles they go out after the barrier, and the wait must then be for zero
// (waiting for kWCopies there, as an earlier form of this kernel did, left up
// to kWCopies activation copies in flight past the barrier, a race whose
// outcome depends on timing, and so on what else shares the compute unit).
// The wave drains every copy before it exits, so no copy can land in the LDS
// of a workgroup that starts on the compute unit after it.
//
// Grouped (MoE) form (GROUPED, 256-row tiles): the work items are (row tile of
// an expert, in expert order; tile column), the row tiles counted from
// expert_offsets by a prefix scan in every workgroup, and dealt to the XCDs
// in contiguous ranges (workgroup id i takes item (i % 8) * per + i / 8,
// per = ceil(items / 8); the host's grid holds 8 workgroups beyond the items
// so every item has an id).  An expert's rows end anywhere: the row blocks of
// 16 past its last row skip their MFMAs (the copies and the decode run as in
// a whole tile, keeping the copy schedule), so an expert of m rows costs the
// decode of its weights once per tile column and MFMAs for ceil(m / 16) row
// blocks.  row_index (optional): grouped row r reads activation row
// row_index[r].  ACT: the MoE activation of the epilogue (decode.h).
template <int MS, bool KFULL, bool F16 = false, bool PRE = false, bool MX = false, bool GROUPED = false,
          int ACT = kActNone>
__global__ void __launch_bounds__(kMfmaWN * 64) k_gemm_mfma(const uint16_t* __restrict__ x, int64_t ld_x, BlobView bv,
                                                        int NU, int KC, int K, int N, const float* __restrict__ gscale,
                                                        int g_is_div, uint16_t* __restrict__ y, int64_t ld_y, int M,
                                                        int t0, int vec_store, const uint16_t* __restrict__ pre,
                                                        const int32_t* __restrict__ offsets = nullptr, int E = 0,
                                                        const int32_t* __restrict__ row_index = nullptr) {
    constexpr int NT = kMfmaNT, WN = kMfmaWN;
    constexpr int kRows = 16 * MS;              // rows of this workgroup
    constexpr int kStage = kRows * 256;         // LDS bytes of one staged activation chunk
    constexpr int kParts = kMfmaTileRows / kRows;
    constexpr int kGroups = 4 * MS;             // issue groups per chunk
    constexpr int kAhead = 3;                   // fragment reads in flight
    static_assert(MS == 4 || MS == 8 || MS == 16, "row blocks per wave");
    __shared__ __attribute__((aligned(16))) uint8_t stage[2][kStage];
    constexpr int kWStage = kMfmaNT * (kCodeBlock + kScaleBlock);   // one chunk of a wave's weights
    __shared__ __attribute__((aligned(16))) uint8_t wstage[kMfmaWN][kWStage];
    // PRE: the 128 pre-quant scale values (256 bytes) of the chunk being staged, per wave
    __shared__ __attribute__((aligned(16))) uint8_t pstage[PRE ? kMfmaWN : 1][PRE ? 2 * kChunkK : 16];
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

    // The hardware deals workgroups to the eight XCDs round-robin (id % 8);
    // each XCD is given a contiguous range of the tile order instead, so the
    // ~32 workgroups an XCD runs together form a block of about 4 tile rows x
    // 8 tile columns whose activations and weights its own L2 holds.
    int e = 0, nt, m0, mend;   // expert, tile column, first row, end of the rows (M, or the expert's end)
    if constexpr (GROUPED) {
        static_assert(MS == 16, "the grouped form runs whole 256-row tiles");
        __shared__ int s_map[3];
        if (tid == 0) s_map[0] = -1;
        __syncthreads();
        if (w == 0) {
            // pass by < 0 counts the row tiles; pass by >= 0 finds row tile by's (expert, tile)
            auto scan = [&](int by) {
                int carry = 0;
                for (int base = 0; base < E; base += 64) {
                    const int ex = base + lane;
                    const int tiles = ex < E ? (offsets[ex + 1] - offsets[ex] + kRows - 1) / kRows : 0;
                    int v = tiles;
#pragma unroll
                    for (int d = 1; d < 64; d <<= 1) {
                        const int t = __shfl_up(v, d);
                        if (lane >= d) v += t;
                    }
                    const int incl = carry + v, excl = incl - tiles;
                    if (by >= 0 && tiles > 0 && by >= excl && by < incl) {
                        s_map[0] = ex;
                        s_map[1] = by - excl;
                    }
                    carry += __shfl(v, 63);
                }
                return carry;
            };
            const int64_t cols = (NU + kMfmaUnits - 1) / kMfmaUnits;
            const int64_t items = (int64_t)scan(-1) * cols, id = blockIdx.x;
            const int64_t per = (items + 7) / 8, item = (id % 8) * per + id / 8;
            if (id / 8 < per && item < items) {
                scan((int)(item / cols));
                if (lane == 0) s_map[2] = (int)(item % cols);
            }
        }
        __syncthreads();
        e = s_map[0];
        if (e < 0) return;                      // past the last item (uniform per workgroup)
        m0 = offsets[e] + s_map[1] * kRows;
        mend = offsets[e + 1];
        nt = s_map[2];
    } else {
        const int xid = [&] {
            const int n = (int)gridDim.x, q8 = n / 8, rem = n % 8, xx = (int)blockIdx.x % 8, k = (int)blockIdx.x / 8;
            return xx * q8 + (xx < rem ? xx : rem) + k;
        }();
        int mt;
        mfma_tile(t0 + xid / kParts, (M + kMfmaTileRows - 1) / kMfmaTileRows, (NU + kMfmaUnits - 1) / kMfmaUnits, mt,
                  nt);
        m0 = mt * kMfmaTileRows + (xid % kParts) * kRows;
        mend = M;
        if (m0 >= M) return;                    // a lower part past the last row (uniform per workgroup)
    }
    // row blocks of 16 holding rows of this tile (the others skip their MFMAs)
    const int msv = GROUPED ? (mend - m0 + 15) / 16 : MS;
    const int u_w = nt * kMfmaUnits + NT * w;   // this wave's first unit

    // ---- activation copies: copy i (0 .. 4 MS - 1) of a chunk moves rows
    // 4 i .. 4 i + 3; wave w issues copies w, w + 4, ..; lane l takes row
    // 4 i + (l >> 4) and the piece stored in slot l & 15.  Rows past mend read
    // row mend - 1 (never stored).  Offsets are 32-bit from the workgroup's
    // first row (at most 255 rows of ld_x <= 2^23 elements: below 2^32 bytes),
    // or from x when gathering (row_index[r] * ld_x * 2 < 2^32: the host bounds
    // the token count times ld_x).
    constexpr int kCopiesPerWave = kRows / 4 / WN;
    const int q = lane & 15;
    const bool gather = GROUPED && row_index != nullptr;
    uint32_t a_src[kCopiesPerWave];   // byte offset of the lane's piece in chunk 0, per copy
#pragma unroll
    for (int k = 0; k < kCopiesPerWave; ++k) {
        const int row = 4 * (w + WN * k) + (lane >> 4);
        const int rrow = m0 + row < mend ? row : mend - 1 - m0;
        const int64_t xrow = gather ? (int64_t)row_index[m0 + rrow] : (int64_t)rrow;
        a_src[k] = (uint32_t)((xrow * ld_x + (q ^ (row & 15)) * 8) * 2);
    }
    const uint8_t* xb = uniform_ptr(reinterpret_cast<const uint8_t*>(gather ? x : x + (int64_t)m0 * ld_x));
    auto copy_piece = [&](int c, int buf, int k) {   // copy w + 4 k of chunk c into stage buf
        const int i = w + WN * k, row = 4 * i + (lane >> 4);
        uint32_t off = a_src[k] + (uint32_t)(c * kChunkK * 2);
        if (!KFULL && c * kChunkK + (q ^ (row & 15)) * 8 >= K) off = a_src[k] - (q ^ (row & 15)) * 16;   // k = 0 of the row
        lds_copy16(lds_addr(stage[buf]) + i * 1024, xb, off);
    };
    auto copy_a = [&](int c, int buf) {
#pragma unroll
        for (int k = 0; k < kCopiesPerWave; ++k) copy_piece(c, buf, k);
    };
    // PRE: the pre-scale values of chunk c (clamped to the last chunk) into this
    // wave's slice, lane l taking elements 2 l, 2 l + 1; elements at k >= K read
    // k = 0 (their activation pieces are zeroed after the scaling).
    const uint8_t* pb = PRE ? uniform_ptr(reinterpret_cast<const uint8_t*>(pre)) : nullptr;
    auto copy_p = [&](int c) {
        const int k = (c < KC ? c : KC - 1) * kChunkK + 2 * lane;
        lds_copy4(lds_addr(pstage[w]), pb, (uint32_t)((KFULL || k < K ? k : 0) * 2));
    };
    // PRE: X' = RNE(X * s) in place on the pieces this lane copied into stage
    // buf (its copies, and the pre-scale copy issued before them, must have
    // landed).  All of a lane's pieces lie in one k slot: copy i = w + 4 k
    // holds row 4 i + (lane >> 4), whose row & 15 is 4 w + (lane >> 4).
    const int kslot = q ^ ((4 * w + (lane >> 4)) & 15);
    auto rescale_a = [&](int buf) {
        const uint4 sp = *reinterpret_cast<const uint4*>(pstage[w] + kslot * 16);
#pragma unroll
        for (int k = 0; k < kCopiesPerWave; ++k) {
            uint4* pc = reinterpret_cast<uint4*>(stage[buf] + (w + WN * k) * 1024 + lane * 16);
            *pc = prescale8<F16>(*pc, sp);
        }
    };
    // Zero the staged pieces of the last chunk that lie at k >= K (their
    // copies read k = 0 of the row).  Thread t zeroes slot t & 15 of row
    // t >> 4, which this thread's own wave copied (rows 4 i .. 4 i + 3 come
    // from copy i, issued by wave i % 4), so its own wait covers the copy.
    auto zero_tail = [&](int buf) {
        const int c = KC - 1;
        for (int t = tid; t < kRows * 16; t += WN * 64) {
            const int row = t >> 4, slot = t & 15;
            if (c * kChunkK + (slot ^ (row & 15)) * 8 >= K)
                *reinterpret_cast<uint4*>(stage[buf] + row * 256 + slot * 16) = make_uint4(0u, 0u, 0u, 0u);
        }
    };

    // ---- weights of this wave's units (units past NU read unit 0, never
    // stored).  A chunk of them (4 code blocks, 4 scale blocks) is copied
    // global -> LDS into the wave's own slice of LDS (no other wave reads it,
    // so only this wave's own wait is needed), then read into registers in
    // one go when the chunk's first decode is due, which frees the slice for
    // the next copy.  (Copying into LDS measured cheaper than loading into
    // registers beside the MFMAs.)
    const uint8_t* cb[NT];   // chunk-0 code block of unit j
    const uint8_t* s_lo[NT / 2];
    uint32_t s_off[NT / 2];  // scale copy p moves unit 2p (lanes 0..31) and 2p + 1 (lanes 32..63)
#pragma unroll
    for (int j = 0; j < NT; ++j) cb[j] = bv.codes + bv.block(e, (u_w + j) < NU ? u_w + j : 0, 0) * kCodeBlock;
#pragma unroll
    for (int p = 0; p < NT / 2; ++p) {
        const uint8_t* s0p = bv.scales + bv.block(e, (u_w + 2 * p) < NU ? u_w + 2 * p : 0, 0) * kScaleBlock;
        const uint8_t* s1p = bv.scales + bv.block(e, (u_w + 2 * p + 1) < NU ? u_w + 2 * p + 1 : 0, 0) * kScaleBlock;
        s_lo[p] = s0p < s1p ? s0p : s1p;
        s_off[p] = (uint32_t)((lane < 32 ? s0p : s1p) - s_lo[p]) + (uint32_t)((lane & 31) * 4);
    }
    const int64_t cstr = bv.chunk_stride * kCodeBlock;
    const uint32_t lane16 = (uint32_t)(lane * 16);
    const uint32_t wdst = lds_addr(wstage[w]);
    // copies of chunk c (clamped to the last chunk: past it they repeat it into a slice nothing reads)
    auto copy_b_codes = [&](int c) {
        const int64_t co = (int64_t)(c < KC ? c : KC - 1) * cstr;
#pragma unroll
        for (int j = 0; j < NT; ++j) lds_copy16(wdst + j * kCodeBlock, uniform_ptr(cb[j] + co), lane16);
    };
    auto copy_b_scales = [&](int c) {
        const int64_t so = ((int64_t)(c < KC ? c : KC - 1) * cstr) >> 3;
#pragma unroll
        for (int p = 0; p < NT / 2; ++p)
            lds_copy4(wdst + NT * kCodeBlock + p * 2 * kScaleBlock, uniform_ptr(s_lo[p] + so), s_off[p]);
    };
    struct BRegs {
        uint4 cw[NT];       // the lane's 16 code bytes (row l & 15, k-group l >> 4) per unit
        uint32_t sw[NT];    // the scale dword holding the lane's two scale bytes, per unit
    };
    auto read_b = [&](BRegs& b) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            b.cw[j] = *reinterpret_cast<const uint4*>(wstage[w] + j * kCodeBlock + lane16);
            b.sw[j] = *reinterpret_cast<const uint32_t*>(wstage[w] + NT * kCodeBlock + (j >> 1) * 2 * kScaleBlock +
                                                         (j & 1) * kScaleBlock + ((lane >> 1) << 2));
        }
    };

    float s0[NT], s1[NT];     // full scales of the lane's two 16-k blocks, per unit
    // fp16 with E4M3 scales: s0 / s1 hold the conversion operands and these the significand factors (half_scale)
    f16x2v sf0[NT], sf1[NT];
    constexpr bool kSplitF16 = F16 && !MX;

    f32x4 acc[MS][NT];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[ms][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    mfma_drain();             // the zeroed accumulators are read by the first MFMAs

    // ---- B fragments.  Unit u's fragment of step t is four dwords (two bf16
    // each); dword d is decoded in four VALU operations (convert, two scale
    // multiplies, pack), so that one operation can sit beside each MFMA.
    uint4 bfa[NT], bfb[NT];   // even steps in bfa, odd steps in bfb
    struct DwordJob {
        f32x2 p;
        float x, y;
        uint32_t h;   // kSplitF16: the converted fp16 pair before its factor
    };
    auto set_dword = [](uint4& v, int d, uint32_t val) {
        if (d == 0) v.x = val;
        else if (d == 1) v.y = val;
        else if (d == 2) v.z = val;
        else v.w = val;
    };
    // operation op (0..3) of decoding dword d (unit d >> 2, dword d & 3) of step t from b into nb
    auto dword_op = [&](const BRegs& b, int t, int d, int op, DwordJob& jb, uint4* nb) {
        const int u = d >> 2, e = d & 3;
        const uint32_t cw = t == 0 ? b.cw[u].x : t == 1 ? b.cw[u].y : t == 2 ? b.cw[u].z : b.cw[u].w;
        const float sc = t < 2 ? s0[u] : s1[u];
        if constexpr (MX) {
            // E8M0: the scale is applied in the conversion, one operation per dword
            if (op == 0) {
                const uint32_t v =
                    F16 ? (e == 0 ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, sc, 0))
                         : e == 1 ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, sc, 1))
                         : e == 2 ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, sc, 2))
                                  : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, sc, 3)))
                        : (e == 0 ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 0))
                         : e == 1 ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 1))
                         : e == 2 ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 2))
                                  : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 3)));
                set_dword(nb[u], e, v);
            }
            return;
        }
        if constexpr (kSplitF16) {
            // the scale's power of two in the conversion, its significand as a packed fp16 multiply
            if (op == 0) {
                jb.h = e == 0 ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, sc, 0))
                     : e == 1 ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, sc, 1))
                     : e == 2 ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, sc, 2))
                              : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, sc, 3));
            } else if (op == 1) {
                const f16x2v f = t < 2 ? sf0[u] : sf1[u];
                set_dword(nb[u], e, __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2v, jb.h) * f));
            }
            return;
        }
        if (op == 0) {
            jb.p = e == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 0)
                 : e == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 1)
                 : e == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 2)
                          : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 3);
        } else if (op == 1) {
            jb.x = jb.p.x * sc;
        } else if (op == 2) {
            jb.y = jb.p.y * sc;
        } else {
            set_dword(nb[u], e, pack_exact<F16>(jb.x, jb.y));
        }
    };
    auto scale_op = [&](const BRegs& b, int u) {   // scales of unit u of chunk b
        const f32x2 v = scale_pair_f32<MX>(scale_pair(b.sw[u], lane));   // E4M3 (E8M0) x 2
        if constexpr (kSplitF16) {
            const HalfScale h0 = half_scale(v.x), h1 = half_scale(v.y);
            s0[u] = h0.cvt;
            s1[u] = h1.cvt;
            sf0[u] = h0.f;
            sf1[u] = h1.f;
        } else {
            s0[u] = v.x;
            s1[u] = v.y;
        }
    };

    // ---- activation fragments: group f = MS t + ms reads fragment f + 3
    // into slot (f + 3) % 8 of a ring that spans chunk boundaries (the first
    // three fragments of chunk c + 1 are read while chunk c's last three
    // groups run).
    constexpr int kRing = 8;
    static_assert(kGroups % kRing == 0, "ring slots line up across chunks");
    uint4 af[kRing];
    auto frag = [&](int buf, int f) {
        const int t = f / MS, ms = f % MS;
        return *reinterpret_cast<const uint4*>(stage[buf] + (16 * ms + r) * 256 + (((4 * g + t) ^ r) << 4));
    };

    // One issue group: the read of fragment f + 3 (if it is in this chunk),
    // then four MFMAs, each followed by its share of the VALU work and a
    // scheduling fence.  VALU work: in steps 0..2 the decode of step t + 1
    // (16 / MS dwords per group); in step 3 the next chunk's scales (group 0)
    // and its step-0 decode (groups 1 .. MS - 1).
    // The copy schedule of a chunk (see the synchronisation note above).
    constexpr int kWCopies = NT + NT / 2;                 // weight copies per chunk
    constexpr int kReadB = 3 * MS;                        // group reading chunk c + 1's weights into registers
    constexpr bool kWBeforeBarrier = kReadB + 2 < kGroups - kAhead;   // chunk c + 2's weight copies precede the barrier
    constexpr int kBarrierWait = kWBeforeBarrier ? kWCopies : 0;      // copies allowed in flight at the barrier
    static_assert(2 * (kCopiesPerWave - 1) < kReadB, "a chunk's activation copies go out before its weights are read");

    auto group = [&](auto fc, int c, int buf, BRegs& b) {
        constexpr int f = decltype(fc)::value, t = f / MS, ms = f % MS;
        if constexpr (f + kAhead < kGroups) af[(f + kAhead) % kRing] = frag(buf, f + kAhead);
        // The activation copies of chunk c + 1 (into the other stage, free
        // since the last barrier) go out on every second group of the first
        // half, unconditionally (past the last chunk they repeat it into a
        // stage nothing reads; a branch per group cost more than the traffic),
        // after the copy of that chunk's pre-scale values (PRE).
        if constexpr (PRE && f == 0) copy_p(c + 1);
        if constexpr (f % 2 == 0 && f / 2 < kCopiesPerWave) copy_piece(c + 1 < KC ? c + 1 : KC - 1, buf ^ 1, f / 2);
        // Step 3: the weights of chunk c + 1 (copied a chunk ago; only the
        // copies issued since, this chunk's activation copies, may still fly)
        // replace chunk c's in registers, then the slice takes the copies of
        // chunk c + 2.
        if constexpr (f == kReadB) {
            wait_vmcnt<kCopiesPerWave>();
            read_b(b);
        }
        if constexpr (f == kReadB + 1) {
            wait_lgkmcnt0();
            copy_b_codes(c + 2);
        }
        if constexpr (f == kReadB + 2) copy_b_scales(c + 2);
        uint4* bf = (t & 1) ? bfb : bfa;
        uint4* nb = (t & 1) ? bfa : bfb;
        constexpr int d_lo = t < 3 ? ms * 16 / MS : (ms == 0 ? 0 : ((ms - 1) * 16 + MS - 2) / (MS - 1));
        constexpr int d_hi = t < 3 ? (ms + 1) * 16 / MS : (ms == 0 ? 0 : (ms * 16 + MS - 2) / (MS - 1));
        // dwords decoded in this group: 16 / MS in steps 0..2, up to ceil(16 / (MS - 1)) in step 3 (6 with
        // 64-row tiles)
        constexpr int kJobs = d_hi - d_lo > 0 ? d_hi - d_lo : 1;
        DwordJob jobs[kJobs];
        static_for<0, NT>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            if (!GROUPED || ms < msv) mfma_acc<F16>(acc[ms][j], bf[j], af[f % kRing]);
            if constexpr (t < 3) {
                static_for<d_lo, d_hi>([&](auto dc) {
                    constexpr int d = decltype(dc)::value;
                    dword_op(b, t + 1, d, j, jobs[d - d_lo], nb);
                });
            } else if constexpr (ms == 0) {
                scale_op(b, j);
            } else {
                static_for<d_lo, d_hi>([&](auto dc) {
                    constexpr int d = decltype(dc)::value;
                    dword_op(b, 0, d, j, jobs[d - d_lo], nb);
                });
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // One chunk on stage buf; b holds its weights until step 3, then the
    // next chunk's.  After group kGroups - 4 the wave waits for its
    // activation copies of chunk c + 1 (the weight copies of chunk c + 2 may
    // still fly if they were issued before this point), scales its own
    // pieces of them (PRE), zeroes their part past K, and meets the others at
    // the barrier; then it reads the first fragments of chunk c + 1 and runs
    // the last three groups, whose fragments are already in registers.
    auto chunk = [&](int c, int buf, BRegs& b) {
        static_for<0, kGroups - kAhead>([&](auto fc) { group(fc, c, buf, b); });
        wait_vmcnt<kBarrierWait>();
        if constexpr (PRE) {
            if (c + 1 < KC) rescale_a(buf ^ 1);
        }
        if (!KFULL && c + 1 == KC - 1) zero_tail(buf ^ 1);
        wait_lgkmcnt0();
        asm volatile("s_barrier" ::: "memory");
        if (c + 1 < KC) {
            static_for<0, kAhead>([&](auto fc) {
                constexpr int f = decltype(fc)::value;
                af[f] = frag(buf ^ 1, f);
            });
        }
        __builtin_amdgcn_sched_barrier(0);
        static_for<kGroups - kAhead, kGroups>([&](auto fc) { group(fc, c, buf, b); });
    };

    // ---- pipeline: chunk c on stage c & 1
    BRegs b;
    if constexpr (PRE) copy_p(0);
    copy_a(0, 0);
    copy_b_codes(0);
    copy_b_scales(0);
    __builtin_amdgcn_s_waitcnt(0);
    if constexpr (PRE) rescale_a(0);
    if (!KFULL && KC == 1) zero_tail(0);
    __syncthreads();
    read_b(b);
    wait_lgkmcnt0();
    copy_b_codes(1);
    copy_b_scales(1);
    static_for<0, NT>([&](auto jc) { scale_op(b, decltype(jc)::value); });
    static_for<0, 16>([&](auto dc) {
        DwordJob jb;
        static_for<0, 4>([&](auto oc) { dword_op(b, 0, decltype(dc)::value, decltype(oc)::value, jb, bfa); });
    });
    static_for<0, kAhead>([&](auto fc) { af[decltype(fc)::value] = frag(0, decltype(fc)::value); });
    for (int c = 0; c < KC; ++c) chunk(c, c & 1, b);
    wait_vmcnt<0>();   // the last chunk's clamped copies: none may land after the workgroup ends
    mfma_drain();

    // ---- epilogue: lane (r, g) holds, for row 16 ms + r, the four columns
    // 16 (u_w + j) + 4 g + i.  They are scaled, rounded to bf16 pairs, and
    // transposed across the four lane rows g and the four units j with two
    // lane-swap rounds, after which lane row g holds the 16 adjacent columns
    // 16 (u_w + g) .. + 15 of its row: two 16-byte stores per row block.
    const float gv = global_scale_at(gscale, e, g_is_div);
    if constexpr (ACT == kActSiluGlu) {
        // units u_w + 2 p (gate) and u_w + 2 p + 1 (up): lane (r, g) holds both
        // for columns 4 g + i of the pair, output column 16 (u_w / 2 + p) + 4 g + i
        // of N / 2 (u_w is a multiple of 4)
        static_for<0, MS>([&](auto msc) {
            constexpr int ms = decltype(msc)::value;
            const int m = m0 + 16 * ms + r;
            if (m < mend) {
                uint16_t* yr = y + (int64_t)m * ld_y;
#pragma unroll
                for (int p = 0; p < NT / 2; ++p)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float hg = act_to_f32<F16>(round_out<F16>(scale_acc(gv, acc[ms][2 * p][i])));
                        const float hu = act_to_f32<F16>(round_out<F16>(scale_acc(gv, acc[ms][2 * p + 1][i])));
                        const int n = (u_w / 2 + p) * kUnitN + 4 * g + i;
                        if (n < N / 2) yr[n] = (uint16_t)round_out<F16>(silu_times(hg, hu));
                    }
            }
        });
        return;
    }
    // the value stored for an accumulator (with kActRelu2, the squared ReLU of
    // the rounded output, rounded again)
    auto outv = [&](float a) {
        if constexpr (ACT == kActRelu2) return relu_squared(act_to_f32<F16>(round_out<F16>(scale_acc(gv, a))));
        else return scale_acc(gv, a);
    };
    static_for<0, MS>([&](auto msc) {
        constexpr int ms = decltype(msc)::value;
        uint32_t pk[NT][2];   // bf16 pairs of columns 4 g + 2 d, + 1 of unit j (then of unit g: 4 j + 2 d)
        static_for<0, NT>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            pk[j][0] = pack_round2<F16>(outv(acc[ms][j][0]), outv(acc[ms][j][1]));
            pk[j][1] = pack_round2<F16>(outv(acc[ms][j][2]), outv(acc[ms][j][3]));
        });
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            lane_swap32(pk[0][d], pk[2][d]);
            lane_swap32(pk[1][d], pk[3][d]);
            lane_swap16(pk[0][d], pk[1][d]);
            lane_swap16(pk[2][d], pk[3][d]);
        }
        const int m = m0 + 16 * ms + r;
        if (m < mend) {
            uint16_t* yr = y + (int64_t)m * ld_y;
            const int n0 = (u_w + g) * kUnitN;
            if (vec_store && n0 + 15 < N) {
                *reinterpret_cast<uint4*>(yr + n0) = make_uint4(pk[0][0], pk[0][1], pk[1][0], pk[1][1]);
                *reinterpret_cast<uint4*>(yr + n0 + 8) = make_uint4(pk[2][0], pk[2][1], pk[3][0], pk[3][1]);
            } else {
#pragma unroll
                for (int k = 0; k < NT; ++k)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n0 + 4 * k + e < N) yr[n0 + 4 * k + e] = (uint16_t)(pk[k][e >> 1] >> (16 * (e & 1)));
            }
        }
    });
}

}  // namespace nvfp4
