// Tile GEMM for rows > 4: a BM x (16 NT UW) output tile per workgroup.
//
//   BM = 16 MS rows.  The workgroup's UW x KW waves are UW unit-waves times
//   KW k-parts: wave (uw, q) owns NT consecutive 16-row units of W and the
//   q-th contiguous part of the workgroup's K range.  At every step the
//   workgroup stages one activation chunk (BM rows x 128 k) per k-part in a
//   double-buffered LDS ring, shared by the UW unit-waves of that part; the
//   global loads of a step's activation pieces ride in the same D-deep
//   register ring as the weight blocks, so no step waits on a load issued
//   in its own iteration.  Each wave decodes its codes straight into exact
//   bf16 v_mfma_f32_16x16x32_bf16 fragments and accumulates MS x NT 16x16
//   sub-tiles in fp32.  The 32 K slots of an MFMA step map to
//   k = 32 g + 8 t + e (lane group g, step t, element e) on both operands, so
//   each weight lane reads a whole 32-wide K group of the repacked layout.
//   The KW partial tiles are summed through LDS in part order 0..KW-1.
//
//   K may also be split S ways across workgroups (grid z).  Each split
//   writes its fp32 partial tile to the workspace, then bumps the tile's
//   counter; the workgroup that arrives last adds the S partials in split
//   order (0..S-1, independent of arrival order, so the result is bitwise
//   reproducible), applies the epilogue and resets the counter to zero for
//   the next call.
//
//   With PRE the pre-quant scale multiplies each activation piece as it is
//   written into the LDS stage (prescale8: RNE(X * s), once per workgroup and
//   piece, never written back to memory).
//
//   Grouped (MoE) form: grid y has R/BM + E row-tile slots, mapped to
//   (expert, tile) by a wave-wide prefix scan of the per-expert tile counts
//   read from expert_offsets; surplus slots exit before touching weights.
//   The work items (row tile in expert order, column group) are dealt to the
//   eight XCDs in contiguous ranges: the hardware hands workgroup ids to the
//   XCDs round robin, so id i takes item (i % 8) * per + i / 8 of the real
//   items (per = ceil(items / 8); ids with i / 8 >= per exit, so no item runs
//   twice, and the host's grid holds at least 8 workgroups more than there
//   can be items, so that every item has an id).  The column groups of a row
//   tile then run together on one XCD and share its activation rows in that
//   XCD's L2, and an expert's row tiles follow each other there and share its
//   weights.
//   ACT: the MoE activation the epilogue applies (decode.h); with
//   kActSiluGlu a wave's NT (even) units are gate / up pairs.
#pragma once
#include "decode.h"
#include "kernels_gemm.h"
#include "layout.h"

namespace nvfp4 {

constexpr int kTileLDA = 136;   // bf16 per LDS row of the activation stage (128 + 8 pad)
constexpr int kXcds = 8;        // XCDs of the MI355X: workgroup ids are dealt to them round robin
constexpr int kTileScanFastE = 256;   // grouped tile mapping: expert counts up to this scan in registers


template <int MS, int NT, int UW, int KW, int D, bool GROUPED, bool KFULL, bool F16 = false, bool PRE = false,
          int ACT = kActNone, bool MX = false>
__global__ void __launch_bounds__(UW * KW * 64, GROUPED ? 2 : 1) k_gemm_tile(const uint16_t* __restrict__ x, int64_t ld_x, BlobView bv,
                                                            int NU, int KC, int K, int N,
                                                            const float* __restrict__ gscale, int g_is_div,
                                                            uint16_t* __restrict__ y, int64_t ld_y, int64_t rows_dense,
                                                            const int32_t* __restrict__ offsets, int E, SplitK sk,
                                                            const int32_t* __restrict__ row_index,
                                                            const uint16_t* __restrict__ pre) {
    constexpr int W = UW * KW;                                     // waves per workgroup
    // Weights stream past the caches (non-temporal) when one row tile covers
    // all rows (tiles of up to 32 rows, dense): no other workgroup reads the
    // same chunk.  With several row tiles a chunk is read once per row tile
    // and caching it is faster (measured).
    constexpr bool kStreamWeights = MS <= 2 && !GROUPED;
    constexpr int BM = 16 * MS;
    constexpr int UG = NT * UW;                                    // units per workgroup
    constexpr int CPIECES = BM * 16;                               // 16-byte pieces per activation chunk
    constexpr int APIECES = KW * CPIECES;                          // pieces per step
    constexpr int APT = (APIECES + W * 64 - 1) / (W * 64);         // pieces per thread
    constexpr int kStage = KW * BM * kTileLDA;                     // bf16 per stage buffer
    constexpr int kRedTile = MS * NT * 256;                        // floats of one wave's partial tile
    static_assert(D >= 2, "the ring stages step i + 1 from another slot while refilling step i's");
    static_assert((KW - 1) * UW * kRedTile * 4 <= 2 * kStage * 2, "k-part reduction fits in the stage buffers");
    __shared__ __attribute__((aligned(16))) uint16_t As[2 * kStage];
    __shared__ int s_map[5];   // expert, its row tile, column group, the expert's first and end row

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int uw = w % UW, q = w / UW;

    // ---- which rows: dense m-tile, or (expert, m-tile) of the grouped form
    int e = 0;
    int bx = (int)blockIdx.x;   // column group
    int64_t row0, rows;
    if (GROUPED) {
        if (tid == 0) s_map[0] = -1;
        __syncthreads();
        if (w == 0) {
            const int64_t groups = gridDim.x;
            const int64_t id = (int64_t)blockIdx.y * groups + blockIdx.x;
            // item of this workgroup once the total is known: items are dealt
            // to the XCDs in contiguous ranges (id % kXcds picks the range)
            auto item_of = [&](int total, int64_t& item) {
                const int64_t items = (int64_t)total * groups, per = (items + kXcds - 1) / kXcds;
                item = (id % kXcds) * per + id / kXcds;
                return id / kXcds < per && item < items;
            };
            if (E <= kTileScanFastE) {
                // up to kTileScanFastE experts: every offset is loaded at once
                // (one memory round trip) and both passes scan registers
                constexpr int NB = kTileScanFastE / 64;
                int lo[NB], hi[NB], tl[NB], incl[NB];
#pragma unroll
                for (int i = 0; i < NB; ++i) {
                    const int ex = 64 * i + lane;
                    lo[i] = ex < E ? offsets[ex] : 0;
                    hi[i] = ex < E ? offsets[ex + 1] : 0;
                }
                int carry = 0;
#pragma unroll
                for (int i = 0; i < NB; ++i) {
                    tl[i] = (hi[i] - lo[i] + BM - 1) / BM;
                    int v = tl[i];
#pragma unroll
                    for (int d = 1; d < 64; d <<= 1) {
                        const int t = __shfl_up(v, d);
                        if (lane >= d) v += t;
                    }
                    incl[i] = carry + v;
                    carry += __shfl(v, 63);
                }
                int64_t item;
                if (item_of(carry, item)) {
                    const int by = (int)(item / groups);
#pragma unroll
                    for (int i = 0; i < NB; ++i) {
                        const int excl = incl[i] - tl[i];
                        if (tl[i] > 0 && by >= excl && by < incl[i]) {
                            s_map[0] = 64 * i + lane;
                            s_map[1] = by - excl;
                            s_map[3] = lo[i];
                            s_map[4] = hi[i];
                        }
                    }
                    if (lane == 0) s_map[2] = (int)(item % groups);
                }
            } else {
                // prefix scan of the per-expert tile counts: pass 0 counts the
                // row tiles, pass 1 finds this workgroup's (expert, tile)
                auto scan = [&](int by) {
                    int carry = 0;
                    for (int base = 0; base < E; base += 64) {
                        const int ex = base + lane;
                        const int lo = ex < E ? offsets[ex] : 0, hi = ex < E ? offsets[ex + 1] : 0;
                        const int tiles = (hi - lo + BM - 1) / BM;
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
                            s_map[3] = lo;
                            s_map[4] = hi;
                        }
                        carry += __shfl(v, 63);
                    }
                    return carry;
                };
                int64_t item;
                if (item_of(scan(-1), item)) {
                    scan((int)(item / groups));
                    if (lane == 0) s_map[2] = (int)(item % groups);
                }
            }
        }
        __syncthreads();
        // the mapping is the same for the whole workgroup: reading it into
        // scalar registers lets every weight address stay scalar
        e = __builtin_amdgcn_readfirstlane(s_map[0]);
        if (e < 0) return;   // uniform: past the last item
        bx = __builtin_amdgcn_readfirstlane(s_map[2]);
        row0 = (int64_t)__builtin_amdgcn_readfirstlane(s_map[3]) + (int64_t)__builtin_amdgcn_readfirstlane(s_map[1]) * BM;
        rows = (int64_t)__builtin_amdgcn_readfirstlane(s_map[4]) - row0;
    } else {
        row0 = (int64_t)blockIdx.y * BM;
        rows = rows_dense - row0;
    }
    if (rows > BM) rows = BM;

    // ---- K ranges: split s of the workgroup (grid z), part q of the wave
    const int S = sk.S, s = (int)blockIdx.z;
    const int C0 = (int)((int64_t)KC * s / S), span = (int)((int64_t)KC * (s + 1) / S) - C0;
    auto part_begin = [&](int qq) { return C0 + span * qq / KW; };
    const int c0 = part_begin(q), len = part_begin(q + 1) - c0;   // this wave's chunks [c0, c0 + len)
    const int steps = (span + KW - 1) / KW;                          // the longest part
    const int u_w = bx * UG + uw * NT;                             // this wave's first unit
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

    // ---- this thread's activation pieces (fixed across steps): piece
    // p = tid + i * threads is row (p % CPIECES) >> 4, k piece p & 15 of the
    // chunk of part p / CPIECES.  Rows past `rows` read row 0 (outputs never
    // stored); pieces past K are zeroed when staged.  Offsets within the
    // row tile fit 32 bits (the host bounds ld_x).
    // grouped row r reads activation row row_index[r] when gathering
    const bool gather = GROUPED && row_index != nullptr;
    const uint16_t* xtile = gather ? x : x + row0 * ld_x;
    uint32_t a_xo[APT], a_off[APT];
    int a_c0[APT], a_last[APT];
#pragma unroll
    for (int i = 0; i < APT; ++i) {
        const int p = tid + i * W * 64;
        const int qa = KW == 1 ? 0 : (p < APIECES ? p : 0) / CPIECES, within = p % CPIECES;
        const int pr = within >> 4;
        a_c0[i] = part_begin(qa);
        const int la = part_begin(qa + 1) - a_c0[i];
        a_last[i] = la > 0 ? la - 1 : 0;
        const int prr = pr < rows ? pr : 0;
        a_xo[i] = (uint32_t)((gather ? (int64_t)row_index[row0 + prr] : (int64_t)prr) * ld_x);
        a_off[i] = (uint32_t)(qa * BM * kTileLDA + pr * kTileLDA + (within & 15) * 8);
    }

    // ---- per-wave ring of D steps: NT code blocks + scale pairs of this
    // wave's chunk, and this thread's activation pieces of the step
    struct Slot {
        uint4 cw[NT];
        uint32_t sw[NT];
        uint4 a[APT];
        uint4 pa[APT];   // pre-quant scale pieces of the activation pieces' k (PRE only)
    };
    const int w_last = len > 0 ? len - 1 : 0;
    auto load_slot = [&](Slot& b, int step) {
        const int c = c0 + (step < w_last ? step : w_last);
        const int64_t boff = (int64_t)c * cstr;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const uint8_t* cp = cb[j] + boff + (uint32_t)(lane * 16);
            const uint8_t* sp = sb[j] + (boff >> 3) + (uint32_t)(lane * 2);
            if constexpr (kStreamWeights) {
                b.cw[j] = load_stream_u4(cp);
                b.sw[j] = load_stream_u16(sp);
            } else {
                b.cw[j] = *reinterpret_cast<const uint4*>(cp);
                b.sw[j] = *reinterpret_cast<const uint16_t*>(sp);
            }
        }
#pragma unroll
        for (int i = 0; i < APT; ++i) {
            const int ca = a_c0[i] + (step < a_last[i] ? step : a_last[i]);
            const int k = ca * kChunkK + (int)((tid + i * W * 64) & 15) * 8;
            const uint32_t kk = (uint32_t)(KFULL || k < K ? k : 0);
            b.a[i] = *reinterpret_cast<const uint4*>(xtile + a_xo[i] + kk);
            if constexpr (PRE) b.pa[i] = *reinterpret_cast<const uint4*>(pre + kk);
        }
    };
    auto store_a = [&](int buf, const Slot& b, int step) {
#pragma unroll
        for (int i = 0; i < APT; ++i) {
            const int p = tid + i * W * 64;
            if (APIECES % (W * 64) != 0 && p >= APIECES) break;
            const int ca = a_c0[i] + (step < a_last[i] ? step : a_last[i]);
            const bool kin = KFULL || (ca * kChunkK + (p & 15) * 8 < K);
            const uint4 v = PRE ? prescale8<F16>(b.a[i], b.pa[i]) : b.a[i];
            *reinterpret_cast<uint4*>(&As[buf * kStage + a_off[i]]) =
                make_uint4(kin ? v.x : 0u, kin ? v.y : 0u, kin ? v.z : 0u, kin ? v.w : 0u);
        }
    };

    f32x4 acc[MS][NT];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[ms][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const Slot& b, int buf) {
        const uint16_t* abase = &As[buf * kStage + q * BM * kTileLDA + r * kTileLDA + g * 32];
        // the lane's two scales (lower and upper 16 k of its 32) as fp32, exact
        float sc[NT][2];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const f32x2 sp = scale_pair_f32<MX>(b.sw[j]);
            sc[j][0] = sp.x;
            sc[j][1] = sp.y;
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            uint4 bf[NT];
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const uint32_t d = t == 0 ? b.cw[j].x : t == 1 ? b.cw[j].y : t == 2 ? b.cw[j].z : b.cw[j].w;
                if constexpr (F16 && !MX) bf[j] = decode8_f16_split(d, half_scale(sc[j][t >> 1]));
                else bf[j] = decode8_fmt<F16, MX>(d, sc[j][t >> 1]);
            }
#pragma unroll
            for (int ms = 0; ms < MS; ++ms) {
                const uint4 af = *reinterpret_cast<const uint4*>(abase + ms * 16 * kTileLDA + t * 8);
#pragma unroll
                for (int j = 0; j < NT; ++j) acc[ms][j] = mma16<F16>(af, bf[j], acc[ms][j]);
            }
        }
    };

    if (steps > 0) {
        Slot ring[D];
#pragma unroll
        for (int d = 0; d < D; ++d) load_slot(ring[d], d);
        store_a(0, ring[0], 0);
        __syncthreads();   // first activation step ready
        // Step i (ring slot i % D, LDS buffer i & 1): stage step i + 1 into
        // the other buffer, refill the slot with step i + D, contract step i
        // (waves whose part is shorter skip its last step), then one barrier.
        int i = 0;
        for (; i + D <= steps; i += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int ii = i + d;
                if (ii + 1 < steps) store_a((ii + 1) & 1, ring[(d + 1) % D], ii + 1);
                const Slot cur = ring[d];
                load_slot(ring[d], ii + D);
                if (ii < len) compute(cur, ii & 1);
                __syncthreads();
            }
        }
#pragma unroll
        for (int d = 0; d < D - 1; ++d) {
            const int ii = i + d;
            if (ii < steps) {
                if (ii + 1 < steps) store_a((ii + 1) & 1, ring[d + 1], ii + 1);
                if (ii < len) compute(ring[d], ii & 1);
                __syncthreads();
            }
        }
    }

    // ---- sum the k-parts through LDS, in part order
    if (KW > 1) {
        __syncthreads();
        float* red = reinterpret_cast<float*>(As);
        if (q > 0) {
            float* mine = red + ((q - 1) * UW + uw) * kRedTile + lane * 4;
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    *reinterpret_cast<f32x4*>(mine + (ms * NT + j) * 256) = acc[ms][j];
        }
        __syncthreads();
        if (q == 0) {
#pragma unroll
            for (int qq = 1; qq < KW; ++qq) {
                const float* other = red + ((qq - 1) * UW + uw) * kRedTile + lane * 4;
#pragma unroll
                for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                    for (int j = 0; j < NT; ++j)
                        acc[ms][j] += *reinterpret_cast<const f32x4*>(other + (ms * NT + j) * 256);
            }
        }
    }

    const float gv = global_scale_at(gscale, e, g_is_div);
    // Lane (r, g) of a part-0 wave holds rows 16 ms + 4 g + i of column
    // 16 (u_w + j) + r.  Output blocks of 16 columns: with kActSiluGlu the
    // unit pair (u_w + 2 b, u_w + 2 b + 1) (gate, up) gives columns
    // 16 (u_w / 2 + b) + r of N / 2, otherwise unit u_w + b gives columns
    // 16 (u_w + b) + r of N.
    static_assert(ACT != kActSiluGlu || NT % 2 == 0, "gate / up units come in pairs");
    constexpr int OB = ACT == kActSiluGlu ? NT / 2 : NT;      // 16-column output blocks of a wave
    const int64_t NO = ACT == kActSiluGlu ? N / 2 : N;        // output columns
    const int64_t col0 = (int64_t)(ACT == kActSiluGlu ? u_w / 2 : u_w) * kUnitN;
    auto out_value = [&](int ms, int b, int i) -> uint32_t {
        if constexpr (ACT == kActSiluGlu) {
            const float hg = act_to_f32<F16>(round_out<F16>(scale_acc(gv, acc[ms][2 * b][i])));
            const float hu = act_to_f32<F16>(round_out<F16>(scale_acc(gv, acc[ms][2 * b + 1][i])));
            return round_out<F16>(silu_times(hg, hu));
        } else {
            uint32_t v = round_out<F16>(scale_acc(gv, acc[ms][b][i]));
            if constexpr (ACT == kActRelu2) v = round_out<F16>(relu_squared(act_to_f32<F16>(v)));
            return v;
        }
    };
    // One 16-bit store per output (any alignment).
    auto store_y_scalar = [&]() {
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int b = 0; b < OB; ++b) {
                const int64_t n = col0 + b * kUnitN + r;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = ms * 16 + g * 4 + i;
                    const uint32_t v = out_value(ms, b, i);
                    if (m < rows && n < NO) y[(row0 + m) * ld_y + n] = (uint16_t)v;
                }
            }
    };
    // Through LDS: a wave stages each 16-row block of its outputs in its own
    // slice of the (idle) stage buffers and writes it back as 16-byte row
    // pieces, 8 columns each.  Needs y 16-byte aligned and ld_y and the
    // output width multiples of 8; the slice is private to the wave, so only
    // the wave's own LDS accesses are ordered (lgkmcnt) between the phases.
    constexpr int OC = OB * kUnitN;                 // output columns of a wave
    constexpr int OLD = OC + 8;                     // 16-bit values per staged row (rows stay 16-byte aligned)
    constexpr int PPR = OC / 8;                     // 16-byte pieces per row
    constexpr int PPL = (16 * PPR + 63) / 64;       // pieces per lane and 16-row block
    static_assert(UW * KW * 16 * OLD <= 2 * kStage, "each wave's 16-row output slice fits in the stage buffers");
    auto store_y_vec = [&]() {
        uint16_t* o = &As[w * 16 * OLD];
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
#pragma unroll
            for (int b = 0; b < OB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[(g * 4 + i) * OLD + b * kUnitN + r] = (uint16_t)out_value(ms, b, i);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
            for (int t = 0; t < PPL; ++t) {
                const int p = lane + 64 * t;
                if ((16 * PPR) % 64 != 0 && p >= 16 * PPR) break;
                const int rr = p / PPR, cp = p % PPR;
                const uint4 v = *reinterpret_cast<const uint4*>(&o[rr * OLD + cp * 8]);
                const int m = ms * 16 + rr;
                const int64_t n = col0 + cp * 8;
                if (m < rows && n < NO) *reinterpret_cast<uint4*>(y + (row0 + m) * ld_y + n) = v;
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // read back before the next block's writes
        }
    };
    const bool vec_out = ((reinterpret_cast<uintptr_t>(y) | (uintptr_t)(ld_y * 2)) & 15u) == 0 && NO % 8 == 0;
    auto store_y = [&]() {
        if (vec_out) store_y_vec();
        else store_y_scalar();
    };
    if (S == 1) {
        if (KW > 1) __syncthreads();   // the k-part sums have been read from the stage buffers
        if (q == 0) store_y();
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
    constexpr int64_t kTilePairs = (int64_t)MS * NT * UW * 64 * 2;   // float pairs per partial tile
    uint64_t* parts = reinterpret_cast<uint64_t*>(sk.partials);
    auto pidx = [&](int ms, int j, int h) { return (((ms * NT + j) * UW + uw) * 64 + lane) * 2 + h; };
    if (q == 0) {
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
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);   // all of this wave's partial stores acknowledged
    __syncthreads();
    if (tid == 0) s_map[2] = atomicAdd(&sk.counters[tile], 1);
    __syncthreads();
    if (s_map[2] != S - 1 || q != 0) return;   // uniform per wave: not the last split, or not a part-0 wave
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
    store_y();
}

}  // namespace nvfp4
