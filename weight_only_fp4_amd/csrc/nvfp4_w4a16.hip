// C ABI of the W4A16 NVFP4 GEMM library (see include/nvfp4_w4a16.h).
//
// Host side: argument checks (all before any launch), size queries, kernel
// choice and launches.  Everything is stream-ordered and asynchronous; the
// host never waits on the device and never reads device memory.  The GEMM
// kernel families are launched from their own translation units (plan.h).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/nvfp4_w4a16.h"
#include "kernels_aux.h"
#include "kernels_moe.h"
#include "launch_mfma.h"
#include "plan.h"

namespace nvfp4 {

namespace {
thread_local char g_err[512] = "";
}  // namespace

nvfp4_status fail(nvfp4_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

nvfp4_status ok() {
    g_err[0] = '\0';
    return NVFP4_OK;
}

nvfp4_status launched(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(NVFP4_ERR_HIP, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace nvfp4

using namespace nvfp4;

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// mx: MXFP4 weights (one E8M0 scale per 32 K) instead of NVFP4 (one E4M3 per 16).
nvfp4_status check_weight_shape(const char* fn, int64_t E, int64_t N, int64_t K, int mx = 0) {
    if (E < 1 || E > kMaxExperts) return fail(NVFP4_ERR_INVALID_ARG, "%s: E = %lld must be in [1, %d]", fn, (long long)E, kMaxExperts);
    if (N < 0 || N > (int64_t)1 << 30) return fail(NVFP4_ERR_INVALID_ARG, "%s: N = %lld must be in [0, 2^30]", fn, (long long)N);
    if (mx && (K < 32 || K % 32 != 0 || K > (int64_t)1 << 30))
        return fail(NVFP4_ERR_INVALID_ARG, "%s: K = %lld must be a positive multiple of 32 (one E8M0 scale per 32 K)", fn, (long long)K);
    if (K < 16 || K % 16 != 0 || K > (int64_t)1 << 30)
        return fail(NVFP4_ERR_INVALID_ARG, "%s: K = %lld must be a positive multiple of 16 (one E4M3 scale per 16 K)", fn, (long long)K);
    return NVFP4_OK;
}

enum Variant { kAuto = 0, kSmall = 1, kLarge = 2, kMfma = 3, kResident = 4, kMfmaQuarter = 5 };

// Activation row stride limit: offsets within a 128-row tile stay in 32 bits.
constexpr int64_t kMaxLdX = int64_t(1) << 23;

// Rows at or below this use the small-M kernel when the variant is automatic.
constexpr int64_t kSmallAuto = 4;

// The automatic variant uses the MFMA-bound kernel from this many rows on,
// when the call has at least kMfmaMinTiles of its 256 x 256 tiles (with fewer
// the chip is not filled and the tile kernel, which can split K, is faster).
constexpr int64_t kMfmaAuto = 256;
constexpr int64_t kMfmaMinTiles = 48;

// Shared checks of the activation / output / pre-scale / workspace arguments.
// no_global: the format has no global scale (MXFP4; gs is NULL).
nvfp4_status check_gemm_io(const char* fn, const void* x, int64_t ld_x, const void* pre, const void* w,
                           const void* gs, const void* y, int64_t ld_y, int64_t rows, int64_t N, int64_t K,
                           const void* ws, int64_t ws_bytes, int64_t ws_need, bool no_global = false) {
    if (rows < 0) return fail(NVFP4_ERR_INVALID_ARG, "%s: row count %lld is negative", fn, (long long)rows);
    if (ld_x < K) return fail(NVFP4_ERR_INVALID_ARG, "%s: ld_x = %lld < K = %lld", fn, (long long)ld_x, (long long)K);
    if (ld_y < N) return fail(NVFP4_ERR_INVALID_ARG, "%s: ld_y = %lld < N = %lld", fn, (long long)ld_y, (long long)N);
    // with no output columns (N == 0) the weights and the output hold no bytes
    if (!w && N > 0) return fail(NVFP4_ERR_INVALID_ARG, "%s: w_repacked is NULL", fn);
    if (!gs && !no_global) return fail(NVFP4_ERR_INVALID_ARG, "%s: global scale pointer is NULL", fn);
    if (rows > 0 && !x) return fail(NVFP4_ERR_INVALID_ARG, "%s: x is NULL", fn);
    if (rows > 0 && N > 0 && !y) return fail(NVFP4_ERR_INVALID_ARG, "%s: y is NULL", fn);
    if (ld_x > kMaxLdX)
        return fail(NVFP4_ERR_INVALID_ARG, "%s: ld_x = %lld exceeds %lld", fn, (long long)ld_x, (long long)kMaxLdX);
    if (!aligned(x, 16) || ld_x % 8 != 0)
        return fail(NVFP4_ERR_ALIGNMENT, "%s: x must be 16-byte aligned with ld_x %% 8 == 0 (ld_x = %lld)", fn, (long long)ld_x);
    if (pre && !aligned(pre, 16)) return fail(NVFP4_ERR_ALIGNMENT, "%s: pre_scale must be 16-byte aligned", fn);
    if (!aligned(w, 16)) return fail(NVFP4_ERR_ALIGNMENT, "%s: w_repacked must be 16-byte aligned", fn);
    if (!aligned(y, 2)) return fail(NVFP4_ERR_ALIGNMENT, "%s: y must be 2-byte aligned", fn);
    if (rows > 0 && ws_need > 0) {
        if (ws_bytes < ws_need || !ws)
            return fail(NVFP4_ERR_BUFFER_TOO_SMALL, "%s: workspace of %lld bytes is below the %lld bytes this call needs", fn,
                        (long long)ws_bytes, (long long)ws_need);
        if (!aligned(ws, 256)) return fail(NVFP4_ERR_ALIGNMENT, "%s: workspace must be 256-byte aligned", fn);
    }
    return NVFP4_OK;
}

// Workspace bytes of a dense call: enough for any kernel variant that takes
// the shape (the small-M kernel up to 16 rows, the activation-resident kernel
// where xres_fits holds, the tile kernel always; the MFMA-bound kernel needs
// none).  A pre-quant scale needs none either: it is applied in the kernels'
// activation loads.
int64_t dense_workspace_bytes(const Layout& L, int64_t M) {
    if (M == 0 || L.N == 0) return 0;
    int64_t need = workspace_for(tile_shape(L, M, false)).total;
    if (M <= kSmallRows) {
        const int64_t small = workspace_for(small_m_shape(L, M, false)).total;
        need = small > need ? small : need;
    }
    if (xres_fits(L, M)) {
        const int64_t xres = workspace_for(xres_shape(L, M)).total;
        need = xres > need ? xres : need;
    }
    return need;
}

// The kernel variant the automatic choice runs for a dense call (kAuto when
// the call launches nothing).
int dense_auto_variant(const Layout& L, int64_t M) {
    if (M == 0 || L.N == 0) return kAuto;
    if (M >= kXresAutoMin && xres_fits(L, M)) return kResident;
    if (M <= kSmallAuto) return kSmall;
    const bool mfma_fits = L.code_bytes() < ((int64_t)1 << 31);
    if (mfma_fits && M >= kMfmaAuto && mfma_plan(L, M).tiles >= kMfmaMinTiles) return kMfma;
    return kLarge;
}

// Limits of the activation-resident kernel, in the words of the error text.
const char* const kXresLimits =
    "M <= 16, K <= 32768 and ceil(N / 16) * ceil(K / 4096) <= 2048 (at most eight 16-row units per workgroup "
    "for about one workgroup per compute unit)";

// The activation-resident launch for the blob's scale format and the
// activation type.
nvfp4_status launch_xres_any(const XresShape& s, const Layout& L, const GemmArgs& a, bool f16) {
    if (f16) return L.mx ? launch_xres<true, true>(s, L, a) : launch_xres<true, false>(s, L, a);
    return L.mx ? launch_xres<false, true>(s, L, a) : launch_xres<false, false>(s, L, a);
}

nvfp4_status dense_gemm(const void* x, int64_t ld_x, const void* pre, const void* w, const float* gs, int g_div,
                        void* y, int64_t ld_y, int64_t M, int64_t N, int64_t K, void* ws, int64_t ws_bytes,
                        int variant, void* stream, const char* fn, bool f16, int mx = 0) {
    nvfp4_status s = check_weight_shape(fn, 1, N, K, mx);
    if (s != NVFP4_OK) return s;
    if (variant < kAuto || variant > kMfmaQuarter) return fail(NVFP4_ERR_INVALID_ARG, "%s: unknown variant %d", fn, variant);
    if (variant == kSmall && M > kSmallRows)
        return fail(NVFP4_ERR_INVALID_ARG, "%s: the small-M variant takes M <= %d (M = %lld)", fn, kSmallRows, (long long)M);
    if (M > (int64_t)1 << 31) return fail(NVFP4_ERR_INVALID_ARG, "%s: M = %lld too large", fn, (long long)M);
    const Layout L = make_layout(1, N, K, mx);
    const bool empty = M == 0 || N == 0;
    if (variant == kResident && !empty && !xres_fits(L, M))
        return fail(NVFP4_ERR_INVALID_ARG, "%s: the activation-resident variant takes %s (M = %lld, N = %lld, K = %lld)",
                    fn, kXresLimits, (long long)M, (long long)N, (long long)K);
    // the MFMA-bound kernel addresses the code and scale regions with 32-bit offsets
    const bool mfma_fits = L.code_bytes() < ((int64_t)1 << 31);
    if ((variant == kMfma || variant == kMfmaQuarter) && !mfma_fits)
        return fail(NVFP4_ERR_INVALID_ARG, "%s: the MFMA-bound variant takes weights below 2 GiB of codes", fn);
    const int v = empty ? kAuto : variant == kAuto ? dense_auto_variant(L, M) : variant;
    Workspace wl{0, 0, 0};
    int64_t split_tiles = 0;
    if (v == kResident) {
        const XresShape xs = xres_shape(L, M);
        wl = workspace_for(xs);
        split_tiles = xs.S > 1 ? xs.groups : 0;
    } else if (v == kSmall) {
        const SmallShape sm = small_m_shape(L, M, false);
        wl = workspace_for(sm);
        split_tiles = sm.S > 1 ? sm.groups : 0;
    } else if (v == kLarge) {
        const TileShape t = tile_shape(L, M, false);
        wl = workspace_for(t);
        split_tiles = t.S > 1 ? t.tiles() : 0;
    }
    if (split_tiles > kMaxSplitTiles)   // the planners never split grids this large
        return fail(NVFP4_ERR_INVALID_ARG, "%s: %lld split-K tiles exceed the %lld counters of a workspace", fn,
                    (long long)split_tiles, (long long)kMaxSplitTiles);
    s = check_gemm_io(fn, x, ld_x, pre, w, gs, y, ld_y, M, N, K, ws, ws_bytes, wl.total, mx != 0);
    if (s != NVFP4_OK) return s;
    if (empty) return ok();   // zero rows or zero columns: nothing is launched
    uint8_t* wsb = static_cast<uint8_t*>(ws);
    GemmArgs a{static_cast<const uint16_t*>(x), ld_x, static_cast<const uint8_t*>(w), gs, g_div,
               static_cast<uint16_t*>(y), ld_y, M, nullptr, nullptr, static_cast<const uint16_t*>(pre),
               SplitK{1, nullptr, nullptr}, static_cast<hipStream_t>(stream)};
    switch (v) {
        case kResident: {
            const XresShape xs = xres_shape(L, M);
            a.sk = split_k(xs.S, wsb, wl);
            return launch_xres_any(xs, L, a, f16);
        }
        case kSmall: {
            const SmallShape sm = small_m_shape(L, M, false);
            a.sk = split_k(sm.S, wsb, wl);
            return f16 ? launch_small<true>(sm, L, a, false) : launch_small<false>(sm, L, a, false);
        }
        case kMfma:
        case kMfmaQuarter: {
            const hipError_t e = launch_gemm_mfma(mfma_plan(L, M), L, a.x, ld_x, a.blob, gs, g_div, a.y, ld_y, M, a.pre,
                                                  v == kMfmaQuarter, a.st, f16);
            if (e != hipSuccess) return fail(NVFP4_ERR_HIP, "%s: MFMA GEMM launch failed: %s", fn, hipGetErrorString(e));
            return ok();
        }
        default: {
            const TileShape t = tile_shape(L, M, false);
            a.sk = split_k(t.S, wsb, wl);
            return f16 ? launch_tile<true>(t, L, a, false) : launch_tile<false>(t, L, a, false);
        }
    }
}

// Grouped kernel choice (the test export nvfp4_w4a16_grouped_gemm_variant
// forces one): automatic, small-M, tile, MFMA-bound.
enum GroupedVariant { kGroupedAuto = 0, kGroupedSmall = 1, kGroupedTile = 2, kGroupedMfma = 3 };
// Average rows per expert from which the automatic choice takes the MFMA-bound
// kernel.  Measured (E = 128 or 64 experts of equal rows, N = 1536, K = 2048):
// its 256-row workgroups take about the same time however few of their rows
// an expert fills (16 to 512 rows: 242-250 us; latency-bound: a workgroup's
// weight copies run one chunk ahead, and distinct experts share nothing in
// L2), against 85, 93, 168, 300 and 295 us on the tile kernel at 16, 64, 128,
// 256 and 512 rows per expert.
constexpr int64_t kGroupedMfmaRowsPerExpert = 256;

// Grouped GEMM, shared by the plain and the gathering entry points: the
// activation has x_rows rows; grouped row r reads row row_index[r] of it
// (row r itself when row_index is NULL).  The grouped kernels never split K,
// so no workspace is needed.
nvfp4_status grouped_gemm(const char* fn, const void* x, int64_t ld_x, const int32_t* row_index,
                          const int32_t* expert_offsets, const void* pre_scale, const void* w_repacked,
                          const float* global_scales, int global_scale_is_divisor, void* y, int64_t ld_y, int64_t R,
                          int64_t E, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes, void* stream,
                          bool f16, int mx = 0, int act = kActNone, int variant = 0) {
    nvfp4_status s = check_weight_shape(fn, E, N, K, mx);
    if (s != NVFP4_OK) return s;
    // the gated epilogue writes N / 2 columns
    s = check_gemm_io(fn, x, ld_x, pre_scale, w_repacked, global_scales, y, ld_y, R, act == kActSiluGlu ? N / 2 : N,
                      K, workspace, workspace_bytes, 0, mx != 0);
    if (s != NVFP4_OK) return s;
    if (!expert_offsets) return fail(NVFP4_ERR_INVALID_ARG, "%s: expert_offsets is NULL", fn);
    if (!aligned(expert_offsets, 4)) return fail(NVFP4_ERR_ALIGNMENT, "%s: expert_offsets must be 4-byte aligned", fn);
    if (R > (int64_t)1 << 31) return fail(NVFP4_ERR_INVALID_ARG, "%s: R = %lld exceeds int32 offsets", fn, (long long)R);
    if (R == 0 || N == 0) return ok();   // zero rows or zero columns: nothing is launched
    const Layout L = make_layout(E, N, K, mx);
    GemmArgs a{static_cast<const uint16_t*>(x), ld_x, static_cast<const uint8_t*>(w_repacked), global_scales,
               global_scale_is_divisor != 0, static_cast<uint16_t*>(y), ld_y, R, expert_offsets, row_index,
               static_cast<const uint16_t*>(pre_scale), SplitK{1, nullptr, nullptr},
               static_cast<hipStream_t>(stream)};
    a.act = act;
    // Kernel: few rows per expert on average: the weight stream dominates, the small-M kernel (passes of 16
    // rows); many: the MFMA-bound kernel in 256-row tiles per expert (weights decoded once per expert and tile
    // column); between them the tile kernel (64-row tiles).
    const bool mfma_fits = L.code_bytes() < ((int64_t)1 << 31);
    if (variant == kGroupedAuto) {
        variant = R <= (int64_t)kSmallRows * E ? kGroupedSmall
                : (mfma_fits && act != kActRelu2 && R >= kGroupedMfmaRowsPerExpert * E) ? kGroupedMfma : kGroupedTile;
    }
    if (variant == kGroupedSmall) {
        const SmallShape sm = small_m_shape(L, R, true, act);
        return f16 ? launch_small<true>(sm, L, a, true) : launch_small<false>(sm, L, a, true);
    }
    if (variant == kGroupedMfma) {
        if (!mfma_fits) return fail(NVFP4_ERR_INVALID_ARG, "%s: the MFMA-bound kernel takes blobs below 2 GiB of codes", fn);
        if (act == kActRelu2) return fail(NVFP4_ERR_INVALID_ARG, "%s: the MFMA-bound kernel has no squared-ReLU epilogue", fn);
        const hipError_t e = launch_gemm_mfma_grouped(L, a.x, ld_x, row_index, expert_offsets, R, a.blob,
                                                      global_scales, a.g_div, a.y, ld_y, a.pre, act, a.st, f16);
        if (e != hipSuccess) return fail(NVFP4_ERR_HIP, "%s: MFMA GEMM launch failed: %s", fn, hipGetErrorString(e));
        return ok();
    }
    if (variant != kGroupedTile) return fail(NVFP4_ERR_INVALID_ARG, "%s: unknown variant %d", fn, variant);
    const TileShape t = tile_shape(L, R, true);
    return f16 ? launch_tile<true>(t, L, a, true) : launch_tile<false>(t, L, a, true);
}

// ---- MoE elementwise steps (bf16, or fp16 when f16)

nvfp4_status moe_silu_mul(const char* fn, const void* h, int64_t ld_h, int64_t R, int64_t I, void* a, int64_t ld_a,
                          void* stream, bool f16) {
    if (R < 0 || I < 1) return fail(NVFP4_ERR_INVALID_ARG, "%s: R = %lld, I = %lld", fn, (long long)R, (long long)I);
    if (ld_h < 2 * I) return fail(NVFP4_ERR_INVALID_ARG, "%s: ld_h = %lld < 2 I = %lld", fn, (long long)ld_h, (long long)(2 * I));
    if (ld_a < I) return fail(NVFP4_ERR_INVALID_ARG, "%s: ld_a = %lld < I = %lld", fn, (long long)ld_a, (long long)I);
    if (R > 0 && (!h || !a)) return fail(NVFP4_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(h, 2) || !aligned(a, 2)) return fail(NVFP4_ERR_ALIGNMENT, "%s: 16-bit arrays must be 2-byte aligned", fn);
    if (R == 0) return ok();
    const int64_t threads = R * ((I + 7) / 8);
    const bool vec = ld_h % 8 == 0 && I % 8 == 0 && ld_a % 8 == 0 && aligned(h, 16) && aligned(a, 16);
    const dim3 grid((unsigned)((threads + 255) / 256));
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (vec && f16) hipLaunchKernelGGL((k_moe_silu_mul<true, true>), grid, dim3(256), 0, st, static_cast<const uint16_t*>(h), ld_h, R, I, static_cast<uint16_t*>(a), ld_a);
    else if (vec) hipLaunchKernelGGL((k_moe_silu_mul<true, false>), grid, dim3(256), 0, st, static_cast<const uint16_t*>(h), ld_h, R, I, static_cast<uint16_t*>(a), ld_a);
    else if (f16) hipLaunchKernelGGL((k_moe_silu_mul<false, true>), grid, dim3(256), 0, st, static_cast<const uint16_t*>(h), ld_h, R, I, static_cast<uint16_t*>(a), ld_a);
    else hipLaunchKernelGGL((k_moe_silu_mul<false, false>), grid, dim3(256), 0, st, static_cast<const uint16_t*>(h), ld_h, R, I, static_cast<uint16_t*>(a), ld_a);
    return launched(fn);
}

nvfp4_status moe_relu2(const char* fn, const void* h, int64_t ld_h, int64_t R, int64_t I, void* a, int64_t ld_a,
                       void* stream, bool f16) {
    if (R < 0 || I < 1) return fail(NVFP4_ERR_INVALID_ARG, "%s: R = %lld, I = %lld", fn, (long long)R, (long long)I);
    if (ld_h < I) return fail(NVFP4_ERR_INVALID_ARG, "%s: ld_h = %lld < I = %lld", fn, (long long)ld_h, (long long)I);
    if (ld_a < I) return fail(NVFP4_ERR_INVALID_ARG, "%s: ld_a = %lld < I = %lld", fn, (long long)ld_a, (long long)I);
    if (R > 0 && (!h || !a)) return fail(NVFP4_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(h, 2) || !aligned(a, 2)) return fail(NVFP4_ERR_ALIGNMENT, "%s: 16-bit arrays must be 2-byte aligned", fn);
    if (R == 0) return ok();
    const int64_t threads = R * ((I + 7) / 8);
    const bool vec = ld_h % 8 == 0 && ld_a % 8 == 0 && aligned(h, 16) && aligned(a, 16);
    const dim3 grid((unsigned)((threads + 255) / 256));
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (vec && f16) hipLaunchKernelGGL((k_moe_relu2<true, true>), grid, dim3(256), 0, st, static_cast<const uint16_t*>(h), ld_h, R, I, static_cast<uint16_t*>(a), ld_a);
    else if (vec) hipLaunchKernelGGL((k_moe_relu2<true, false>), grid, dim3(256), 0, st, static_cast<const uint16_t*>(h), ld_h, R, I, static_cast<uint16_t*>(a), ld_a);
    else if (f16) hipLaunchKernelGGL((k_moe_relu2<false, true>), grid, dim3(256), 0, st, static_cast<const uint16_t*>(h), ld_h, R, I, static_cast<uint16_t*>(a), ld_a);
    else hipLaunchKernelGGL((k_moe_relu2<false, false>), grid, dim3(256), 0, st, static_cast<const uint16_t*>(h), ld_h, R, I, static_cast<uint16_t*>(a), ld_a);
    return launched(fn);
}

nvfp4_status moe_combine(const char* fn, const void* y, int64_t ld_y, const int32_t* token_row,
                         const float* topk_weights, int64_t T, int64_t k, int64_t H, void* out, int64_t ld_o,
                         void* stream, bool f16) {
    if (T < 0 || k < 1 || H < 1)
        return fail(NVFP4_ERR_INVALID_ARG, "%s: T = %lld, k = %lld, H = %lld", fn, (long long)T, (long long)k, (long long)H);
    if (ld_y < H || ld_o < H) return fail(NVFP4_ERR_INVALID_ARG, "%s: ld_y and ld_o must be >= H", fn);
    if (T > 0 && (!y || !token_row || !topk_weights || !out)) return fail(NVFP4_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(y, 2) || !aligned(out, 2) || !aligned(token_row, 4) || !aligned(topk_weights, 4))
        return fail(NVFP4_ERR_ALIGNMENT, "%s: misaligned pointer", fn);
    if (T == 0) return ok();
    const int64_t threads = T * ((H + 7) / 8);
    const bool vec = ld_y % 8 == 0 && ld_o % 8 == 0 && aligned(y, 16) && aligned(out, 16);
    const dim3 grid((unsigned)((threads + 255) / 256));
    hipStream_t st = static_cast<hipStream_t>(stream);
    const uint16_t* yy = static_cast<const uint16_t*>(y);
    uint16_t* oo = static_cast<uint16_t*>(out);
    if (vec && f16) hipLaunchKernelGGL((k_moe_combine<true, true>), grid, dim3(256), 0, st, yy, ld_y, token_row, topk_weights, T, (int)k, H, oo, ld_o);
    else if (vec) hipLaunchKernelGGL((k_moe_combine<true, false>), grid, dim3(256), 0, st, yy, ld_y, token_row, topk_weights, T, (int)k, H, oo, ld_o);
    else if (f16) hipLaunchKernelGGL((k_moe_combine<false, true>), grid, dim3(256), 0, st, yy, ld_y, token_row, topk_weights, T, (int)k, H, oo, ld_o);
    else hipLaunchKernelGGL((k_moe_combine<false, false>), grid, dim3(256), 0, st, yy, ld_y, token_row, topk_weights, T, (int)k, H, oo, ld_o);
    return launched(fn);
}

}  // namespace

extern "C" {

const char* nvfp4_last_error(void) { return g_err; }

int64_t nvfp4_repack_bytes(int64_t E, int64_t N, int64_t K) {
    if (check_weight_shape("nvfp4_repack_bytes", E, N, K) != NVFP4_OK) return -1;
    return make_layout(E, N, K).total_bytes();
}

}  // extern "C"

namespace {

nvfp4_status repack_impl(const char* fn, const uint8_t* w_packed, int64_t ld_w, const uint8_t* w_scale, int64_t ld_s,
                         int64_t E, int64_t N, int64_t K, void* out, int64_t out_bytes, void* stream, int mx,
                         int64_t gate_I = 0, int up_first = 0) {
    nvfp4_status s = check_weight_shape(fn, E, N, K, mx);
    if (s != NVFP4_OK) return s;
    if (gate_I > 0 && (N != 2 * gate_I || gate_I % kUnitN != 0))
        return fail(NVFP4_ERR_INVALID_ARG, "%s: the gated layout needs I = %lld to be a multiple of 16", fn,
                    (long long)gate_I);
    if (N == 0) return ok();   // no rows: nothing to repack, nothing is launched
    if (!w_packed) return fail(NVFP4_ERR_INVALID_ARG, "%s: w_packed is NULL", fn);
    if (!w_scale) return fail(NVFP4_ERR_INVALID_ARG, "%s: w_scale is NULL", fn);
    if (!out) return fail(NVFP4_ERR_INVALID_ARG, "%s: out is NULL", fn);
    if (ld_w < K / 2) return fail(NVFP4_ERR_INVALID_ARG, "%s: ld_w = %lld < K/2 = %lld", fn, (long long)ld_w, (long long)(K / 2));
    const int64_t group = mx ? 32 : 16;
    if (ld_s < K / group)
        return fail(NVFP4_ERR_INVALID_ARG, "%s: ld_s = %lld < K/%lld = %lld", fn, (long long)ld_s, (long long)group,
                    (long long)(K / group));
    if (!aligned(out, 16)) return fail(NVFP4_ERR_ALIGNMENT, "%s: out must be 16-byte aligned", fn);
    const Layout L = make_layout(E, N, K, mx);
    if (out_bytes < L.total_bytes())
        return fail(NVFP4_ERR_BUFFER_TOO_SMALL, "%s: out_bytes = %lld < %lld", fn, (long long)out_bytes, (long long)L.total_bytes());
    const int64_t lanes = L.blocks() * 64;
    uint8_t* o = static_cast<uint8_t*>(out);
    hipLaunchKernelGGL(k_repack, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, static_cast<hipStream_t>(stream),
                       w_packed, ld_w, w_scale, ld_s, N, K, L.NU, L.KC, lanes, make_view(L, o), o, o + L.code_bytes(),
                       mx, gate_I, up_first);
    return launched(fn);
}

nvfp4_status dequant_impl(const char* fn, const void* w_repacked, int64_t E, int64_t N, int64_t K, void* out,
                          int64_t ld_out, void* stream, int mx) {
    nvfp4_status s = check_weight_shape(fn, E, N, K, mx);
    if (s != NVFP4_OK) return s;
    if (N == 0) return ok();
    if (!w_repacked || !out) return fail(NVFP4_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (ld_out < K) return fail(NVFP4_ERR_INVALID_ARG, "%s: ld_out = %lld < K", fn, (long long)ld_out);
    if (!aligned(w_repacked, 16) || !aligned(out, 2)) return fail(NVFP4_ERR_ALIGNMENT, "%s: misaligned pointer", fn);
    const Layout L = make_layout(E, N, K, mx);
    const int64_t lanes = L.blocks() * 64;
    const uint8_t* b = static_cast<const uint8_t*>(w_repacked);
    hipLaunchKernelGGL(k_dequant, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, static_cast<hipStream_t>(stream),
                       make_view(L, b), N, K, L.NU, L.KC, lanes, static_cast<uint16_t*>(out), ld_out);
    return launched(fn);
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_repack(const uint8_t* w_packed, int64_t ld_w, const uint8_t* w_scale, int64_t ld_s, int64_t E,
                          int64_t N, int64_t K, void* out, int64_t out_bytes, void* stream) {
    return repack_impl("nvfp4_repack", w_packed, ld_w, w_scale, ld_s, E, N, K, out, out_bytes, stream, 0);
}

int64_t nvfp4_repack_gated_bytes(int64_t E, int64_t I, int64_t K) {
    if (I < 0 || I % kUnitN != 0) return -1;
    return nvfp4_repack_bytes(E, 2 * I, K);
}

nvfp4_status nvfp4_repack_gated(const uint8_t* w_packed, int64_t ld_w, const uint8_t* w_scale, int64_t ld_s,
                                int64_t E, int64_t I, int64_t K, int up_first, void* out, int64_t out_bytes,
                                void* stream) {
    const char* fn = "nvfp4_repack_gated";
    if (I < 0 || I % kUnitN != 0)
        return fail(NVFP4_ERR_INVALID_ARG, "%s: I = %lld must be a non-negative multiple of 16", fn, (long long)I);
    if (up_first != 0 && up_first != 1) return fail(NVFP4_ERR_INVALID_ARG, "%s: up_first must be 0 or 1", fn);
    return repack_impl(fn, w_packed, ld_w, w_scale, ld_s, E, 2 * I, K, out, out_bytes, stream, 0, I, up_first);
}

nvfp4_status nvfp4_dequant_bf16(const void* w_repacked, int64_t E, int64_t N, int64_t K, void* out, int64_t ld_out,
                                void* stream) {
    return dequant_impl("nvfp4_dequant_bf16", w_repacked, E, N, K, out, ld_out, stream, 0);
}

nvfp4_status nvfp4_bench_stream_read(const void* p, int64_t bytes, uint32_t* out, int64_t workgroups, int unroll,
                                     void* stream) {
    const char* fn = "nvfp4_bench_stream_read";
    if (bytes < 0 || bytes % 16 != 0) return fail(NVFP4_ERR_INVALID_ARG, "%s: bytes = %lld must be a multiple of 16", fn, (long long)bytes);
    if (workgroups < 1 || workgroups > (1 << 20)) return fail(NVFP4_ERR_INVALID_ARG, "%s: workgroups = %lld", fn, (long long)workgroups);
    if (bytes > 0 && (!p || !out)) return fail(NVFP4_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(p, 16) || !aligned(out, 4)) return fail(NVFP4_ERR_ALIGNMENT, "%s: misaligned pointer", fn);
    if (bytes == 0) return ok();
    const uint8_t* src = static_cast<const uint8_t*>(p);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)workgroups);
    switch (unroll) {
        case 1: hipLaunchKernelGGL(k_stream_read<1>, grid, dim3(256), 0, st, src, bytes / 16, out); break;
        case 2: hipLaunchKernelGGL(k_stream_read<2>, grid, dim3(256), 0, st, src, bytes / 16, out); break;
        case 4: hipLaunchKernelGGL(k_stream_read<4>, grid, dim3(256), 0, st, src, bytes / 16, out); break;
        case 8: hipLaunchKernelGGL(k_stream_read<8>, grid, dim3(256), 0, st, src, bytes / 16, out); break;
        default: return fail(NVFP4_ERR_INVALID_ARG, "%s: unroll = %d must be 1, 2, 4 or 8", fn, unroll);
    }
    return launched(fn);
}

int64_t nvfp4_w4a16_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || M > (int64_t)1 << 31 || check_weight_shape("nvfp4_w4a16_gemm_workspace_bytes", 1, N, K) != NVFP4_OK)
        return -1;
    return dense_workspace_bytes(make_layout(1, N, K), M);
}

int nvfp4_w4a16_gemm_variant_takes(int64_t M, int64_t N, int64_t K, int variant) {
    if (M < 0 || M > (int64_t)1 << 31 || check_weight_shape("nvfp4_w4a16_gemm_variant_takes", 1, N, K) != NVFP4_OK)
        return -1;
    const Layout L = make_layout(1, N, K);
    switch (variant) {
        case kAuto: case kLarge: return 1;
        case kSmall: return M <= kSmallRows;
        case kResident: return M == 0 || N == 0 || xres_fits(L, M);
        case kMfma: case kMfmaQuarter: return L.code_bytes() < ((int64_t)1 << 31);
        default: return -1;
    }
}

int nvfp4_w4a16_gemm_plan(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || M > (int64_t)1 << 31 || check_weight_shape("nvfp4_w4a16_gemm_plan", 1, N, K) != NVFP4_OK) return -1;
    return dense_auto_variant(make_layout(1, N, K), M);
}

nvfp4_status nvfp4_w4a16_gemm(const void* x, int64_t ld_x, const void* pre_scale, const void* w_repacked,
                              const float* global_scale, int global_scale_is_divisor, void* y, int64_t ld_y,
                              int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                              void* stream) {
    return dense_gemm(x, ld_x, pre_scale, w_repacked, global_scale, global_scale_is_divisor != 0, y, ld_y, M, N, K,
                      workspace, workspace_bytes, kAuto, stream, "nvfp4_w4a16_gemm", false);
}

nvfp4_status nvfp4_w4a16_gemm_f16(const void* x, int64_t ld_x, const void* pre_scale, const void* w_repacked,
                                  const float* global_scale, int global_scale_is_divisor, void* y, int64_t ld_y,
                                  int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                                  void* stream) {
    return dense_gemm(x, ld_x, pre_scale, w_repacked, global_scale, global_scale_is_divisor != 0, y, ld_y, M, N, K,
                      workspace, workspace_bytes, kAuto, stream, "nvfp4_w4a16_gemm_f16", true);
}

nvfp4_status nvfp4_w4a16_gemm_variant(const void* x, int64_t ld_x, const void* pre_scale, const void* w_repacked,
                                      const float* global_scale, int global_scale_is_divisor, void* y, int64_t ld_y,
                                      int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                                      int variant, void* stream) {
    return dense_gemm(x, ld_x, pre_scale, w_repacked, global_scale, global_scale_is_divisor != 0, y, ld_y, M, N, K,
                      workspace, workspace_bytes, variant, stream, "nvfp4_w4a16_gemm", false);
}

nvfp4_status nvfp4_w4a16_gemm_variant_f16(const void* x, int64_t ld_x, const void* pre_scale, const void* w_repacked,
                                          const float* global_scale, int global_scale_is_divisor, void* y,
                                          int64_t ld_y, int64_t M, int64_t N, int64_t K, void* workspace,
                                          int64_t workspace_bytes, int variant, void* stream) {
    return dense_gemm(x, ld_x, pre_scale, w_repacked, global_scale, global_scale_is_divisor != 0, y, ld_y, M, N, K,
                      workspace, workspace_bytes, variant, stream, "nvfp4_w4a16_gemm_f16", true);
}

int64_t nvfp4_w4a16_grouped_gemm_workspace_bytes(int64_t R, int64_t E, int64_t N, int64_t K) {
    if (R < 0 || check_weight_shape("nvfp4_w4a16_grouped_gemm_workspace_bytes", E, N, K) != NVFP4_OK) return -1;
    return 0;   // the grouped kernels never split K, and the pre-scale needs no copy
}

nvfp4_status nvfp4_w4a16_grouped_gemm(const void* x, int64_t ld_x, const int32_t* expert_offsets, const void* pre_scale,
                                      const void* w_repacked, const float* global_scales, int global_scale_is_divisor,
                                      void* y, int64_t ld_y, int64_t R, int64_t E, int64_t N, int64_t K,
                                      void* workspace, int64_t workspace_bytes, void* stream) {
    return grouped_gemm("nvfp4_w4a16_grouped_gemm", x, ld_x, nullptr, expert_offsets, pre_scale, w_repacked,
                        global_scales, global_scale_is_divisor, y, ld_y, R, E, N, K, workspace, workspace_bytes, stream,
                        false);
}

nvfp4_status nvfp4_w4a16_grouped_gemm_f16(const void* x, int64_t ld_x, const int32_t* expert_offsets,
                                          const void* pre_scale, const void* w_repacked, const float* global_scales,
                                          int global_scale_is_divisor, void* y, int64_t ld_y, int64_t R, int64_t E,
                                          int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                                          void* stream) {
    return grouped_gemm("nvfp4_w4a16_grouped_gemm_f16", x, ld_x, nullptr, expert_offsets, pre_scale, w_repacked,
                        global_scales, global_scale_is_divisor, y, ld_y, R, E, N, K, workspace, workspace_bytes, stream,
                        true);
}

int64_t nvfp4_w4a16_grouped_gemm_gather_workspace_bytes(int64_t T, int64_t R, int64_t E, int64_t N, int64_t K) {
    if (T < 0 || R < 0 || check_weight_shape("nvfp4_w4a16_grouped_gemm_gather_workspace_bytes", E, N, K) != NVFP4_OK)
        return -1;
    return 0;   // no K split, and the pre-scale needs no copy
}

static nvfp4_status grouped_gemm_gather(const char* fn, const void* x, int64_t ld_x, int64_t T,
                                        const int32_t* row_token, const int32_t* expert_offsets,
                                        const void* pre_scale, const void* w_repacked, const float* global_scales,
                                        int global_scale_is_divisor, void* y, int64_t ld_y, int64_t R, int64_t E,
                                        int64_t N, int64_t K, void* workspace, int64_t workspace_bytes, void* stream,
                                        bool f16, int act = kActNone, int variant = 0, int mx = 0) {
    if (T < 0) return fail(NVFP4_ERR_INVALID_ARG, "%s: token count %lld is negative", fn, (long long)T);
    if (R > 0 && !row_token) return fail(NVFP4_ERR_INVALID_ARG, "%s: row_token is NULL", fn);
    if (!aligned(row_token, 4)) return fail(NVFP4_ERR_ALIGNMENT, "%s: row_token must be 4-byte aligned", fn);
    if (R > 0 && T == 0) return fail(NVFP4_ERR_INVALID_ARG, "%s: %lld rows gather from 0 tokens", fn, (long long)R);
    // the kernels address a gathered row with a 32-bit byte offset from x
    if (T * ld_x >= ((int64_t)1 << 31))
        return fail(NVFP4_ERR_INVALID_ARG, "%s: T * ld_x = %lld must stay below 2^31", fn, (long long)(T * ld_x));
    return grouped_gemm(fn, x, ld_x, row_token, expert_offsets, pre_scale, w_repacked, global_scales,
                        global_scale_is_divisor, y, ld_y, R, E, N, K, workspace, workspace_bytes, stream, f16, mx, act,
                        variant);
}

// FC1 of a MoE layer with its activation in the epilogue: gated SiLU on a
// blob from nvfp4_repack_gated / mxfp4_repack_gated (N = 2 I), or the
// squared ReLU on a plain blob (N = I); row_token NULL: x holds the R
// grouped rows.  mx: an MXFP4 blob (no global scales).
static nvfp4_status moe_fc1(const char* fn, const void* x, int64_t ld_x, int64_t T, const int32_t* row_token,
                            const int32_t* expert_offsets, const void* pre_scale, const void* w_fc1,
                            const float* global_scales, int global_scale_is_divisor, int activation, void* a,
                            int64_t ld_a, int64_t R, int64_t E, int64_t I, int64_t K, void* stream, bool f16,
                            int mx = 0) {
    int act;
    if (activation == NVFP4_MOE_SILU_GLU) act = kActSiluGlu;
    else if (activation == NVFP4_MOE_RELU2) act = kActRelu2;
    else return fail(NVFP4_ERR_INVALID_ARG, "%s: activation %d is not NVFP4_MOE_SILU_GLU or NVFP4_MOE_RELU2", fn,
                     activation);
    if (I < 0) return fail(NVFP4_ERR_INVALID_ARG, "%s: I = %lld is negative", fn, (long long)I);
    if (act == kActSiluGlu && I % kUnitN != 0)
        return fail(NVFP4_ERR_INVALID_ARG, "%s: the gated layout needs I = %lld to be a multiple of 16", fn,
                    (long long)I);
    if (ld_a < I) return fail(NVFP4_ERR_INVALID_ARG, "%s: ld_a = %lld < I = %lld", fn, (long long)ld_a, (long long)I);
    const int64_t N = act == kActSiluGlu ? 2 * I : I;
    if (!row_token) {
        if (T != R) return fail(NVFP4_ERR_INVALID_ARG, "%s: without row_token x holds the R grouped rows (T = R)", fn);
        return grouped_gemm(fn, x, ld_x, nullptr, expert_offsets, pre_scale, w_fc1, global_scales,
                            global_scale_is_divisor, a, ld_a, R, E, N, K, nullptr, 0, stream, f16, mx, act);
    }
    return grouped_gemm_gather(fn, x, ld_x, T, row_token, expert_offsets, pre_scale, w_fc1, global_scales,
                               global_scale_is_divisor, a, ld_a, R, E, N, K, nullptr, 0, stream, f16, act,
                               kGroupedAuto, mx);
}

nvfp4_status nvfp4_w4a16_grouped_gemm_gather(const void* x, int64_t ld_x, int64_t T, const int32_t* row_token,
                                             const int32_t* expert_offsets, const void* pre_scale,
                                             const void* w_repacked, const float* global_scales,
                                             int global_scale_is_divisor, void* y, int64_t ld_y, int64_t R,
                                             int64_t E, int64_t N, int64_t K, void* workspace,
                                             int64_t workspace_bytes, void* stream) {
    return grouped_gemm_gather("nvfp4_w4a16_grouped_gemm_gather", x, ld_x, T, row_token, expert_offsets, pre_scale,
                               w_repacked, global_scales, global_scale_is_divisor, y, ld_y, R, E, N, K, workspace,
                               workspace_bytes, stream, false);
}

nvfp4_status nvfp4_w4a16_grouped_gemm_gather_f16(const void* x, int64_t ld_x, int64_t T, const int32_t* row_token,
                                                 const int32_t* expert_offsets, const void* pre_scale,
                                                 const void* w_repacked, const float* global_scales,
                                                 int global_scale_is_divisor, void* y, int64_t ld_y, int64_t R,
                                                 int64_t E, int64_t N, int64_t K, void* workspace,
                                                 int64_t workspace_bytes, void* stream) {
    return grouped_gemm_gather("nvfp4_w4a16_grouped_gemm_gather_f16", x, ld_x, T, row_token, expert_offsets,
                               pre_scale, w_repacked, global_scales, global_scale_is_divisor, y, ld_y, R, E, N, K,
                               workspace, workspace_bytes, stream, true);
}

nvfp4_status nvfp4_w4a16_grouped_gemm_variant(const void* x, int64_t ld_x, int64_t T, const int32_t* row_token,
                                              const int32_t* expert_offsets, const void* pre_scale, const void* w,
                                              const float* global_scales, int global_scale_is_divisor, int activation,
                                              void* y, int64_t ld_y, int64_t R, int64_t E, int64_t N, int64_t K,
                                              int variant, int f16, int mx, void* stream) {
    const char* fn = "nvfp4_w4a16_grouped_gemm_variant";
    if (mx != 0 && mx != 1) return fail(NVFP4_ERR_INVALID_ARG, "%s: mx must be 0 or 1", fn);
    int act;
    if (activation == 0) act = kActNone;
    else if (activation == NVFP4_MOE_SILU_GLU) act = kActSiluGlu;
    else if (activation == NVFP4_MOE_RELU2) act = kActRelu2;
    else return fail(NVFP4_ERR_INVALID_ARG, "%s: unknown activation %d", fn, activation);
    if (variant < kGroupedAuto || variant > kGroupedMfma)
        return fail(NVFP4_ERR_INVALID_ARG, "%s: unknown variant %d", fn, variant);
    if (act == kActSiluGlu && N % (2 * kUnitN) != 0)
        return fail(NVFP4_ERR_INVALID_ARG, "%s: the gated layout needs N = %lld to be a multiple of 32", fn,
                    (long long)N);
    if (!row_token) {
        if (T != R) return fail(NVFP4_ERR_INVALID_ARG, "%s: without row_token x holds the R grouped rows (T = R)", fn);
        return grouped_gemm(fn, x, ld_x, nullptr, expert_offsets, pre_scale, w, mx ? nullptr : global_scales,
                            global_scale_is_divisor, y, ld_y, R, E, N, K, nullptr, 0, stream, f16 != 0, mx, act,
                            variant);
    }
    return grouped_gemm_gather(fn, x, ld_x, T, row_token, expert_offsets, pre_scale, w, mx ? nullptr : global_scales,
                               global_scale_is_divisor, y, ld_y, R, E, N, K, nullptr, 0, stream, f16 != 0, act,
                               variant, mx);
}

nvfp4_status nvfp4_moe_fc1(const void* x, int64_t ld_x, int64_t T, const int32_t* row_token,
                           const int32_t* expert_offsets, const void* pre_scale, const void* w_fc1,
                           const float* global_scales, int global_scale_is_divisor, int activation, void* a,
                           int64_t ld_a, int64_t R, int64_t E, int64_t I, int64_t K, void* stream) {
    return moe_fc1("nvfp4_moe_fc1", x, ld_x, T, row_token, expert_offsets, pre_scale, w_fc1, global_scales,
                   global_scale_is_divisor, activation, a, ld_a, R, E, I, K, stream, false);
}

nvfp4_status nvfp4_moe_fc1_f16(const void* x, int64_t ld_x, int64_t T, const int32_t* row_token,
                               const int32_t* expert_offsets, const void* pre_scale, const void* w_fc1,
                               const float* global_scales, int global_scale_is_divisor, int activation, void* a,
                               int64_t ld_a, int64_t R, int64_t E, int64_t I, int64_t K, void* stream) {
    return moe_fc1("nvfp4_moe_fc1_f16", x, ld_x, T, row_token, expert_offsets, pre_scale, w_fc1, global_scales,
                   global_scale_is_divisor, activation, a, ld_a, R, E, I, K, stream, true);
}

// --------------------------------------------------- no-allocation entry --
// nvfp4_w4a16_gemm_noalloc keeps its split-K partials and counters in a
// file-scope device array instead of a caller's workspace.  The array's name
// is a host-side stand-in in host code: the kernels get the address that
// hipGetSymbolAddress returns for the current device, taken once per device
// on that device's first call and kept.

}  // extern "C"

namespace {

constexpr int64_t kScratchBytes = int64_t(4) << 20;   // 4 MiB per device (a call needing more is rejected)
static_assert(kScratchBytes > kMaxSplitTiles * 4, "the counter prefix fits");
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

// Zero n dwords (a fill kernel rather than a memset, so that a call under
// graph capture records nothing but kernels).
__global__ void __launch_bounds__(256) k_zero_dwords(uint32_t* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// The device address of this device's scratch array.  On the device's first
// call: the address from hipGetSymbolAddress (checked), and the counter
// prefix cleared on `st` (split-K calls leave the counters they use at zero,
// so it stays clear from then on; the array starts zeroed when the code
// object loads, the clear makes that explicit).
nvfp4_status scratch_address(const char* fn, hipStream_t st, uint8_t** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(NVFP4_ERR_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kScratchDevices)
        return fail(NVFP4_ERR_INVALID_ARG, "%s: device %d beyond the %d this library tracks", fn, dev, kScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(NVFP4_ERR_HIP, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", fn, dev,
                        hipGetErrorString(e));
        hipLaunchKernelGGL(k_zero_dwords, dim3((unsigned)((kMaxSplitTiles + 255) / 256)), dim3(256), 0, st,
                           static_cast<uint32_t*>(p), kMaxSplitTiles);
        const nvfp4_status s = launched(fn);
        if (s != NVFP4_OK) return s;
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<uint8_t*>(g_scratch_ptr[dev]);
    return NVFP4_OK;
}

}  // namespace

extern "C" {

int64_t nvfp4_w4a16_gemm_noalloc_max_scratch_bytes(void) { return kScratchBytes; }

nvfp4_status nvfp4_w4a16_gemm_noalloc(const void* x, int64_t ld_x, const void* pre_scale, const void* w_repacked,
                                      const float* global_scale, int global_scale_is_divisor, void* y, int64_t ld_y,
                                      int64_t M, int64_t N, int64_t K, void* stream) {
    const char* fn = "nvfp4_w4a16_gemm_noalloc";
    if (check_weight_shape(fn, 1, N, K) != NVFP4_OK) return NVFP4_ERR_INVALID_ARG;
    if (M < 0 || M > (int64_t)1 << 31) return fail(NVFP4_ERR_INVALID_ARG, "%s: M = %lld out of range", fn, (long long)M);
    const int64_t need = dense_workspace_bytes(make_layout(1, N, K), M);
    if (need > kScratchBytes)
        return fail(NVFP4_ERR_BUFFER_TOO_SMALL,
                    "%s: this call needs %lld bytes of split-K scratch, above the %lld bytes of the no-allocation "
                    "entry point (nvfp4_w4a16_gemm with a workspace takes it)",
                    fn, (long long)need, (long long)kScratchBytes);
    uint8_t* ws = nullptr;
    if (need > 0) {
        const nvfp4_status s = scratch_address(fn, static_cast<hipStream_t>(stream), &ws);
        if (s != NVFP4_OK) return s;
    }
    return dense_gemm(x, ld_x, pre_scale, w_repacked, global_scale, global_scale_is_divisor != 0, y, ld_y, M, N, K,
                      ws, need > 0 ? kScratchBytes : 0, kAuto, stream, fn, false);
}

// ---------------------------------------------------------------- MXFP4 --
// The same GEMMs on MXFP4 weights: one E8M0 scale per 32 K and no global
// scale.  Repacked into the NVFP4 layout (the blob size and the workspace
// sizes are those of the NVFP4 calls), decoded with E8M0 scales.

int64_t mxfp4_repack_bytes(int64_t E, int64_t N, int64_t K) {
    if (check_weight_shape("mxfp4_repack_bytes", E, N, K, 1) != NVFP4_OK) return -1;
    return make_layout(E, N, K, 1).total_bytes();
}

nvfp4_status mxfp4_repack(const uint8_t* w_packed, int64_t ld_w, const uint8_t* w_scale, int64_t ld_s, int64_t E,
                          int64_t N, int64_t K, void* out, int64_t out_bytes, void* stream) {
    return repack_impl("mxfp4_repack", w_packed, ld_w, w_scale, ld_s, E, N, K, out, out_bytes, stream, 1);
}

int64_t mxfp4_repack_gated_bytes(int64_t E, int64_t I, int64_t K) {
    if (I < 0 || I % kUnitN != 0) return -1;
    return mxfp4_repack_bytes(E, 2 * I, K);
}

nvfp4_status mxfp4_repack_gated(const uint8_t* w_packed, int64_t ld_w, const uint8_t* w_scale, int64_t ld_s,
                                int64_t E, int64_t I, int64_t K, int up_first, void* out, int64_t out_bytes,
                                void* stream) {
    const char* fn = "mxfp4_repack_gated";
    if (I < 0 || I % kUnitN != 0)
        return fail(NVFP4_ERR_INVALID_ARG, "%s: I = %lld must be a non-negative multiple of 16", fn, (long long)I);
    if (up_first != 0 && up_first != 1) return fail(NVFP4_ERR_INVALID_ARG, "%s: up_first must be 0 or 1", fn);
    return repack_impl(fn, w_packed, ld_w, w_scale, ld_s, E, 2 * I, K, out, out_bytes, stream, 1, I, up_first);
}

nvfp4_status mxfp4_moe_fc1(const void* x, int64_t ld_x, int64_t T, const int32_t* row_token,
                           const int32_t* expert_offsets, const void* pre_scale, const void* w_fc1, int activation,
                           void* a, int64_t ld_a, int64_t R, int64_t E, int64_t I, int64_t K, void* stream) {
    return moe_fc1("mxfp4_moe_fc1", x, ld_x, T, row_token, expert_offsets, pre_scale, w_fc1, nullptr, 0, activation,
                   a, ld_a, R, E, I, K, stream, false, 1);
}

nvfp4_status mxfp4_moe_fc1_f16(const void* x, int64_t ld_x, int64_t T, const int32_t* row_token,
                               const int32_t* expert_offsets, const void* pre_scale, const void* w_fc1, int activation,
                               void* a, int64_t ld_a, int64_t R, int64_t E, int64_t I, int64_t K, void* stream) {
    return moe_fc1("mxfp4_moe_fc1_f16", x, ld_x, T, row_token, expert_offsets, pre_scale, w_fc1, nullptr, 0,
                   activation, a, ld_a, R, E, I, K, stream, true, 1);
}

nvfp4_status mxfp4_dequant_bf16(const void* w_repacked, int64_t E, int64_t N, int64_t K, void* out, int64_t ld_out,
                                void* stream) {
    return dequant_impl("mxfp4_dequant_bf16", w_repacked, E, N, K, out, ld_out, stream, 1);
}

nvfp4_status mxfp4_w4a16_gemm(const void* x, int64_t ld_x, const void* pre_scale, const void* w_repacked, void* y,
                              int64_t ld_y, int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                              void* stream) {
    return dense_gemm(x, ld_x, pre_scale, w_repacked, nullptr, 0, y, ld_y, M, N, K, workspace, workspace_bytes, kAuto,
                      stream, "mxfp4_w4a16_gemm", false, 1);
}

nvfp4_status mxfp4_w4a16_gemm_f16(const void* x, int64_t ld_x, const void* pre_scale, const void* w_repacked, void* y,
                                  int64_t ld_y, int64_t M, int64_t N, int64_t K, void* workspace,
                                  int64_t workspace_bytes, void* stream) {
    return dense_gemm(x, ld_x, pre_scale, w_repacked, nullptr, 0, y, ld_y, M, N, K, workspace, workspace_bytes, kAuto,
                      stream, "mxfp4_w4a16_gemm_f16", true, 1);
}

nvfp4_status mxfp4_w4a16_gemm_variant(const void* x, int64_t ld_x, const void* pre_scale, const void* w_repacked,
                                      void* y, int64_t ld_y, int64_t M, int64_t N, int64_t K, void* workspace,
                                      int64_t workspace_bytes, int variant, int f16, void* stream) {
    return dense_gemm(x, ld_x, pre_scale, w_repacked, nullptr, 0, y, ld_y, M, N, K, workspace, workspace_bytes,
                      variant, stream, "mxfp4_w4a16_gemm_variant", f16 != 0, 1);
}

nvfp4_status mxfp4_w4a16_grouped_gemm(const void* x, int64_t ld_x, const int32_t* expert_offsets, const void* pre_scale,
                                      const void* w_repacked, void* y, int64_t ld_y, int64_t R, int64_t E, int64_t N,
                                      int64_t K, void* workspace, int64_t workspace_bytes, void* stream) {
    return grouped_gemm("mxfp4_w4a16_grouped_gemm", x, ld_x, nullptr, expert_offsets, pre_scale, w_repacked, nullptr, 0,
                        y, ld_y, R, E, N, K, workspace, workspace_bytes, stream, false, 1);
}

nvfp4_status mxfp4_w4a16_grouped_gemm_f16(const void* x, int64_t ld_x, const int32_t* expert_offsets,
                                          const void* pre_scale, const void* w_repacked, void* y, int64_t ld_y,
                                          int64_t R, int64_t E, int64_t N, int64_t K, void* workspace,
                                          int64_t workspace_bytes, void* stream) {
    return grouped_gemm("mxfp4_w4a16_grouped_gemm_f16", x, ld_x, nullptr, expert_offsets, pre_scale, w_repacked,
                        nullptr, 0, y, ld_y, R, E, N, K, workspace, workspace_bytes, stream, true, 1);
}

// ------------------------------------------------------------------ MoE --

int64_t nvfp4_moe_route_workspace_bytes(int64_t T, int64_t k, int64_t E) {
    if (T < 0 || k < 1 || E < 1 || E > kRouteMaxExperts || T * k >= ((int64_t)1 << 31)) return -1;
    return (T * k + kRouteThreads - 1) / kRouteThreads * E * 4;
}

nvfp4_status nvfp4_moe_route(const int32_t* topk_ids, int64_t T, int64_t k, int64_t E, int32_t* expert_offsets,
                             int32_t* row_token, int32_t* token_row, void* workspace, int64_t workspace_bytes,
                             void* stream) {
    const char* fn = "nvfp4_moe_route";
    if (T < 0) return fail(NVFP4_ERR_INVALID_ARG, "%s: token count %lld is negative", fn, (long long)T);
    if (E < 1 || E > kRouteMaxExperts)
        return fail(NVFP4_ERR_INVALID_ARG, "%s: E = %lld must be in [1, %d]", fn, (long long)E, kRouteMaxExperts);
    if (k < 1 || k > E) return fail(NVFP4_ERR_INVALID_ARG, "%s: k = %lld must be in [1, E]", fn, (long long)k);
    if (T * k >= ((int64_t)1 << 31)) return fail(NVFP4_ERR_INVALID_ARG, "%s: T * k must stay below 2^31", fn);
    if (!expert_offsets) return fail(NVFP4_ERR_INVALID_ARG, "%s: expert_offsets is NULL", fn);
    if (T > 0 && (!topk_ids || !row_token || !token_row))
        return fail(NVFP4_ERR_INVALID_ARG, "%s: topk_ids, row_token and token_row must not be NULL", fn);
    if (!aligned(topk_ids, 4) || !aligned(expert_offsets, 4) || !aligned(row_token, 4) || !aligned(token_row, 4))
        return fail(NVFP4_ERR_ALIGNMENT, "%s: int32 arrays must be 4-byte aligned", fn);
    const int64_t need = nvfp4_moe_route_workspace_bytes(T, k, E);
    if (T > 0 && (workspace_bytes < need || !workspace))
        return fail(NVFP4_ERR_BUFFER_TOO_SMALL, "%s: workspace of %lld bytes is below the %lld bytes this call needs",
                    fn, (long long)workspace_bytes, (long long)need);
    if (!aligned(workspace, 4)) return fail(NVFP4_ERR_ALIGNMENT, "%s: workspace must be 4-byte aligned", fn);
    if (T == 0) return ok();   // zero tokens: nothing is launched
    const int64_t P = T * k, blocks = (P + kRouteThreads - 1) / kRouteThreads;
    if (blocks > INT32_MAX) return fail(NVFP4_ERR_INVALID_ARG, "%s: too many pairs", fn);
    hipStream_t st = static_cast<hipStream_t>(stream);
    int32_t* hist = static_cast<int32_t*>(workspace);
    if (blocks == 1) {   // one workgroup counts, scans and places
        hipLaunchKernelGGL(k_moe_route_place, dim3(1), dim3(kRouteThreads), 0, st, topk_ids, P, (int)E,
                           (const int32_t*)nullptr, row_token, token_row, (int)k, expert_offsets);
        return launched(fn);
    }
    hipLaunchKernelGGL(k_moe_route_count, dim3((unsigned)blocks), dim3(kRouteThreads), 0, st, topk_ids, P, (int)E, hist);
    if (blocks <= kRouteRawBlocks) {   // the place workgroups scan the raw counts themselves: no scan launch
        hipLaunchKernelGGL(k_moe_route_place, dim3((unsigned)blocks), dim3(kRouteThreads), 0, st, topk_ids, P, (int)E,
                           (const int32_t*)hist, row_token, token_row, (int)k, expert_offsets, (int)blocks);
        return launched(fn);
    }
    hipLaunchKernelGGL(k_moe_route_scan, dim3(1), dim3(kRouteThreads), 0, st, hist, blocks, (int)E, P, expert_offsets);
    hipLaunchKernelGGL(k_moe_route_place, dim3((unsigned)blocks), dim3(kRouteThreads), 0, st, topk_ids, P, (int)E,
                       (const int32_t*)hist, row_token, token_row, (int)k, expert_offsets, 0);
    return launched(fn);
}

nvfp4_status nvfp4_moe_silu_mul(const void* h, int64_t ld_h, int64_t R, int64_t I, void* a, int64_t ld_a,
                                void* stream) {
    return moe_silu_mul("nvfp4_moe_silu_mul", h, ld_h, R, I, a, ld_a, stream, false);
}

nvfp4_status nvfp4_moe_silu_mul_f16(const void* h, int64_t ld_h, int64_t R, int64_t I, void* a, int64_t ld_a,
                                    void* stream) {
    return moe_silu_mul("nvfp4_moe_silu_mul_f16", h, ld_h, R, I, a, ld_a, stream, true);
}

nvfp4_status nvfp4_moe_relu2(const void* h, int64_t ld_h, int64_t R, int64_t I, void* a, int64_t ld_a,
                             void* stream) {
    return moe_relu2("nvfp4_moe_relu2", h, ld_h, R, I, a, ld_a, stream, false);
}

nvfp4_status nvfp4_moe_relu2_f16(const void* h, int64_t ld_h, int64_t R, int64_t I, void* a, int64_t ld_a,
                                 void* stream) {
    return moe_relu2("nvfp4_moe_relu2_f16", h, ld_h, R, I, a, ld_a, stream, true);
}

nvfp4_status nvfp4_moe_combine(const void* y, int64_t ld_y, const int32_t* token_row, const float* topk_weights,
                               int64_t T, int64_t k, int64_t H, void* out, int64_t ld_o, void* stream) {
    return moe_combine("nvfp4_moe_combine", y, ld_y, token_row, topk_weights, T, k, H, out, ld_o, stream, false);
}

nvfp4_status nvfp4_moe_combine_f16(const void* y, int64_t ld_y, const int32_t* token_row, const float* topk_weights,
                                   int64_t T, int64_t k, int64_t H, void* out, int64_t ld_o, void* stream) {
    return moe_combine("nvfp4_moe_combine_f16", y, ld_y, token_row, topk_weights, T, k, H, out, ld_o, stream, true);
}

}  // extern "C"
