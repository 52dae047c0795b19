// C ABI of the W4A16 NVFP4 GEMM library (see include/nvfp4_w4a16.h).
//
// Host side: argument checks (all before any launch), size queries, kernel
// choice and launches.  Everything is stream-ordered and asynchronous; the
// host never waits on the device and never reads device memory.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/nvfp4_w4a16.h"
#include "kernels_aux.h"
#include "kernels_gemm.h"
#include "kernels_moe.h"
#include "kernels_tile.h"
#include "kernels_xres.h"
#include "launch_mfma.h"

using namespace nvfp4;

namespace {

thread_local char g_err[512] = "";

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

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

nvfp4_status launched(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(NVFP4_ERR_HIP, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

nvfp4_status check_weight_shape(const char* fn, int64_t E, int64_t N, int64_t K) {
    if (E < 1 || E > kMaxExperts) return fail(NVFP4_ERR_INVALID_ARG, "%s: E = %lld must be in [1, %d]", fn, (long long)E, kMaxExperts);
    if (N < 1 || N > (int64_t)1 << 30) return fail(NVFP4_ERR_INVALID_ARG, "%s: N = %lld must be in [1, 2^30]", fn, (long long)N);
    if (K < 16 || K % 16 != 0 || K > (int64_t)1 << 30)
        return fail(NVFP4_ERR_INVALID_ARG, "%s: K = %lld must be a positive multiple of 16 (one E4M3 scale per 16 K)", fn, (long long)K);
    return NVFP4_OK;
}

// Bytes of the pre-scaled activation copy kept in the workspace.
int64_t prescale_bytes(int64_t rows, int64_t K) { return round_up(rows * K * 2, 256); }

enum Variant { kAuto = 0, kSmall = 1, kLarge = 2, kMfma = 3, kResident = 4 };

// Small-M launch shape: row form mg (1, 2: 4x4x4 with that many row groups;
// 16: 16x16x32), nt units per wave, w waves per workgroup, ring depth d, and
// K splits S across workgroups (dense only).  Only the (mg, nt, w, d) tuples
// listed in NVFP4_SMALL_CONFIGS are compiled.
struct SmallShape {
    int mg, nt, w, d, S;
    int64_t groups;   // workgroups along N (units / nt)
};

// (mg, nt, w, d) for the dense form; the grouped form is always (0, 1, w, 4).
#define NVFP4_SMALL_CONFIGS(X) \
    X(1, 1, 1, 4) X(1, 1, 2, 4) X(1, 1, 4, 4) X(1, 1, 8, 4) X(1, 1, 16, 4) \
    X(2, 1, 1, 4) X(2, 1, 2, 4) X(2, 1, 4, 4) X(2, 1, 8, 4) X(2, 2, 2, 4) X(2, 2, 4, 4) X(2, 2, 8, 4) \
    X(16, 2, 4, 2) X(16, 2, 8, 2) X(16, 4, 4, 2) X(16, 4, 8, 2) X(16, 8, 4, 2) X(16, 8, 8, 2)

// Is (mg, nt, w, d) one of the compiled dense shapes?
bool small_compiled(const SmallShape& s) {
    bool found = false;
#define NVFP4_SMALL_FIND(MG, NT, W, D) found = found || (s.mg == MG && s.nt == NT && s.w == W && s.d == D);
    NVFP4_SMALL_CONFIGS(NVFP4_SMALL_FIND)
#undef NVFP4_SMALL_FIND
    return found;
}

// Shapes from launch sweeps on MI355X (graph-replayed, weights rotated past
// the Infinity Cache).  Rows <= 8: one unit per wave, waves sized so the
// workgroups x waves x ring depth product aims at about 32 KB of weight
// loads in flight per CU.  Rows 9..16 (16x16x32 form, about two VALU
// operations per weight to decode) share each activation fragment over four
// units per wave; the automatic choice sends those rows to the tile kernel,
// which measured as fast.
SmallShape small_m_shape(const Layout& L, int64_t rows, bool grouped) {
    SmallShape s;
    s.S = 1;
    if (grouped) {
        s.mg = 0; s.nt = 1; s.d = 4;
    } else if (rows <= 8) {
        s.mg = rows <= 4 ? 1 : 2; s.nt = 1; s.d = 4;
    } else {
        s.mg = 16; s.nt = 4; s.d = 2; s.w = 4;
    }
    s.groups = (L.NU + s.nt - 1) / s.nt;
    if (s.mg == 16) {
        // a K split costs a device-scope publish / count / reload round trip
        // at the end of the kernel: split only grids that fill under half
        // of the CUs
        while (s.S < 8 && s.groups * s.S < 128 && L.KC >= 2 * s.w * 2 * s.S) s.S *= 2;
        return s;
    }
    const int64_t ctas = s.groups * (grouped ? (L.E + 1) / 2 : 1);
    s.w = 1;
    // 16 waves cap a kernel at 128 VGPRs: only the one-row-group form fits
    const int wmax = s.mg == 1 ? 16 : 8;
    while (s.w < wmax && ctas * (2 * s.w) * s.d <= 8192 && L.KC >= 4 * (2 * s.w)) s.w *= 2;
    if (s.w < 2 && L.KC >= 8) s.w = 2;
    while (!grouped && s.w > 1 && !small_compiled(s)) s.w /= 2;
    return s;
}


template <int MG, int NT, int W, int D, bool GROUPED>
void launch_small_t(const SmallShape& s, const Layout& L, const uint16_t* x, int64_t ld_x, const uint8_t* blob,
                    const float* gs, int g_div, uint16_t* y, int64_t ld_y, int64_t rows, const int32_t* offsets,
                    SplitK sk, hipStream_t st, bool f16, const int32_t* row_index = nullptr) {
    const BlobView bv = make_view(L, blob);
    const dim3 grid((unsigned)s.groups, GROUPED ? (unsigned)L.E : 1u, (unsigned)s.S);
    const bool kfull = L.K % kChunkK == 0;
#define NVFP4_SMALL_LAUNCH(KF, F16)                                                                              \
    hipLaunchKernelGGL((k_gemm_small_m<MG, NT, W, D, GROUPED, KF, F16>), grid, dim3(W * 64), 0, st, x, ld_x, bv, \
                       (int)L.NU, (int)L.KC, (int)L.K, (int)L.N, gs, g_div, y, ld_y, rows, offsets, sk, row_index)
    if (f16) {
        if (kfull) NVFP4_SMALL_LAUNCH(true, true);
        else NVFP4_SMALL_LAUNCH(false, true);
    } else {
        if (kfull) NVFP4_SMALL_LAUNCH(true, false);
        else NVFP4_SMALL_LAUNCH(false, false);
    }
#undef NVFP4_SMALL_LAUNCH
}

template <bool GROUPED>
nvfp4_status launch_small(const SmallShape& s, const Layout& L, const uint16_t* x, int64_t ld_x, const uint8_t* blob,
                          const float* gs, int g_div, uint16_t* y, int64_t ld_y, int64_t rows_dense,
                          const int32_t* offsets, SplitK sk, hipStream_t st, bool f16,
                          const int32_t* row_index = nullptr) {
    bool done = false;
    if constexpr (GROUPED) {
        switch (s.w) {
            case 1: launch_small_t<0, 1, 1, 4, true>(s, L, x, ld_x, blob, gs, g_div, y, ld_y, 0, offsets, sk, st, f16, row_index); break;
            case 2: launch_small_t<0, 1, 2, 4, true>(s, L, x, ld_x, blob, gs, g_div, y, ld_y, 0, offsets, sk, st, f16, row_index); break;
            case 4: launch_small_t<0, 1, 4, 4, true>(s, L, x, ld_x, blob, gs, g_div, y, ld_y, 0, offsets, sk, st, f16, row_index); break;
            default: launch_small_t<0, 1, 8, 4, true>(s, L, x, ld_x, blob, gs, g_div, y, ld_y, 0, offsets, sk, st, f16, row_index); break;
        }
        done = true;
    } else {
#define NVFP4_SMALL_DISPATCH(MG, NT, W, D)                                                                        \
    if (!done && s.mg == MG && s.nt == NT && s.w == W && s.d == D) {                                            \
        launch_small_t<MG, NT, W, D, false>(s, L, x, ld_x, blob, gs, g_div, y, ld_y, rows_dense, nullptr, sk, st, f16); \
        done = true;                                                                                            \
    }
        NVFP4_SMALL_CONFIGS(NVFP4_SMALL_DISPATCH)
#undef NVFP4_SMALL_DISPATCH
    }
    if (!done)
        return fail(NVFP4_ERR_INVALID_ARG, "small-M GEMM: no compiled kernel for shape mg=%d nt=%d w=%d d=%d", s.mg,
                    s.nt, s.w, s.d);
    return launched("small-M GEMM");
}

// ------------------------------------------------------------- tile path --
// Tile shapes by row count, from launch-shape sweeps on MI355X: the fastest
// decode-sized shapes run about one 16-wave workgroup per CU, four unit-waves
// times four k-parts.  K is further split across workgroups (grid z) while
// the workgroup count stays at or below 256 and every wave keeps >= 2
// chunks.  The choice is a pure function of (rows, N, K), so the workspace
// query reproduces it.
struct TileShape {
    int ms, nt, uw, kw, d, S;
    int64_t groups, mtiles;
    int64_t tiles() const { return groups * mtiles; }
    int bm() const { return 16 * ms; }
    int ug() const { return nt * uw; }
};

TileShape tile_shape(const Layout& L, int64_t rows, bool grouped) {
    TileShape t;
    bool split = true;
    if (grouped) {
        t.ms = 4; t.nt = 4; t.uw = 4; t.kw = 1; t.d = 2; split = false;
    } else if (rows <= 16) {
        t.ms = 1; t.nt = 1; t.uw = 4; t.kw = 4; t.d = 2;
    } else if (rows <= 32) {
        t.ms = 2; t.nt = 1; t.uw = 4; t.kw = 2; t.d = 4;
    } else if (rows <= 192) {
        // 64-row tiles: up to three row tiles still beat 128-row tiles here
        // (measured); wide N (LM heads) takes 512 columns per workgroup with
        // a 3-deep weight ring
        if (L.NU >= 4096) { t.ms = 4; t.nt = 4; t.uw = 8; t.kw = 1; t.d = 3; }
        else { t.ms = 4; t.nt = 1; t.uw = 4; t.kw = 4; t.d = 2; }
    } else {
        t.ms = 8; t.nt = 2; t.uw = 8; t.kw = 1; t.d = 2;
    }
    t.groups = (L.NU + t.ug() - 1) / t.ug();
    t.mtiles = (rows + t.bm() - 1) / t.bm() + (grouped ? L.E : 0);
    t.S = 1;
    while (split && t.S < 16 && t.tiles() * 2 * t.S <= 256 && L.KC >= 2 * t.kw * (2 * t.S)) t.S *= 2;
    return t;
}

// Byte offsets in the caller's workspace: split-K counters (must be zero
// before the first call; every call leaves them zero), split-K partials, and
// the pre-scaled activation.
struct Workspace {
    int64_t counters, partials, prescale, total;
};

// split_tiles tiles of tile_floats fp32 each, S splits (no split-K area when S == 1).
Workspace workspace_layout(int S, int64_t split_tiles, int64_t tile_floats, int64_t rows, int64_t K, bool pre) {
    Workspace w{0, 0, 0, 0};
    int64_t off = 0;
    if (S > 1) {
        w.counters = off;
        off += round_up(split_tiles * 4, 256);
        w.partials = off;
        off += round_up((int64_t)S * split_tiles * tile_floats * 4, 256);
    }
    if (pre) {
        w.prescale = off;
        off += prescale_bytes(rows, K);
    }
    w.total = off;
    return w;
}

Workspace workspace_for(const TileShape& t, int64_t rows, int64_t K, bool pre) {
    return workspace_layout(t.S, t.tiles(), (int64_t)t.bm() * t.ug() * 16, rows, K, pre);
}

Workspace workspace_for(const SmallShape& s, int64_t rows, int64_t K, bool pre) {
    return workspace_layout(s.S, s.groups, (int64_t)kSmallRows * 16 * s.nt, rows, K, pre);
}

SplitK split_k(int S, uint8_t* ws, const Workspace& wl) {
    return SplitK{S, S > 1 ? reinterpret_cast<float*>(ws + wl.partials) : nullptr,
                  S > 1 ? reinterpret_cast<int*>(ws + wl.counters) : nullptr};
}

template <int MS, int NT, int UW, int KW, int D, bool GROUPED>
void launch_tile_t(const TileShape& t, const Layout& L, const uint16_t* x, int64_t ld_x, BlobView bv, const float* gs,
                   int g_div, uint16_t* y, int64_t ld_y, int64_t rows, const int32_t* offsets, SplitK sk,
                   hipStream_t st, bool f16, const int32_t* row_index) {
    const dim3 grid((unsigned)t.groups, (unsigned)t.mtiles, (unsigned)t.S);
    const bool kfull = L.K % kChunkK == 0;
#define NVFP4_TILE_LAUNCH(KF, F16)                                                                                 \
    hipLaunchKernelGGL((k_gemm_tile<MS, NT, UW, KW, D, GROUPED, KF, F16>), grid, dim3(UW * KW * 64), 0, st, x, ld_x, \
                       bv, (int)L.NU, (int)L.KC, (int)L.K, (int)L.N, gs, g_div, y, ld_y, rows, offsets, (int)L.E, sk,  \
                       row_index)
    if (f16) {
        if (kfull) NVFP4_TILE_LAUNCH(true, true);
        else NVFP4_TILE_LAUNCH(false, true);
    } else {
        if (kfull) NVFP4_TILE_LAUNCH(true, false);
        else NVFP4_TILE_LAUNCH(false, false);
    }
#undef NVFP4_TILE_LAUNCH
}

template <bool GROUPED>
nvfp4_status launch_tile(const TileShape& t, const Layout& L, const uint16_t* x, int64_t ld_x, const uint8_t* blob,
                         const float* gs, int g_div, uint16_t* y, int64_t ld_y, int64_t rows, const int32_t* offsets,
                         uint8_t* ws, const Workspace& wl, hipStream_t st, bool f16,
                         const int32_t* row_index = nullptr) {
    if (t.mtiles > 65535) return fail(NVFP4_ERR_INVALID_ARG, "tile GEMM: %lld row tiles exceed the grid limit", (long long)t.mtiles);
    const SplitK sk = split_k(t.S, ws, wl);
    const BlobView bv = make_view(L, blob);
#define NVFP4_TILE(MS, NT, UW, KW, D) \
    launch_tile_t<MS, NT, UW, KW, D, GROUPED>(t, L, x, ld_x, bv, gs, g_div, y, ld_y, rows, offsets, sk, st, f16, row_index)
    if constexpr (GROUPED) {
        NVFP4_TILE(4, 4, 4, 1, 2);
    } else {
        if (t.ms == 1) NVFP4_TILE(1, 1, 4, 4, 2);
        else if (t.ms == 2) NVFP4_TILE(2, 1, 4, 2, 4);
        else if (t.ms == 4 && t.kw == 1) NVFP4_TILE(4, 4, 8, 1, 3);
        else if (t.ms == 4) NVFP4_TILE(4, 1, 4, 4, 2);
        else NVFP4_TILE(8, 2, 8, 1, 2);
    }
#undef NVFP4_TILE
    return launched("tile GEMM");
}

// ------------------------------------------------ activation-resident path --
// (ch, u, w, d): chunks per wave, units per workgroup, waves, ring depth.
// From launch sweeps on MI355X (graph-replayed, weights rotated past the
// Infinity Cache): 16 waves with a 2-deep ring for K up to 4096, the
// workgroup count near the CU count (u = ceil(row units / 256)).
#define NVFP4_XRES_CONFIGS(X) \
    X(1, 1, 16, 2) X(1, 2, 16, 2) X(1, 3, 16, 2) X(1, 4, 16, 2) X(1, 5, 16, 2) X(1, 6, 16, 2) X(1, 7, 16, 2) \
    X(1, 8, 16, 2) X(2, 1, 16, 2) X(2, 2, 16, 2) X(2, 3, 16, 2) X(2, 4, 16, 2) X(2, 5, 16, 2) X(2, 6, 16, 2) \
    X(2, 7, 16, 2) X(2, 8, 16, 2)

// Rows from which the automatic choice takes the activation-resident kernel
// (below it the small-M kernel, measured faster at one row).
constexpr int64_t kXresAutoMin = 5;
constexpr int kXresMaxSplits = 8;
constexpr int kXresMaxK = kXresMaxSplits * 2 * 16 * kChunkK;   // two chunks for each of 16 waves, per split
constexpr int kXresMaxN = 8 * 256 * kUnitN;   // eight units for each of 256 workgroups

struct XresShape {
    int ch, u, w, d, S;
    int64_t groups;
};

bool xres_compiled(const XresShape& s) {
    bool found = false;
#define NVFP4_XRES_FIND(CH, U, W, D) found = found || (s.ch == CH && s.u == U && s.w == W && s.d == D);
    NVFP4_XRES_CONFIGS(NVFP4_XRES_FIND)
#undef NVFP4_XRES_FIND
    return found;
}

// 16 waves own one or two chunks each; K beyond 32 chunks is split S ways
// across workgroups; units per workgroup by N and S, so that the grid is
// about one workgroup per CU.  A shape outside the compiled set means the
// kernel does not take the call (K above 8 splits, or too many row units).
XresShape xres_shape(const Layout& L) {
    XresShape s{L.KC <= 16 ? 1 : 2, 0, 16, 2, 1, 0};
    s.S = (int)((L.KC + 31) / 32);
    const int64_t u = (L.NU * s.S + 255) / 256;
    s.u = (int)(u < 1 ? 1 : u > 64 ? 64 : u);
    s.groups = (L.NU + s.u - 1) / s.u;
    return s;
}

// Does the activation-resident kernel take this dense call?
bool xres_fits(const Layout& L, int64_t rows) {
    const XresShape s = xres_shape(L);
    return rows <= kSmallRows && s.S <= kXresMaxSplits && (int64_t)s.S * s.w * s.ch >= L.KC && xres_compiled(s) &&
           s.groups <= 65535;
}

Workspace workspace_for(const XresShape& s, int64_t rows, int64_t K, bool pre) {
    return workspace_layout(s.S, s.groups, (int64_t)s.u * 256, rows, K, pre);
}

nvfp4_status launch_xres(const XresShape& s, const Layout& L, const uint16_t* x, int64_t ld_x, const uint8_t* blob,
                         const float* gs, int g_div, uint16_t* y, int64_t ld_y, int64_t rows, SplitK sk,
                         hipStream_t st, bool f16) {
    const BlobView bv = make_view(L, blob);
    const dim3 grid((unsigned)s.groups, (unsigned)s.S);
    bool done = false;
#define NVFP4_XRES_LAUNCH(CH, U, W, D, FULL, F16)                                                               \
    hipLaunchKernelGGL((k_gemm_xres<CH, U, W, D, FULL, F16>), grid, dim3(W * 64), 0, st, x, ld_x, bv, (int)L.NU, \
                       (int)L.KC, (int)L.K, (int)L.N, gs, g_div, y, ld_y, (int)rows, sk)
#define NVFP4_XRES_DISPATCH(CH, U, W, D)                                                                          \
    if (!done && s.ch == CH && s.u == U && s.w == W && s.d == D) {                                               \
        const bool full = L.K == (int64_t)s.S * CH * W * kChunkK;                                               \
        if (f16 && full) NVFP4_XRES_LAUNCH(CH, U, W, D, true, true);                                            \
        else if (f16) NVFP4_XRES_LAUNCH(CH, U, W, D, false, true);                                              \
        else if (full) NVFP4_XRES_LAUNCH(CH, U, W, D, true, false);                                             \
        else NVFP4_XRES_LAUNCH(CH, U, W, D, false, false);                                                      \
        done = true;                                                                                             \
    }
    NVFP4_XRES_CONFIGS(NVFP4_XRES_DISPATCH)
#undef NVFP4_XRES_DISPATCH
#undef NVFP4_XRES_LAUNCH
    if (!done) return fail(NVFP4_ERR_INVALID_ARG, "activation-resident GEMM: no compiled kernel for this shape");
    return launched("activation-resident GEMM");
}

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
nvfp4_status check_gemm_io(const char* fn, const void* x, int64_t ld_x, const void* pre, const void* w,
                           const void* gs, const void* y, int64_t ld_y, int64_t rows, int64_t N, int64_t K,
                           const void* ws, int64_t ws_bytes, int64_t ws_need) {
    if (rows < 0) return fail(NVFP4_ERR_INVALID_ARG, "%s: row count %lld is negative", fn, (long long)rows);
    if (ld_x < K) return fail(NVFP4_ERR_INVALID_ARG, "%s: ld_x = %lld < K = %lld", fn, (long long)ld_x, (long long)K);
    if (ld_y < N) return fail(NVFP4_ERR_INVALID_ARG, "%s: ld_y = %lld < N = %lld", fn, (long long)ld_y, (long long)N);
    if (!w) return fail(NVFP4_ERR_INVALID_ARG, "%s: w_repacked is NULL", fn);
    if (!gs) return fail(NVFP4_ERR_INVALID_ARG, "%s: global scale pointer is NULL", fn);
    if (rows > 0 && !x) return fail(NVFP4_ERR_INVALID_ARG, "%s: x is NULL", fn);
    if (rows > 0 && !y) return fail(NVFP4_ERR_INVALID_ARG, "%s: y is NULL", fn);
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

// Pre-quant scale: X' = RNE_bf16(X * s) into the workspace; returns the
// activation the GEMM kernel reads.
nvfp4_status apply_prescale(const void* x, int64_t& ld_x, const void* pre, int64_t rows, int64_t K, void* ws,
                            const uint16_t*& xp, hipStream_t st, bool f16) {
    xp = static_cast<const uint16_t*>(x);
    if (!pre) return NVFP4_OK;
    const int64_t threads = rows * (K / 8);
    if (f16)
        hipLaunchKernelGGL(k_prescale<true>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                           static_cast<const uint16_t*>(x), ld_x, static_cast<const uint16_t*>(pre), rows, K,
                           static_cast<uint16_t*>(ws), K);
    else
        hipLaunchKernelGGL(k_prescale<false>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                           static_cast<const uint16_t*>(x), ld_x, static_cast<const uint16_t*>(pre), rows, K,
                           static_cast<uint16_t*>(ws), K);
    const nvfp4_status s = launched("pre-quant scale");
    if (s != NVFP4_OK) return s;
    xp = static_cast<const uint16_t*>(ws);
    ld_x = K;
    return NVFP4_OK;
}

// Workspace bytes of a dense call: enough for either kernel, with or without a pre-scale.
int64_t dense_workspace_bytes(const Layout& L, int64_t M) {
    int64_t need = workspace_for(tile_shape(L, M, false), M, L.K, true).total;
    if (M <= kSmallRows) {
        const int64_t small = workspace_for(small_m_shape(L, M, false), M, L.K, true).total;
        need = small > need ? small : need;
        const int64_t xres = workspace_for(xres_shape(L), M, L.K, true).total;
        need = xres > need ? xres : need;
    }
    return need;
}

nvfp4_status dense_gemm(const void* x, int64_t ld_x, const void* pre, const void* w, const float* gs, int g_div,
                        void* y, int64_t ld_y, int64_t M, int64_t N, int64_t K, void* ws, int64_t ws_bytes,
                        int variant, void* stream, const char* fn, bool f16) {
    nvfp4_status s = check_weight_shape(fn, 1, N, K);
    if (s != NVFP4_OK) return s;
    if (variant < kAuto || variant > kResident) return fail(NVFP4_ERR_INVALID_ARG, "%s: unknown variant %d", fn, variant);
    if (variant == kSmall && M > kSmallRows)
        return fail(NVFP4_ERR_INVALID_ARG, "%s: the small-M variant takes M <= %d (M = %lld)", fn, kSmallRows, (long long)M);
    if (M > (int64_t)1 << 31) return fail(NVFP4_ERR_INVALID_ARG, "%s: M = %lld too large", fn, (long long)M);
    const Layout L = make_layout(1, N, K);
    const TileShape t = tile_shape(L, M, false);
    const SmallShape sm = small_m_shape(L, M, false);
    if (variant == kResident && !xres_fits(L, M))
        return fail(NVFP4_ERR_INVALID_ARG,
                    "%s: the activation-resident variant takes M <= %d, K <= %d and N <= %d (M = %lld, N = %lld, K = %lld)",
                    fn, kSmallRows, kXresMaxK, kXresMaxN, (long long)M, (long long)N, (long long)K);
    const bool resident =
        variant == kResident || (variant == kAuto && M >= kXresAutoMin && xres_fits(L, M));
    const XresShape xs = xres_shape(L);
    const bool small = variant == kSmall || (variant == kAuto && !resident && M <= kSmallAuto);
    // the MFMA-bound kernel addresses the code and scale regions with 32-bit offsets
    const bool mfma_fits = L.code_bytes() < ((int64_t)1 << 31);
    if (variant == kMfma && !mfma_fits)
        return fail(NVFP4_ERR_INVALID_ARG, "%s: the MFMA-bound variant takes weights below 2 GiB of codes", fn);
    const bool mfma = variant == kMfma ||
                      (variant == kAuto && mfma_fits && M >= kMfmaAuto && mfma_plan(L, M).tiles >= kMfmaMinTiles);
    const Workspace wl = resident ? workspace_for(xs, M, K, pre != nullptr)
                         : small  ? workspace_for(sm, M, K, pre != nullptr)
                         : mfma ? workspace_layout(1, 0, 0, M, K, pre != nullptr)
                                : workspace_for(t, M, K, pre != nullptr);
    s = check_gemm_io(fn, x, ld_x, pre, w, gs, y, ld_y, M, N, K, ws, ws_bytes, wl.total);
    if (s != NVFP4_OK) return s;
    if (M == 0) return ok();   // zero rows: nothing is launched
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t* wsb = static_cast<uint8_t*>(ws);
    const uint16_t* xp;
    s = apply_prescale(x, ld_x, pre, M, K, pre ? wsb + wl.prescale : nullptr, xp, st, f16);
    if (s != NVFP4_OK) return s;
    const uint8_t* blob = static_cast<const uint8_t*>(w);
    uint16_t* yo = static_cast<uint16_t*>(y);
    if (resident) return launch_xres(xs, L, xp, ld_x, blob, gs, g_div, yo, ld_y, M, split_k(xs.S, wsb, wl), st, f16);
    if (small)
        return launch_small<false>(sm, L, xp, ld_x, blob, gs, g_div, yo, ld_y, M, nullptr, split_k(sm.S, wsb, wl), st,
                                   f16);
    if (mfma) {
        const hipError_t e = launch_gemm_mfma(mfma_plan(L, M), L, xp, ld_x, blob, gs, g_div, yo, ld_y, M, st, f16);
        if (e != hipSuccess) return fail(NVFP4_ERR_HIP, "%s: MFMA GEMM launch failed: %s", fn, hipGetErrorString(e));
        return ok();
    }
    return launch_tile<false>(t, L, xp, ld_x, blob, gs, g_div, yo, ld_y, M, nullptr, wsb, wl, st, f16);
}

// Grouped GEMM, shared by the plain and the gathering entry points: the
// activation has x_rows rows; grouped row r reads row row_index[r] of it
// (row r itself when row_index is NULL).
nvfp4_status grouped_gemm(const char* fn, const void* x, int64_t ld_x, int64_t x_rows, const int32_t* row_index,
                          const int32_t* expert_offsets, const void* pre_scale, const void* w_repacked,
                          const float* global_scales, int global_scale_is_divisor, void* y, int64_t ld_y, int64_t R,
                          int64_t E, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes, void* stream,
                          bool f16) {
    nvfp4_status s = check_weight_shape(fn, E, N, K);
    if (s != NVFP4_OK) return s;
    const Workspace wl = workspace_layout(1, 0, 0, x_rows, K, pre_scale != nullptr);
    s = check_gemm_io(fn, x, ld_x, pre_scale, w_repacked, global_scales, y, ld_y, R, N, K, workspace, workspace_bytes,
                      wl.total);
    if (s != NVFP4_OK) return s;
    if (!expert_offsets) return fail(NVFP4_ERR_INVALID_ARG, "%s: expert_offsets is NULL", fn);
    if (!aligned(expert_offsets, 4)) return fail(NVFP4_ERR_ALIGNMENT, "%s: expert_offsets must be 4-byte aligned", fn);
    if (R > (int64_t)1 << 31) return fail(NVFP4_ERR_INVALID_ARG, "%s: R = %lld exceeds int32 offsets", fn, (long long)R);
    if (R == 0) return ok();   // zero rows: nothing is launched
    const Layout L = make_layout(E, N, K);
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t* wsb = static_cast<uint8_t*>(workspace);
    const uint16_t* xp;
    s = apply_prescale(x, ld_x, pre_scale, x_rows, K, pre_scale ? wsb + wl.prescale : nullptr, xp, st, f16);
    if (s != NVFP4_OK) return s;
    const uint8_t* blob = static_cast<const uint8_t*>(w_repacked);
    uint16_t* yo = static_cast<uint16_t*>(y);
    const int g_div = global_scale_is_divisor != 0;
    // Few rows per expert on average: the weight stream dominates, use the small-M kernel (passes of 16 rows).
    if (R <= (int64_t)kSmallRows * E)
        return launch_small<true>(small_m_shape(L, R, true), L, xp, ld_x, blob, global_scales, g_div, yo, ld_y, 0,
                                  expert_offsets, split_k(1, wsb, wl), st, f16, row_index);
    const TileShape t = tile_shape(L, R, true);
    return launch_tile<true>(t, L, xp, ld_x, blob, global_scales, g_div, yo, ld_y, R, expert_offsets, wsb, wl, st,
                             f16, row_index);
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

nvfp4_status nvfp4_repack(const uint8_t* w_packed, int64_t ld_w, const uint8_t* w_scale, int64_t ld_s, int64_t E,
                          int64_t N, int64_t K, void* out, int64_t out_bytes, void* stream) {
    const char* fn = "nvfp4_repack";
    nvfp4_status s = check_weight_shape(fn, E, N, K);
    if (s != NVFP4_OK) return s;
    if (!w_packed) return fail(NVFP4_ERR_INVALID_ARG, "%s: w_packed is NULL", fn);
    if (!w_scale) return fail(NVFP4_ERR_INVALID_ARG, "%s: w_scale is NULL", fn);
    if (!out) return fail(NVFP4_ERR_INVALID_ARG, "%s: out is NULL", fn);
    if (ld_w < K / 2) return fail(NVFP4_ERR_INVALID_ARG, "%s: ld_w = %lld < K/2 = %lld", fn, (long long)ld_w, (long long)(K / 2));
    if (ld_s < K / 16) return fail(NVFP4_ERR_INVALID_ARG, "%s: ld_s = %lld < K/16 = %lld", fn, (long long)ld_s, (long long)(K / 16));
    if (!aligned(out, 16)) return fail(NVFP4_ERR_ALIGNMENT, "%s: out must be 16-byte aligned", fn);
    const Layout L = make_layout(E, N, K);
    if (out_bytes < L.total_bytes())
        return fail(NVFP4_ERR_BUFFER_TOO_SMALL, "%s: out_bytes = %lld < %lld", fn, (long long)out_bytes, (long long)L.total_bytes());
    const int64_t lanes = L.blocks() * 64;
    uint8_t* o = static_cast<uint8_t*>(out);
    hipLaunchKernelGGL(k_repack, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, static_cast<hipStream_t>(stream),
                       w_packed, ld_w, w_scale, ld_s, N, K, L.NU, L.KC, lanes, make_view(L, o), o, o + L.code_bytes());
    return launched(fn);
}

nvfp4_status nvfp4_dequant_bf16(const void* w_repacked, int64_t E, int64_t N, int64_t K, void* out, int64_t ld_out,
                                void* stream) {
    const char* fn = "nvfp4_dequant_bf16";
    nvfp4_status s = check_weight_shape(fn, E, N, K);
    if (s != NVFP4_OK) return s;
    if (!w_repacked || !out) return fail(NVFP4_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (ld_out < K) return fail(NVFP4_ERR_INVALID_ARG, "%s: ld_out = %lld < K", fn, (long long)ld_out);
    if (!aligned(w_repacked, 16) || !aligned(out, 2)) return fail(NVFP4_ERR_ALIGNMENT, "%s: misaligned pointer", fn);
    const Layout L = make_layout(E, N, K);
    const int64_t lanes = L.blocks() * 64;
    const uint8_t* b = static_cast<const uint8_t*>(w_repacked);
    hipLaunchKernelGGL(k_dequant, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, static_cast<hipStream_t>(stream),
                       make_view(L, b), N, K, L.NU, L.KC, lanes, static_cast<uint16_t*>(out), ld_out);
    return launched(fn);
}

int64_t nvfp4_w4a16_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || check_weight_shape("nvfp4_w4a16_gemm_workspace_bytes", 1, N, K) != NVFP4_OK) return -1;
    return dense_workspace_bytes(make_layout(1, N, K), M);
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
    return workspace_layout(1, 0, 0, R, K, true).total;   // the grouped kernels never split K
}

nvfp4_status nvfp4_w4a16_grouped_gemm(const void* x, int64_t ld_x, const int32_t* expert_offsets, const void* pre_scale,
                                      const void* w_repacked, const float* global_scales, int global_scale_is_divisor,
                                      void* y, int64_t ld_y, int64_t R, int64_t E, int64_t N, int64_t K,
                                      void* workspace, int64_t workspace_bytes, void* stream) {
    return grouped_gemm("nvfp4_w4a16_grouped_gemm", x, ld_x, R, nullptr, expert_offsets, pre_scale, w_repacked,
                        global_scales, global_scale_is_divisor, y, ld_y, R, E, N, K, workspace, workspace_bytes, stream,
                        false);
}

nvfp4_status nvfp4_w4a16_grouped_gemm_f16(const void* x, int64_t ld_x, const int32_t* expert_offsets,
                                          const void* pre_scale, const void* w_repacked, const float* global_scales,
                                          int global_scale_is_divisor, void* y, int64_t ld_y, int64_t R, int64_t E,
                                          int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                                          void* stream) {
    return grouped_gemm("nvfp4_w4a16_grouped_gemm_f16", x, ld_x, R, nullptr, expert_offsets, pre_scale, w_repacked,
                        global_scales, global_scale_is_divisor, y, ld_y, R, E, N, K, workspace, workspace_bytes, stream,
                        true);
}

int64_t nvfp4_w4a16_grouped_gemm_gather_workspace_bytes(int64_t T, int64_t R, int64_t E, int64_t N, int64_t K) {
    if (T < 0 || R < 0 || check_weight_shape("nvfp4_w4a16_grouped_gemm_gather_workspace_bytes", E, N, K) != NVFP4_OK)
        return -1;
    return workspace_layout(1, 0, 0, T, K, true).total;   // the pre-scaled token rows
}

static nvfp4_status grouped_gemm_gather(const char* fn, const void* x, int64_t ld_x, int64_t T,
                                        const int32_t* row_token, const int32_t* expert_offsets,
                                        const void* pre_scale, const void* w_repacked, const float* global_scales,
                                        int global_scale_is_divisor, void* y, int64_t ld_y, int64_t R, int64_t E,
                                        int64_t N, int64_t K, void* workspace, int64_t workspace_bytes, void* stream,
                                        bool f16) {
    if (T < 0) return fail(NVFP4_ERR_INVALID_ARG, "%s: token count %lld is negative", fn, (long long)T);
    if (R > 0 && !row_token) return fail(NVFP4_ERR_INVALID_ARG, "%s: row_token is NULL", fn);
    if (!aligned(row_token, 4)) return fail(NVFP4_ERR_ALIGNMENT, "%s: row_token must be 4-byte aligned", fn);
    if (R > 0 && T == 0) return fail(NVFP4_ERR_INVALID_ARG, "%s: %lld rows gather from 0 tokens", fn, (long long)R);
    // the kernels address a gathered row with a 32-bit byte offset from x
    if (T * ld_x >= ((int64_t)1 << 31))
        return fail(NVFP4_ERR_INVALID_ARG, "%s: T * ld_x = %lld must stay below 2^31", fn, (long long)(T * ld_x));
    return grouped_gemm(fn, x, ld_x, T, row_token, expert_offsets, pre_scale, w_repacked, global_scales,
                        global_scale_is_divisor, y, ld_y, R, E, N, K, workspace, workspace_bytes, stream, f16);
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
    hipLaunchKernelGGL(k_moe_route_scan, dim3(1), dim3(kRouteThreads), 0, st, hist, blocks, (int)E, P, expert_offsets);
    hipLaunchKernelGGL(k_moe_route_place, dim3((unsigned)blocks), dim3(kRouteThreads), 0, st, topk_ids, P, (int)E,
                       hist, row_token, token_row, (int)k, expert_offsets);
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
