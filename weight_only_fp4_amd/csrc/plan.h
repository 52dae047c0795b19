// Host-side planning shared by the library's translation units: the launch
// shape of each GEMM kernel family (pure functions of the call's sizes, so
// the workspace queries reproduce them), the arguments every GEMM launch
// takes, and the launchers that each family's translation units define
// (one unit per kernel family and activation type, compiled in parallel).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/nvfp4_w4a16.h"
#include "kernels_gemm.h"
#include "layout.h"

namespace nvfp4 {

// Error reporting (nvfp4_w4a16.hip): the message of the last failed call on
// this thread, returned by nvfp4_last_error().
nvfp4_status fail(nvfp4_status st, const char* fmt, ...);
nvfp4_status ok();
nvfp4_status launched(const char* what);   // HIP status of the last launch

inline int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// Everything a GEMM launch needs besides its shape.  rows: dense row count
// (unused by the grouped forms, which read expert_offsets on the device).
struct GemmArgs {
    const uint16_t* x;
    int64_t ld_x;
    const uint8_t* blob;
    const float* gs;
    int g_div;
    uint16_t* y;
    int64_t ld_y;
    int64_t rows;
    const int32_t* offsets;     // grouped forms: expert_offsets [E + 1]
    const int32_t* row_index;   // grouped forms: row r reads activation row row_index[r] (or NULL)
    const uint16_t* pre;        // pre-quant scale [K] or NULL
    SplitK sk;
    hipStream_t st;
    int act = kActNone;         // grouped forms: the MoE activation of the epilogue (decode.h)
};

// ---------------------------------------------------------------- small-M --
// Small-M launch shape: row form mg (1, 2: 4x4x4 with that many row groups;
// 16: 16x16x32), nt units per wave, w waves per workgroup, ring depth d, and
// K splits S across workgroups (dense only).  Only the (mg, nt, w, d) tuples
// listed in NVFP4_SMALL_CONFIGS are compiled.
struct SmallShape {
    int mg, nt, w, d, S;
    int64_t groups;   // workgroups along N (units / nt)
};

// (mg, nt, w, d) for the dense form, exactly the shapes small_m_shape picks;
// the grouped form is always (0, 1, w, 4).
#define NVFP4_SMALL_CONFIGS(X) \
    X(1, 1, 1, 4) X(1, 1, 2, 4) X(1, 1, 4, 4) X(1, 1, 8, 4) X(1, 1, 16, 4) X(1, 2, 1, 4) \
    X(2, 1, 1, 4) X(2, 1, 2, 4) X(2, 1, 4, 4) X(2, 1, 8, 4) X(2, 2, 1, 4) \
    X(16, 4, 4, 2)

// Is (mg, nt, w, d) one of the compiled dense shapes?
inline bool small_compiled(const SmallShape& s) {
    bool found = false;
#define NVFP4_SMALL_FIND(MG, NT, W, D) found = found || (s.mg == MG && s.nt == NT && s.w == W && s.d == D);
    NVFP4_SMALL_CONFIGS(NVFP4_SMALL_FIND)
#undef NVFP4_SMALL_FIND
    return found;
}

// Shapes from launch sweeps on MI355X (graph-replayed, weights rotated past
// the Infinity Cache).  Rows <= 8: one unit per wave, waves sized so the
// workgroups x waves x ring depth product aims at about 32 KB of weight
// loads in flight per CU; from 2048 row units on (N >= 32768, LM heads) two
// units per wave and one wave per workgroup, which shares each activation
// piece, and its pre-quant scaling, over two units (N = 131072, K = 4096:
// 47.8 us with a pre-scale and 45-47 without, against 56.9 / 45.1 us with one
// unit and two waves at M = 1, 46.6 against 54.8 us at M = 4).  Rows 9..16
// (16x16x32 form, about two VALU operations per weight to decode) share each
// activation fragment over four units per wave; the automatic choice sends
// those rows to the activation-resident kernel.
inline SmallShape small_m_shape(const Layout& L, int64_t rows, bool grouped, int act = kActNone) {
    SmallShape s;
    s.S = 1;
    if (grouped) {
        // the gated epilogue needs each gate / up unit pair in one workgroup.
        // At most one row per expert on average (decode-sized MoE batches):
        // the 4-row form, in passes of 4 rows, whose lower register count
        // fits more waves per SIMD (MoE T = 16, E = 128, top-8: FC1 25.3 us
        // against 27.8, FC2 14.0 against 15.2 with a 6-deep ring); with more
        // rows the dynamic form (4 or 16 rows per pass), since an expert of
        // many rows would take one pass per 4 of them (T = 64: FC1 81.7 us
        // against 57.5)
        s.nt = act == kActSiluGlu ? 2 : 1;
        s.mg = rows <= L.E ? 1 : 0;
        s.d = s.mg == 1 && s.nt == 1 ? 6 : 4;
    } else if (rows <= 8) {
        s.mg = rows <= 4 ? 1 : 2; s.nt = L.NU >= 2048 ? 2 : 1; s.d = 4;
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
    s.w = 1;
    if (!grouped && s.nt == 2) return s;   // wide N: one wave per workgroup
    // grouped: sized by units and a ring depth of 4 whatever the form's, so
    // that the paired (gated) form splits K over the same waves as the plain
    // form and sums in the same order; at most 8 waves (the grouped launchers)
    const int64_t ctas = grouped ? L.NU * ((L.E + 1) / 2) : s.groups;
    const int dw = grouped ? 4 : s.d;
    // 16 waves cap a kernel at 128 VGPRs: only the one-row-group form fits
    const int wmax = s.mg == 1 && !grouped ? 16 : 8;
    while (s.w < wmax && ctas * (2 * s.w) * dw <= 8192 && L.KC >= 4 * (2 * s.w)) s.w *= 2;
    if (s.w < 2 && L.KC >= 8) s.w = 2;
    while (!grouped && s.w > 1 && !small_compiled(s)) s.w /= 2;
    return s;
}

// ------------------------------------------------------------------- tile --
// Tile shapes by row count, from launch-shape sweeps on MI355X: the fastest
// decode-sized shapes run about one 16-wave workgroup per CU, four unit-waves
// times four k-parts.  K is further split across workgroups (grid z) while
// the workgroup count stays at or below 256 and every wave keeps >= 2
// chunks.
struct TileShape {
    int ms, nt, uw, kw, d, S;
    int64_t groups, mtiles;
    int64_t tiles() const { return groups * mtiles; }
    int bm() const { return 16 * ms; }
    int ug() const { return nt * uw; }
};

inline TileShape tile_shape(const Layout& L, int64_t rows, bool grouped) {
    TileShape t;
    bool split = true;
    if (grouped) {
        t.ms = 4; t.nt = 4; t.uw = 4; t.kw = 1; t.d = 3; split = false;
    } else if (rows <= 16) {
        t.ms = 1; t.nt = 1; t.uw = 4; t.kw = 4; t.d = 2;
    } else if (rows <= 32) {
        t.ms = 2; t.nt = 1; t.uw = 4; t.kw = 2; t.d = 4;
    } else if (rows <= 192) {
        // 64-row tiles: up to three row tiles still beat 128-row tiles here
        // (measured); wide N (LM heads) takes 512 columns per workgroup with
        // a 4-deep weight ring (M = 64, N = 131072, K = 4096: 95.6 us against
        // 103.5 with 3 deep and 139 with 5)
        if (L.NU >= 4096) { t.ms = 4; t.nt = 4; t.uw = 8; t.kw = 1; t.d = 4; }
        else { t.ms = 4; t.nt = 1; t.uw = 4; t.kw = 4; t.d = 2; }
    } else {
        t.ms = 8; t.nt = 2; t.uw = 8; t.kw = 1; t.d = 2;
    }
    t.groups = (L.NU + t.ug() - 1) / t.ug();
    // grouped: row tiles are at most rows / BM + E; the kernel deals (row
    // tile, column group) items to the XCDs in ranges of ceil(items / 8) and
    // needs 8 workgroups beyond the item count for that
    t.mtiles = (rows + t.bm() - 1) / t.bm() + (grouped ? L.E + (8 + t.groups - 1) / t.groups : 0);
    t.S = 1;
    while (split && t.S < 16 && t.tiles() * 2 * t.S <= 256 && L.KC >= 2 * t.kw * (2 * t.S)) t.S *= 2;
    return t;
}

// ---------------------------------------------------- activation-resident --
// (ch, u, w, d): chunks per wave, units per workgroup, waves, ring depth.
// From launch sweeps on MI355X (graph-replayed, weights rotated past the
// Infinity Cache; decode M = 16 / M = 8, K = 4096, N = 14336): 9..16 rows take
// 16 waves with a 6-deep ring (9.5 us, against 10.1 with a 2-deep ring), up to
// 8 rows 8 waves of twice the chunks with a 4-deep ring (8.7 us, against
// 10.0 with 16 waves), where half the activation rows leave room for it; the
// workgroup count near the CU count (u = ceil(row units x splits / 256)).
#define NVFP4_XRES_U(X, CH, W, D) \
    X(CH, 1, W, D) X(CH, 2, W, D) X(CH, 3, W, D) X(CH, 4, W, D) X(CH, 5, W, D) X(CH, 6, W, D) X(CH, 7, W, D) X(CH, 8, W, D)
#define NVFP4_XRES_CONFIGS(X) \
    NVFP4_XRES_U(X, 1, 16, 6) NVFP4_XRES_U(X, 2, 16, 6) NVFP4_XRES_U(X, 2, 8, 4) NVFP4_XRES_U(X, 4, 8, 4)

// Rows from which the automatic choice takes the activation-resident kernel
// (below it the small-M kernel, measured faster at one row).
constexpr int64_t kXresAutoMin = 5;
constexpr int kXresMaxSplits = 8;

struct XresShape {
    int ch, u, w, d, S;
    int64_t groups;
};

inline bool xres_compiled(const XresShape& s) {
    bool found = false;
#define NVFP4_XRES_FIND(CH, U, W, D) found = found || (s.ch == CH && s.u == U && s.w == W && s.d == D);
    NVFP4_XRES_CONFIGS(NVFP4_XRES_FIND)
#undef NVFP4_XRES_FIND
    return found;
}

// A workgroup's waves own ch chunks each (32 chunks in all, 16 when K fits
// 16 chunks); K beyond that is split S ways across workgroups; units per
// workgroup by N and S, so that the grid is about one workgroup per CU.  A
// shape outside the compiled set means the kernel does not take the call (K
// above 8 splits, or too many row units).
inline XresShape xres_shape(const Layout& L, int64_t rows) {
    const bool eight = rows <= 8;
    XresShape s{0, 0, eight ? 8 : 16, eight ? 4 : 6, 1, 0};
    s.ch = (L.KC <= 16 ? 16 : 32) / s.w;
    s.S = (int)((L.KC + 31) / 32);
    const int64_t u = (L.NU * s.S + 255) / 256;
    s.u = (int)(u < 1 ? 1 : u > 64 ? 64 : u);
    s.groups = (L.NU + s.u - 1) / s.u;
    return s;
}

// Does the activation-resident kernel take this dense call?  (M <= 16,
// K <= 32768, and ceil(N / 16) * ceil(K / 4096) <= 2048.)
inline bool xres_fits(const Layout& L, int64_t rows) {
    const XresShape s = xres_shape(L, rows);
    return rows <= kSmallRows && s.S <= kXresMaxSplits && (int64_t)s.S * s.w * s.ch >= L.KC && xres_compiled(s) &&
           s.groups <= 65535;
}

// -------------------------------------------------------------- workspace --
// Byte offsets in the caller's workspace: split-K arrival counters, then
// split-K partials.  The counters take a fixed prefix of kMaxSplitTiles
// entries, whatever the call, so that no call's partials overlap any call's
// counters: every call leaves the counters it used at zero, so a workspace
// (zero-filled once) can serve calls of any shapes one after another.  A
// call without a K split needs no workspace.
constexpr int64_t kMaxSplitTiles = 1024;

struct Workspace {
    int64_t counters, partials, total;
};

// split_tiles tiles of tile_floats fp32 each, S splits (no split-K area when
// S == 1).  The planners split only grids of at most a few hundred tiles.
inline Workspace workspace_layout(int S, int64_t split_tiles, int64_t tile_floats) {
    Workspace w{0, 0, 0};
    if (S > 1) {
        w.counters = 0;
        w.partials = kMaxSplitTiles * 4;
        w.total = w.partials + round_up((int64_t)S * split_tiles * tile_floats * 4, 256);
    }
    return w;
}

inline Workspace workspace_for(const TileShape& t) {
    return workspace_layout(t.S, t.tiles(), (int64_t)t.bm() * t.ug() * 16);
}
inline Workspace workspace_for(const SmallShape& s) {
    return workspace_layout(s.S, s.groups, (int64_t)kSmallRows * 16 * s.nt);
}
inline Workspace workspace_for(const XresShape& s) { return workspace_layout(s.S, s.groups, (int64_t)s.u * 256); }

inline SplitK split_k(int S, uint8_t* ws, const Workspace& wl) {
    return SplitK{S, S > 1 ? reinterpret_cast<float*>(ws + wl.partials) : nullptr,
                  S > 1 ? reinterpret_cast<int*>(ws + wl.counters) : nullptr};
}

// ---------------------------------------------------------------- launchers --
// One translation unit per family and activation type (F16) defines each;
// the activation-resident family has one per scale format (MX) too.  The
// small-M family reads its scales through a table in LDS built for the
// blob's format, and the tile launcher picks the kernel compiled for it, so
// both take the format at run time.
template <bool F16>
nvfp4_status launch_small(const SmallShape& s, const Layout& L, const GemmArgs& a, bool grouped);
template <bool F16>
nvfp4_status launch_tile(const TileShape& t, const Layout& L, const GemmArgs& a, bool grouped);
template <bool F16, bool MX>
nvfp4_status launch_xres(const XresShape& s, const Layout& L, const GemmArgs& a);

}  // namespace nvfp4
