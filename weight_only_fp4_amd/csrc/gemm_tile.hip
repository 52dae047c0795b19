// Launchers of the tile kernel family (kernels_tile.h) for one activation
// type: this unit is compiled once per type, with NVFP4_ACT_F16 = 0 (bf16)
// and 1 (fp16).
#include "kernels_tile.h"
#include "plan.h"

#ifndef NVFP4_ACT_F16
#error "compile with -DNVFP4_ACT_F16=0 (bf16) or -DNVFP4_ACT_F16=1 (fp16)"
#endif

namespace nvfp4 {

namespace {

constexpr bool kF16 = NVFP4_ACT_F16 != 0;

template <int MS, int NT, int UW, int KW, int D, bool GROUPED, int ACT = kActNone>
void launch_tile_t(const TileShape& t, const Layout& L, const GemmArgs& a) {
    const BlobView bv = make_view(L, a.blob);
    const dim3 grid((unsigned)t.groups, (unsigned)t.mtiles, (unsigned)t.S);
    const int64_t rows = GROUPED ? 0 : a.rows;
#define NVFP4_TILE_LAUNCH(KF, PRE, MX)                                                                                  \
    hipLaunchKernelGGL((k_gemm_tile<MS, NT, UW, KW, D, GROUPED, KF, kF16, PRE, ACT, MX>), grid, dim3(UW * KW * 64), 0, \
                       a.st, a.x, a.ld_x, bv, (int)L.NU, (int)L.KC, (int)L.K, (int)L.N, a.gs, a.g_div, a.y, a.ld_y, rows,  \
                       a.offsets, (int)L.E, a.sk, a.row_index, a.pre)
#define NVFP4_TILE_LAUNCH_FMT(KF, PRE)                                                                                  \
    if (L.mx) NVFP4_TILE_LAUNCH(KF, PRE, true);                                                                         \
    else NVFP4_TILE_LAUNCH(KF, PRE, false)
    if (L.K % kChunkK == 0) {
        if (a.pre) { NVFP4_TILE_LAUNCH_FMT(true, true); }
        else { NVFP4_TILE_LAUNCH_FMT(true, false); }
    } else {
        if (a.pre) { NVFP4_TILE_LAUNCH_FMT(false, true); }
        else { NVFP4_TILE_LAUNCH_FMT(false, false); }
    }
#undef NVFP4_TILE_LAUNCH_FMT
#undef NVFP4_TILE_LAUNCH
}

}  // namespace

template <bool F16>
nvfp4_status launch_tile(const TileShape& t, const Layout& L, const GemmArgs& a, bool grouped) {
    static_assert(F16 == kF16, "this unit holds one activation type");
    if (t.mtiles > 65535)
        return fail(NVFP4_ERR_INVALID_ARG, "tile GEMM: %lld row tiles exceed the grid limit", (long long)t.mtiles);
    if (grouped) {
        // four units per wave (gate / up pairs stay in one wave), a 3-deep ring
        // (MoE T = 2048 FC1 / FC2: 188 / 113 us against 194 / 117 us with 2 deep;
        // deeper, narrower, shorter or taller tiles measured slower)
        if (a.act == kActSiluGlu) launch_tile_t<4, 4, 4, 1, 3, true, kActSiluGlu>(t, L, a);
        else if (a.act == kActRelu2) launch_tile_t<4, 4, 4, 1, 3, true, kActRelu2>(t, L, a);
        else launch_tile_t<4, 4, 4, 1, 3, true>(t, L, a);
    } else {
        if (t.ms == 1) launch_tile_t<1, 1, 4, 4, 2, false>(t, L, a);
        else if (t.ms == 2) launch_tile_t<2, 1, 4, 2, 4, false>(t, L, a);
        else if (t.ms == 4 && t.kw == 1) launch_tile_t<4, 4, 8, 1, 4, false>(t, L, a);
        else if (t.ms == 4) launch_tile_t<4, 1, 4, 4, 2, false>(t, L, a);
        else launch_tile_t<8, 2, 8, 1, 2, false>(t, L, a);
    }
    return launched("tile GEMM");
}

template nvfp4_status launch_tile<kF16>(const TileShape&, const Layout&, const GemmArgs&, bool);

}  // namespace nvfp4
