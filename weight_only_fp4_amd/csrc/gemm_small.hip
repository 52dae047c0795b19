// Launchers of the small-M kernel family (kernels_gemm.h) for one activation
// type: this unit is compiled once per type, with NVFP4_ACT_F16 = 0 (bf16)
// and 1 (fp16), so the two sets of kernels build in parallel.
#include "plan.h"

#ifndef NVFP4_ACT_F16
#error "compile with -DNVFP4_ACT_F16=0 (bf16) or -DNVFP4_ACT_F16=1 (fp16)"
#endif

namespace nvfp4 {

namespace {

constexpr bool kF16 = NVFP4_ACT_F16 != 0;

template <int MG, int NT, int W, int D, bool GROUPED, int ACT = kActNone>
void launch_small_t(const SmallShape& s, const Layout& L, const GemmArgs& a) {
    const BlobView bv = make_view(L, a.blob);
    const dim3 grid((unsigned)s.groups, GROUPED ? (unsigned)L.E : 1u, (unsigned)s.S);
    const int64_t rows = GROUPED ? 0 : a.rows;
#define NVFP4_SMALL_LAUNCH(KF, PRE)                                                                                \
    hipLaunchKernelGGL((k_gemm_small_m<MG, NT, W, D, GROUPED, KF, kF16, PRE, ACT>), grid, dim3(W * 64), 0, a.st,   \
                       a.x, a.ld_x, bv, (int)L.NU, (int)L.KC, (int)L.K, (int)L.N, a.gs, a.g_div, a.y, a.ld_y, rows, \
                       a.offsets, a.sk, a.row_index, a.pre)
    if (L.K % kChunkK == 0) {
        if (a.pre) NVFP4_SMALL_LAUNCH(true, true);
        else NVFP4_SMALL_LAUNCH(true, false);
    } else {
        if (a.pre) NVFP4_SMALL_LAUNCH(false, true);
        else NVFP4_SMALL_LAUNCH(false, false);
    }
#undef NVFP4_SMALL_LAUNCH
}

}  // namespace

template <bool F16>
nvfp4_status launch_small(const SmallShape& s, const Layout& L, const GemmArgs& a, bool grouped) {
    static_assert(F16 == kF16, "this unit holds one activation type");
    bool done = false;
    if (grouped) {
        if ((a.act == kActSiluGlu) != (s.nt == 2))
            return fail(NVFP4_ERR_INVALID_ARG, "small-M GEMM: the gated epilogue takes unit pairs");
#define NVFP4_SMALL_GROUPED_W(MG, NT, D, ACT)                                  \
    switch (s.w) {                                                            \
        case 1: launch_small_t<MG, NT, 1, D, true, ACT>(s, L, a); break;      \
        case 2: launch_small_t<MG, NT, 2, D, true, ACT>(s, L, a); break;      \
        case 4: launch_small_t<MG, NT, 4, D, true, ACT>(s, L, a); break;      \
        default: launch_small_t<MG, NT, 8, D, true, ACT>(s, L, a); break;     \
    }
#define NVFP4_SMALL_GROUPED(NT, ACT)                                           \
    if (s.mg == 1) {                                                          \
        NVFP4_SMALL_GROUPED_W(1, NT, (NT == 1 ? 6 : 4), ACT)                  \
    } else {                                                                  \
        NVFP4_SMALL_GROUPED_W(0, NT, 4, ACT)                                  \
    }
        if ((s.mg != 0 && s.mg != 1) || s.d != (s.mg == 1 && s.nt == 1 ? 6 : 4))
            return fail(NVFP4_ERR_INVALID_ARG, "small-M GEMM: no grouped kernel for mg=%d d=%d", s.mg, s.d);
        if (a.act == kActSiluGlu) NVFP4_SMALL_GROUPED(2, kActSiluGlu)
        else if (a.act == kActRelu2) NVFP4_SMALL_GROUPED(1, kActRelu2)
        else NVFP4_SMALL_GROUPED(1, kActNone)
#undef NVFP4_SMALL_GROUPED
#undef NVFP4_SMALL_GROUPED_W
        done = true;
    } else {
#define NVFP4_SMALL_DISPATCH(MG, NT, W, D)                             \
    if (!done && s.mg == MG && s.nt == NT && s.w == W && s.d == D) { \
        launch_small_t<MG, NT, W, D, false>(s, L, a);                \
        done = true;                                                 \
    }
        NVFP4_SMALL_CONFIGS(NVFP4_SMALL_DISPATCH)
#undef NVFP4_SMALL_DISPATCH
    }
    if (!done)
        return fail(NVFP4_ERR_INVALID_ARG, "small-M GEMM: no compiled kernel for shape mg=%d nt=%d w=%d d=%d", s.mg,
                    s.nt, s.w, s.d);
    return launched("small-M GEMM");
}

template nvfp4_status launch_small<kF16>(const SmallShape&, const Layout&, const GemmArgs&, bool);

}  // namespace nvfp4
