// Launchers of the activation-resident kernel family (kernels_xres.h) for
// one activation type: this unit is compiled once per type, with
// NVFP4_ACT_F16 = 0 (bf16) and 1 (fp16).
#include "kernels_xres.h"
#include "plan.h"

#ifndef NVFP4_ACT_F16
#error "compile with -DNVFP4_ACT_F16=0 (bf16) or -DNVFP4_ACT_F16=1 (fp16)"
#endif

namespace nvfp4 {

namespace {
constexpr bool kF16 = NVFP4_ACT_F16 != 0;
}  // namespace

template <bool F16>
nvfp4_status launch_xres(const XresShape& s, const Layout& L, const GemmArgs& a) {
    static_assert(F16 == kF16, "this unit holds one activation type");
    const BlobView bv = make_view(L, a.blob);
    const dim3 grid((unsigned)s.groups, (unsigned)s.S);
    bool done = false;
#define NVFP4_XRES_LAUNCH(CH, U, W, D, FULL, PRE)                                                                    \
    hipLaunchKernelGGL((k_gemm_xres<CH, U, W, D, FULL, kF16, PRE>), grid, dim3(W * 64), 0, a.st, a.x, a.ld_x, bv,   \
                       (int)L.NU, (int)L.KC, (int)L.K, (int)L.N, a.gs, a.g_div, a.y, a.ld_y, (int)a.rows, a.sk, a.pre)
#define NVFP4_XRES_DISPATCH(CH, U, W, D)                                        \
    if (!done && s.ch == CH && s.u == U && s.w == W && s.d == D) {             \
        const bool full = L.K == (int64_t)s.S * CH * W * kChunkK;             \
        if (full && a.pre) NVFP4_XRES_LAUNCH(CH, U, W, D, true, true);        \
        else if (full) NVFP4_XRES_LAUNCH(CH, U, W, D, true, false);           \
        else if (a.pre) NVFP4_XRES_LAUNCH(CH, U, W, D, false, true);          \
        else NVFP4_XRES_LAUNCH(CH, U, W, D, false, false);                    \
        done = true;                                                           \
    }
    NVFP4_XRES_CONFIGS(NVFP4_XRES_DISPATCH)
#undef NVFP4_XRES_DISPATCH
#undef NVFP4_XRES_LAUNCH
    if (!done) return fail(NVFP4_ERR_INVALID_ARG, "activation-resident GEMM: no compiled kernel for this shape");
    return launched("activation-resident GEMM");
}

template nvfp4_status launch_xres<kF16>(const XresShape&, const Layout&, const GemmArgs&);

}  // namespace nvfp4
