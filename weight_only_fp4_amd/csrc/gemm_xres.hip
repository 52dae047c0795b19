// Launchers of the activation-resident kernel family (kernels_xres.h) for
// one activation type and one scale format: this unit is compiled four
// times, with NVFP4_ACT_F16 = 0 (bf16) / 1 (fp16) and NVFP4_MX = 0 (NVFP4:
// E4M3 scales per 16) / 1 (MXFP4: E8M0 scales per 32).
#include "kernels_xres.h"
#include "plan.h"

#if !defined(NVFP4_ACT_F16) || !defined(NVFP4_MX)
#error "compile with -DNVFP4_ACT_F16=0|1 and -DNVFP4_MX=0|1"
#endif

namespace nvfp4 {

namespace {
constexpr bool kF16 = NVFP4_ACT_F16 != 0;
constexpr bool kMx = NVFP4_MX != 0;
}  // namespace

template <bool F16, bool MX>
nvfp4_status launch_xres(const XresShape& s, const Layout& L, const GemmArgs& a) {
    static_assert(F16 == kF16 && MX == kMx, "this unit holds one activation type and one scale format");
    if (L.mx != (int)MX) return fail(NVFP4_ERR_INVALID_ARG, "activation-resident GEMM: scale format mismatch");
    const BlobView bv = make_view(L, a.blob);
    const dim3 grid((unsigned)s.groups, (unsigned)s.S);
    bool done = false;
#define NVFP4_XRES_LAUNCH(CH, U, W, D, FULL, PRE)                                                                    \
    hipLaunchKernelGGL((k_gemm_xres<CH, U, W, D, FULL, kF16, PRE, kMx>), grid, dim3(W * 64), 0, a.st, a.x, a.ld_x, bv,   \
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

template nvfp4_status launch_xres<kF16, kMx>(const XresShape&, const Layout&, const GemmArgs&);

}  // namespace nvfp4
