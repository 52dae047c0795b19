// Launchers of the MFMA-bound kernel (kernels_mfma.h) for one activation
// type, one pre-scale form and one scale format: this unit is compiled eight
// times, with NVFP4_ACT_F16 = 0 (bf16) / 1 (fp16), NVFP4_PRE = 0 / 1 and
// NVFP4_MX = 0 (NVFP4) / 1 (MXFP4), so that its large kernels build in
// parallel.  It is built without the register-form MFMA
// flag of the other units (this kernel keeps its accumulators in the
// accumulation registers).
#include "kernels_mfma.h"
#include "launch_mfma.h"

#if !defined(NVFP4_ACT_F16) || !defined(NVFP4_PRE) || !defined(NVFP4_MX)
#error "compile with -DNVFP4_ACT_F16=0|1, -DNVFP4_PRE=0|1 and -DNVFP4_MX=0|1"
#endif

namespace nvfp4 {

static_assert(kMfmaRows == kMfmaTileRows && kMfmaTileUnits == kMfmaUnits, "one tile shape");

namespace {

constexpr bool kF16 = NVFP4_ACT_F16 != 0;
constexpr bool kPre = NVFP4_PRE != 0;
constexpr bool kMx = NVFP4_MX != 0;

template <int MS, bool KFULL>
hipError_t launch_part(int64_t wgs, int64_t t0, const Layout& L, const uint16_t* x, int64_t ld_x, const uint8_t* blob,
                       const float* gs, int g_div, uint16_t* y, int64_t ld_y, int64_t M, const uint16_t* pre,
                       hipStream_t st) {
    if (wgs == 0) return hipSuccess;
    // 16-byte output stores need 16-byte aligned rows
    const int vec = (ld_y % 8 == 0) && (reinterpret_cast<uintptr_t>(y) % 16 == 0);
    hipLaunchKernelGGL((k_gemm_mfma<MS, KFULL, kF16, kPre, kMx>), dim3((unsigned)wgs), dim3(kMfmaWN * 64), 0, st, x, ld_x,
                       make_view(L, blob), (int)L.NU, (int)L.KC, (int)L.K, (int)L.N, gs, g_div, y, ld_y, (int)M,
                       (int)t0, vec, pre);
    return hipGetLastError();
}

template <bool KFULL>
hipError_t launch_k(const MfmaPlan& p, const Layout& L, const uint16_t* x, int64_t ld_x, const uint8_t* blob,
                    const float* gs, int g_div, uint16_t* y, int64_t ld_y, int64_t M, const uint16_t* pre,
                    bool quarter, hipStream_t st) {
    if (quarter)   // every tile as four 64-row workgroups (several share a compute unit)
        return launch_part<4, KFULL>(4 * p.tiles, 0, L, x, ld_x, blob, gs, g_div, y, ld_y, M, pre, st);
    hipError_t e = launch_part<16, KFULL>(p.t_full, 0, L, x, ld_x, blob, gs, g_div, y, ld_y, M, pre, st);
    if (e != hipSuccess) return e;
    return launch_part<8, KFULL>(2 * (p.tiles - p.t_full), p.t_full, L, x, ld_x, blob, gs, g_div, y, ld_y, M, pre, st);
}

}  // namespace

template <bool F16, bool PRE, bool MX>
hipError_t launch_mfma_t(const MfmaPlan& p, const Layout& L, const uint16_t* x, int64_t ld_x, const uint8_t* blob,
                         const float* gs, int g_div, uint16_t* y, int64_t ld_y, int64_t M, const uint16_t* pre,
                         bool quarter, hipStream_t st) {
    static_assert(F16 == kF16 && PRE == kPre && MX == kMx, "this unit holds one form");
    if (L.mx != (int)MX) return hipErrorInvalidValue;
    return L.K % kChunkK == 0 ? launch_k<true>(p, L, x, ld_x, blob, gs, g_div, y, ld_y, M, pre, quarter, st)
                              : launch_k<false>(p, L, x, ld_x, blob, gs, g_div, y, ld_y, M, pre, quarter, st);
}

template <bool F16, bool PRE, bool MX>
hipError_t launch_mfma_grouped_t(const Layout& L, const uint16_t* x, int64_t ld_x, const int32_t* row_index,
                                 const int32_t* offsets, int64_t R, const uint8_t* blob, const float* gs, int g_div,
                                 uint16_t* y, int64_t ld_y, const uint16_t* pre, int act, hipStream_t st) {
    static_assert(F16 == kF16 && PRE == kPre && MX == kMx, "this unit holds one form");
    if (L.mx != (int)MX || act == kActRelu2) return hipErrorInvalidValue;   // the squared ReLU runs on the tile kernel
    const int64_t cols = (L.NU + kMfmaTileUnits - 1) / kMfmaTileUnits;
    const int64_t wgs = ((R + kMfmaRows - 1) / kMfmaRows + L.E) * cols + 8;
    // 16-byte output stores need 16-byte aligned rows
    const int vec = (ld_y % 8 == 0) && (reinterpret_cast<uintptr_t>(y) % 16 == 0);
    const BlobView bv = make_view(L, blob);
#define NVFP4_MFMA_GROUPED(KF, ACT)                                                                                    \
    hipLaunchKernelGGL((k_gemm_mfma<16, KF, kF16, kPre, kMx, true, ACT>), dim3((unsigned)wgs), dim3(kMfmaWN * 64), 0, \
                       st, x, ld_x, bv, (int)L.NU, (int)L.KC, (int)L.K, (int)L.N, gs, g_div, y, ld_y, 0, 0, vec, pre, \
                       offsets, (int)L.E, row_index)
#define NVFP4_MFMA_GROUPED_ACT(KF)                                      \
    if (act == kActSiluGlu) NVFP4_MFMA_GROUPED(KF, kActSiluGlu);       \
    else NVFP4_MFMA_GROUPED(KF, kActNone);
    if (L.K % kChunkK == 0) {
        NVFP4_MFMA_GROUPED_ACT(true)
    } else {
        NVFP4_MFMA_GROUPED_ACT(false)
    }
#undef NVFP4_MFMA_GROUPED_ACT
#undef NVFP4_MFMA_GROUPED
    return hipGetLastError();
}

template hipError_t launch_mfma_grouped_t<kF16, kPre, kMx>(const Layout&, const uint16_t*, int64_t, const int32_t*,
                                                           const int32_t*, int64_t, const uint8_t*, const float*, int,
                                                           uint16_t*, int64_t, const uint16_t*, int, hipStream_t);

template hipError_t launch_mfma_t<kF16, kPre, kMx>(const MfmaPlan&, const Layout&, const uint16_t*, int64_t, const uint8_t*,
                                              const float*, int, uint16_t*, int64_t, int64_t, const uint16_t*, bool,
                                              hipStream_t);

}  // namespace nvfp4
