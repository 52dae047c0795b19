// Work split and form dispatch of the MFMA-bound dense kernel (see
// launch_mfma.h); the kernels themselves are launched from gemm_mfma.hip.
#include "launch_mfma.h"

namespace nvfp4 {

// Compute units of the current device.  One workgroup of the whole-tile
// kernel fits on a compute unit at a time (its staged activations take
// 128 KB of LDS).
static int compute_units() {
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64 && cache[dev] > 0) return cache[dev];
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    if (dev < 64) cache[dev] = n;
    return n;
}

MfmaPlan mfma_plan(const Layout& L, int64_t M) {
    MfmaPlan p;
    p.tiles = ((L.NU + kMfmaTileUnits - 1) / kMfmaTileUnits) * ((M + kMfmaRows - 1) / kMfmaRows);
    p.t_full = p.tiles;
    // The tiles of the last wave of workgroups run as two half-height
    // workgroups each when those all fit in one wave of the chip: that wave
    // then takes about half as long.
    const int64_t slots = compute_units();
    const int64_t rem = p.tiles % slots;
    if (rem > 0 && 2 * rem <= slots) p.t_full = p.tiles - rem;
    return p;
}

hipError_t launch_gemm_mfma(const MfmaPlan& p, const Layout& L, const uint16_t* x, int64_t ld_x, const uint8_t* blob,
                            const float* gs, int g_div, uint16_t* y, int64_t ld_y, int64_t M, const uint16_t* pre,
                            bool quarter, hipStream_t st, bool f16) {
#define NVFP4_MFMA_FORM(F16, PRE, MX) \
    return launch_mfma_t<F16, PRE, MX>(p, L, x, ld_x, blob, gs, g_div, y, ld_y, M, pre, quarter, st)
#define NVFP4_MFMA_PRE(F16, MX) \
    if (pre) NVFP4_MFMA_FORM(F16, true, MX); \
    NVFP4_MFMA_FORM(F16, false, MX)
    if (f16) {
        if (L.mx) { NVFP4_MFMA_PRE(true, true); }
        NVFP4_MFMA_PRE(true, false);
    }
    if (L.mx) { NVFP4_MFMA_PRE(false, true); }
    NVFP4_MFMA_PRE(false, false);
#undef NVFP4_MFMA_PRE
#undef NVFP4_MFMA_FORM
}

hipError_t launch_gemm_mfma_grouped(const Layout& L, const uint16_t* x, int64_t ld_x, const int32_t* row_index,
                                    const int32_t* offsets, int64_t R, const uint8_t* blob, const float* gs, int g_div,
                                    uint16_t* y, int64_t ld_y, const uint16_t* pre, int act, hipStream_t st, bool f16) {
#define NVFP4_MFMA_GFORM(F16, PRE, MX) \
    return launch_mfma_grouped_t<F16, PRE, MX>(L, x, ld_x, row_index, offsets, R, blob, gs, g_div, y, ld_y, pre, act, st)
#define NVFP4_MFMA_GPRE(F16, MX) \
    if (pre) NVFP4_MFMA_GFORM(F16, true, MX); \
    NVFP4_MFMA_GFORM(F16, false, MX)
    if (f16) {
        if (L.mx) { NVFP4_MFMA_GPRE(true, true); }
        NVFP4_MFMA_GPRE(true, false);
    }
    if (L.mx) { NVFP4_MFMA_GPRE(false, true); }
    NVFP4_MFMA_GPRE(false, false);
#undef NVFP4_MFMA_GPRE
#undef NVFP4_MFMA_GFORM
}

}  // namespace nvfp4
