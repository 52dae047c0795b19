// Translation unit of the MFMA-bound dense kernel (see launch_mfma.h).
#include "kernels_mfma.h"
#include "launch_mfma.h"

namespace nvfp4 {

static_assert(kMfmaRows == kMfmaTileRows, "one tile height");

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
    p.tiles = ((L.NU + kMfmaUnits - 1) / kMfmaUnits) * ((M + kMfmaTileRows - 1) / kMfmaTileRows);
    p.t_full = p.tiles;
    // The tiles of the last wave of workgroups run as two half-height
    // workgroups each when those all fit in one wave of the chip: that wave
    // then takes about half as long.
    const int64_t slots = compute_units();
    const int64_t rem = p.tiles % slots;
    if (rem > 0 && 2 * rem <= slots) p.t_full = p.tiles - rem;
    return p;
}

template <int MS, bool KFULL, bool F16>
static hipError_t launch_part(int64_t wgs, int64_t t0, const Layout& L, const uint16_t* x, int64_t ld_x,
                              const uint8_t* blob, const float* gs, int g_div, uint16_t* y, int64_t ld_y, int64_t M,
                              hipStream_t st) {
    if (wgs == 0) return hipSuccess;
    // 16-byte output stores need 16-byte aligned rows
    const int vec = (ld_y % 8 == 0) && (reinterpret_cast<uintptr_t>(y) % 16 == 0);
    hipLaunchKernelGGL((k_gemm_mfma<MS, KFULL, F16>), dim3((unsigned)wgs), dim3(kMfmaWN * 64), 0, st, x, ld_x,
                       make_view(L, blob), (int)L.NU, (int)L.KC, (int)L.K, (int)L.N, gs, g_div, y, ld_y, (int)M, (int)t0,
                       vec);
    return hipGetLastError();
}

template <bool KFULL, bool F16>
static hipError_t launch_mfma_k(const MfmaPlan& p, const Layout& L, const uint16_t* x, int64_t ld_x, const uint8_t* blob,
                                const float* gs, int g_div, uint16_t* y, int64_t ld_y, int64_t M, hipStream_t st) {
    hipError_t e = launch_part<16, KFULL, F16>(p.t_full, 0, L, x, ld_x, blob, gs, g_div, y, ld_y, M, st);
    if (e != hipSuccess) return e;
    return launch_part<8, KFULL, F16>(2 * (p.tiles - p.t_full), p.t_full, L, x, ld_x, blob, gs, g_div, y, ld_y, M, st);
}

hipError_t launch_gemm_mfma(const MfmaPlan& p, const Layout& L, const uint16_t* x, int64_t ld_x, const uint8_t* blob,
                            const float* gs, int g_div, uint16_t* y, int64_t ld_y, int64_t M, hipStream_t st,
                            bool f16) {
    const bool kfull = L.K % kChunkK == 0;
    if (f16)
        return kfull ? launch_mfma_k<true, true>(p, L, x, ld_x, blob, gs, g_div, y, ld_y, M, st)
                     : launch_mfma_k<false, true>(p, L, x, ld_x, blob, gs, g_div, y, ld_y, M, st);
    return kfull ? launch_mfma_k<true, false>(p, L, x, ld_x, blob, gs, g_div, y, ld_y, M, st)
                 : launch_mfma_k<false, false>(p, L, x, ld_x, blob, gs, g_div, y, ld_y, M, st);
}

}  // namespace nvfp4
