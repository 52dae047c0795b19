// Translation unit of the MFMA-bound dense kernel (see launch_mfma.h).
#include "kernels_mfma.h"
#include "launch_mfma.h"

namespace nvfp4 {

static_assert(kMfmaRows == kMfmaBM, "one tile height");

constexpr int kMfmaNT = 4;   // units per wave: 128 x 64 outputs, 128 accumulators
constexpr int kMfmaWN = 8;   // waves per workgroup (two per SIMD): 128 x 512 outputs

template <bool KFULL>
static hipError_t launch_mfma_k(const Layout& L, const uint16_t* x, int64_t ld_x, const uint8_t* blob, const float* gs,
                                int g_div, uint16_t* y, int64_t ld_y, int64_t M, hipStream_t st) {
    const dim3 grid((unsigned)((L.NU + kMfmaNT * kMfmaWN - 1) / (kMfmaNT * kMfmaWN)), (unsigned)((M + kMfmaBM - 1) / kMfmaBM));
    hipLaunchKernelGGL((k_gemm_mfma<kMfmaNT, kMfmaWN, KFULL>), grid, dim3(kMfmaWN * 64), 0, st, x, ld_x, make_view(L, blob), (int)L.NU,
                       (int)L.KC, (int)L.K, (int)L.N, gs, g_div, y, ld_y, (int)M);
    return hipGetLastError();
}

hipError_t launch_gemm_mfma(const Layout& L, const uint16_t* x, int64_t ld_x, const uint8_t* blob, const float* gs,
                            int g_div, uint16_t* y, int64_t ld_y, int64_t M, hipStream_t st) {
    return L.K % kChunkK == 0 ? launch_mfma_k<true>(L, x, ld_x, blob, gs, g_div, y, ld_y, M, st)
                              : launch_mfma_k<false>(L, x, ld_x, blob, gs, g_div, y, ld_y, M, st);
}

}  // namespace nvfp4
