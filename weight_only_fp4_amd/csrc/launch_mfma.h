// Host launcher of the MFMA-bound dense kernel (kernels_mfma.h).  It lives
// in its own translation unit, built without the register-form flag of the
// other kernels' unit (this kernel keeps its accumulators in the
// accumulation registers).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace nvfp4 {

// Rows of one whole output tile of the MFMA-bound kernel (256 x 256).
constexpr int kMfmaRows = 256;

// Work split of one call: `tiles` output tiles; the first t_full run as whole
// tiles, the rest as two half-height workgroups each.
struct MfmaPlan {
    int64_t tiles, t_full;
};
MfmaPlan mfma_plan(const Layout& L, int64_t M);

// Launches Y[M, N] = g * X[M, K] . dequant(W)^T on `st` (dense, E = 1) with
// the work split of `plan` (at most two kernel launches); X and Y are bf16,
// or fp16 when f16.  Arguments are checked by the caller; returns the launch
// status.
hipError_t launch_gemm_mfma(const MfmaPlan& plan, const Layout& L, const uint16_t* x, int64_t ld_x, const uint8_t* blob,
                            const float* gs, int g_div, uint16_t* y, int64_t ld_y, int64_t M, hipStream_t st,
                            bool f16);

}  // namespace nvfp4
