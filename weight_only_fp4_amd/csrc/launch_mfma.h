// Host launcher of the MFMA-bound dense kernel (kernels_mfma.h).  It lives
// in its own translation unit, compiled without the flag that keeps MFMA
// results in architectural VGPRs: its 8 x 8 accumulator tiles need the
// accumulation registers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace nvfp4 {

// Rows per workgroup tile of the MFMA-bound kernel.
constexpr int kMfmaRows = 128;

// Launches Y[M, N] = g * X[M, K] . dequant(W)^T on `st` (dense, E = 1).
// Arguments are checked by the caller; returns the launch status.
hipError_t launch_gemm_mfma(const Layout& L, const uint16_t* x, int64_t ld_x, const uint8_t* blob, const float* gs,
                            int g_div, uint16_t* y, int64_t ld_y, int64_t M, hipStream_t st);

}  // namespace nvfp4
