// Host launcher of the MFMA-bound dense kernel (kernels_mfma.h).  Its
// kernels live in their own translation units (gemm_mfma.hip), built without
// the register-form flag of the other kernels' units (this kernel keeps its
// accumulators in the accumulation registers).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace nvfp4 {

// One whole output tile of the MFMA-bound kernel: 256 rows x 16 units (256 columns).
constexpr int kMfmaRows = 256;
constexpr int kMfmaTileUnits = 16;

// Work split of one call: `tiles` output tiles; the first t_full run as whole
// tiles, the rest as two half-height workgroups each.
struct MfmaPlan {
    int64_t tiles, t_full;
};
MfmaPlan mfma_plan(const Layout& L, int64_t M);

// Launches Y[M, N] = g * (X[M, K] (.) pre) . dequant(W)^T on `st` (dense,
// E = 1) with the work split of `plan` (at most two kernel launches); X, pre
// and Y are bf16, or fp16 when f16; pre may be NULL.  quarter: every tile
// runs as four 64-row workgroups instead (one launch; several workgroups
// share a compute unit).  Arguments are checked by the caller; returns the
// launch status.
hipError_t launch_gemm_mfma(const MfmaPlan& plan, const Layout& L, const uint16_t* x, int64_t ld_x, const uint8_t* blob,
                            const float* gs, int g_div, uint16_t* y, int64_t ld_y, int64_t M, const uint16_t* pre,
                            bool quarter, hipStream_t st, bool f16);

// The launch of one activation type (F16), pre-scale form (PRE) and scale
// format (MX: E8M0 per 32, else E4M3 per 16), defined in the gemm_mfma.hip
// unit compiled for that form.
template <bool F16, bool PRE, bool MX>
hipError_t launch_mfma_t(const MfmaPlan& plan, const Layout& L, const uint16_t* x, int64_t ld_x, const uint8_t* blob,
                         const float* gs, int g_div, uint16_t* y, int64_t ld_y, int64_t M, const uint16_t* pre,
                         bool quarter, hipStream_t st);

// Grouped (MoE) form over E experts (L.E): rows [offsets[e], offsets[e+1])
// use expert e (R rows in all); grouped row r reads activation row
// row_index[r] when row_index is given.  act: the epilogue's MoE activation
// (decode.h: kActNone, or kActSiluGlu on a gated blob).  One launch
// of (R / 256 + E) x (tile columns) + 8 workgroups.
hipError_t launch_gemm_mfma_grouped(const Layout& L, const uint16_t* x, int64_t ld_x, const int32_t* row_index,
                                    const int32_t* offsets, int64_t R, const uint8_t* blob, const float* gs, int g_div,
                                    uint16_t* y, int64_t ld_y, const uint16_t* pre, int act, hipStream_t st, bool f16);
template <bool F16, bool PRE, bool MX>
hipError_t launch_mfma_grouped_t(const Layout& L, const uint16_t* x, int64_t ld_x, const int32_t* row_index,
                                 const int32_t* offsets, int64_t R, const uint8_t* blob, const float* gs, int g_div,
                                 uint16_t* y, int64_t ld_y, const uint16_t* pre, int act, hipStream_t st);

}  // namespace nvfp4
