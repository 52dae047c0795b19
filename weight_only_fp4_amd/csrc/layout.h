// Repacked weight layout shared by every kernel of the library.
//
// A weight matrix of N rows (output features) and K columns (reduction) is
// cut into units of 16 rows by 128 columns.  N is padded to a multiple of 16
// and K to a multiple of 128 with zero codes and zero scale bytes, which
// decode to +0 and contribute nothing.  The order of the (unit, chunk)
// blocks within an expert is set by kChunkMajor below.
//
// codes region  : E x NU x KC blocks of 1024 bytes.  In a block, lane l of a
//                 wave owns bytes [16 l, 16 l + 16): the canonical bytes of
//                 row 16 u + (l & 15) covering k in [128 c + 32 (l >> 4), +32)
//                 (low nibble = even k, as in the canonical input).  One
//                 128-bit load per lane therefore hands lane l the 32 codes
//                 of one row and one 32-wide K group, and a wave's load is
//                 one contiguous kilobyte.
// scales region : E x NU x KC blocks of 128 bytes, in the same order.  Lane l owns bytes
//                 [2 l, 2 l + 2): the E4M3 scales of the two 16-wide blocks
//                 of its 32-wide K group (low byte = lower k).
//
// Total size: E * NU * KC * 1152 bytes, i.e. 0.5625 bytes per weight plus
// padding.
//
// MXFP4 weights (one E8M0 scale per 32 K) use the same layout: a lane's 32
// codes are exactly one MXFP4 group, and both of its scale bytes hold that
// group's E8M0 byte.  The blob does not record its format; `mx` in the
// layout and the view (set by the mxfp4_* entry points) selects the scale
// decode.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kUnitN = 16;
constexpr int kChunkK = 128;
constexpr int kCodeBlock = 1024;
constexpr int kScaleBlock = 128;

// Order of the (row unit, K chunk) blocks of one expert.  Unit-major keeps
// the K stream of a row unit contiguous; chunk-major keeps the blocks of all
// row units for one K chunk contiguous.
constexpr bool kChunkMajor = false;

struct Layout {
    int64_t E, N, K;
    int64_t NU;   // row units (ceil(N / 16))
    int64_t KC;   // K chunks (ceil(K / 128))
    int mx;       // scale bytes are E8M0 (MXFP4), not E4M3 (NVFP4)
    int64_t blocks() const { return E * NU * KC; }
    int64_t code_bytes() const { return blocks() * kCodeBlock; }
    int64_t total_bytes() const { return blocks() * (kCodeBlock + kScaleBlock); }
    int64_t unit_stride() const { return kChunkMajor ? 1 : KC; }    // in blocks
    int64_t chunk_stride() const { return kChunkMajor ? NU : 1; }   // in blocks
};

inline Layout make_layout(int64_t E, int64_t N, int64_t K, int mx = 0) {
    return Layout{E, N, K, (N + kUnitN - 1) / kUnitN, (K + kChunkK - 1) / kChunkK, mx};
}

// What a kernel needs to address the blocks of a repacked blob.
struct BlobView {
    const uint8_t* codes;
    const uint8_t* scales;
    int64_t expert_blocks;   // blocks per expert (NU * KC)
    int64_t unit_stride;     // blocks between consecutive row units
    int64_t chunk_stride;    // blocks between consecutive K chunks
    int mx;                  // scale bytes are E8M0 (MXFP4), not E4M3 (NVFP4)
    __host__ __device__ int64_t block(int64_t e, int64_t u, int64_t c) const {
        return e * expert_blocks + u * unit_stride + c * chunk_stride;
    }
};

inline BlobView make_view(const Layout& L, const uint8_t* blob) {
    return BlobView{blob, blob + L.code_bytes(), L.NU * L.KC, L.unit_stride(), L.chunk_stride(), L.mx};
}

}  // namespace nvfp4
