// Device-side number formats: E4M3 scale bytes, E2M1 codes, bf16 rounding.
//
// The hardware conversion v_cvt_scalef32_pk_{f32,bf16}_fp4 turns two E2M1
// codes (one byte, low nibble first) into two values and multiplies them by
// 2^exponent(scale operand): only the exponent field of the fp32 scale is
// used, its sign and mantissa are ignored.  An E4M3 scale has a 4-bit
// significand, so the decode applies the scale in two parts: the power of
// two inside the conversion (or a multiply by 1.0 there and a full fp32
// multiply after it), and the remaining significand factor by an fp32
// multiply.  e2m1 * e4m3 has at most 6 significant bits and lies in
// [2^-10, 2688], so every product is exact in fp32 and in bf16.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// E4M3 (OCP E4M3FN: bias 7, subnormal m * 2^-9, 0x7F / 0xFF NaN) -> fp32, exact.
// Branch-free: the exponent and mantissa bits are placed under an fp32
// exponent field biased by 120, so normal codes become 2^(e-127) (1 + m/8)
// and subnormal codes (e = 0) the fp32 denormal m 2^-129; one multiply by
// 2^120 then gives 2^(e-7) (1 + m/8), resp. m 2^-9, exactly (fp32 denormals
// are kept, the default of this target).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    const float mag = __uint_as_float((b & 0x7Fu) << 20) * 0x1p120f;
    const float v = ((b & 0x7Fu) == 0x7Fu) ? __uint_as_float(0x7FC00000u) : mag;
    return __uint_as_float(__float_as_uint(v) | ((b & 0x80u) << 24));
}

// E8M0 (OCP MX scale: 2^(e-127), 0xFF NaN) -> fp32, exact: the byte becomes
// the fp32 exponent field, except 0 (2^-127, an fp32 denormal) and 0xFF.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
    b &= 0xFFu;
    const uint32_t bits = b == 0u ? 0x00400000u : b == 0xFFu ? 0x7FC00000u : b << 23;
    return __uint_as_float(bits);
}

// The two scale bytes of a lane (bits 0..15, low byte = lower k) -> fp32:
// E4M3 by the hardware conversion (NVFP4), or E8M0 (MXFP4, where both bytes
// hold the lane's one group scale).  The format is a compile-time choice so
// that the NVFP4 loops carry no test of it.
template <bool MX>
__device__ __forceinline__ f32x2 scale_pair_f32(uint32_t sp) {
    if constexpr (MX) {
        // the repack stores the lane's one E8M0 group scale in both bytes: convert it once
        const float v = e8m0_to_f32(sp);
        return f32x2{v, v};
    } else {
        return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sp, 1.0f, false);
    }
}

// Split a scale s into the operand handed to the exponent-only conversion
// (its exponent is applied there) and the fp32 factor that completes it:
// e2m1 * s == (e2m1 * 2^exp(cvt_scale)) * factor, exactly.  Zero and NaN
// scales convert with 1.0 and carry the whole value in the factor.
__device__ __forceinline__ void split_scale(float s, float& cvt_scale, float& factor) {
    const uint32_t u = __float_as_uint(s);
    const bool special = (s == 0.0f) || (s != s);
    cvt_scale = special ? 1.0f : s;
    factor = special ? s : __uint_as_float((u & 0x807FFFFFu) | 0x3F800000u);
}

// Round-to-nearest-even fp32 -> bf16 bit pattern (NaN kept quiet, sign kept).
// Written as a select, not a branch: the compiler otherwise turns the NaN
// test into divergent control flow around every rounding.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t rne = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    const uint32_t qnan = ((u >> 16) & 0x8000u) | 0x7FC0u;
    return (u & 0x7FFFFFFFu) > 0x7F800000u ? qnan : rne;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Upper halves of two fp32 values -> one dword of two bf16 (lo first).  Exact
// when both values are representable in bf16 (true for decoded weights).
__device__ __forceinline__ uint32_t pack_hi_halves(float lo, float hi) {
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Eight E2M1 codes of one dword (code of the lowest k in the lowest nibble)
// times a full fp32 scale -> eight bf16 in k order, exact.
__device__ __forceinline__ uint4 decode8_bf16(uint32_t codes, float scale) {
    const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
    const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
    const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
    const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
    uint4 r;
    r.x = pack_hi_halves(p0.x * scale, p0.y * scale);
    r.y = pack_hi_halves(p1.x * scale, p1.y * scale);
    r.z = pack_hi_halves(p2.x * scale, p2.y * scale);
    r.w = pack_hi_halves(p3.x * scale, p3.y * scale);
    return r;
}

// Four E2M1 codes (two bytes of a dword, BYTE and BYTE + 1) times
// 2^exp(cvt_scale) -> four bf16 in k order, exact.
template <int BYTE>
__device__ __forceinline__ s16x4 decode4_bf16_pow2(uint32_t codes, float cvt_scale) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, cvt_scale, BYTE);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, cvt_scale, BYTE + 1);
    const uint32_t ua = __builtin_bit_cast(uint32_t, a), ub = __builtin_bit_cast(uint32_t, b);
    s16x4 r;
    r[0] = (short)(ua & 0xFFFFu);
    r[1] = (short)(ua >> 16);
    r[2] = (short)(ub & 0xFFFFu);
    r[3] = (short)(ub >> 16);
    return r;
}

__device__ __forceinline__ s16x4 dwords_to_s16x4(uint32_t lo, uint32_t hi) {
    s16x4 r;
    r[0] = (short)(lo & 0xFFFFu);
    r[1] = (short)(lo >> 16);
    r[2] = (short)(hi & 0xFFFFu);
    r[3] = (short)(hi >> 16);
    return r;
}

__device__ __forceinline__ bf16x8 uint4_to_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---- activation element type: bf16 (F16 = false) or fp16 (F16 = true).
// X and Y share the type; weights decode to it exactly (e2m1 * e4m3 has at
// most 6 significant bits and lies in [2^-10, 2688], inside the normal range
// of both types), and the MFMAs take it with fp32 accumulation.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two exact fp32 values -> one dword of two 16-bit values (lo first).
template <bool F16>
__device__ __forceinline__ uint32_t pack_exact(float lo, float hi) {
    if constexpr (F16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
    else return pack_hi_halves(lo, hi);
}

// Eight E2M1 codes times a full fp32 scale -> eight values in k order, exact.
template <bool F16>
__device__ __forceinline__ uint4 decode8(uint32_t codes, float scale) {
    if constexpr (!F16) return decode8_bf16(codes, scale);
    const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
    const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
    const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
    const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
    uint4 r;
    r.x = pack_exact<true>(p0.x * scale, p0.y * scale);
    r.y = pack_exact<true>(p1.x * scale, p1.y * scale);
    r.z = pack_exact<true>(p2.x * scale, p2.y * scale);
    r.w = pack_exact<true>(p3.x * scale, p3.y * scale);
    return r;
}

// Eight E2M1 codes of one dword times a power-of-two scale (an E8M0 value,
// MXFP4), the scale applied inside the conversion: one operation per two
// values.  For every E8M0 byte this gives the bits decode8 gives (exact
// products; 2^-127 and overflow to infinity included), except the NaN code,
// which is NaN either way but of the other sign (checked over all 16 codes x
// 256 bytes on the device, bf16 and fp16).
template <bool F16>
__device__ __forceinline__ uint4 decode8_pow2(uint32_t codes, float scale) {
    if constexpr (F16)
        return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 0)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 1)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 2)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, scale, 3)));
    else
        return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3)));
}

// fp16 decode of E4M3-scaled codes in two operations per two values: the
// scale's power of two goes into the conversion (its exponent only), its
// significand factor (1.mmm; the whole scale for zero and NaN, see
// split_scale) multiplies the fp16 pairs.  e2m1 * 2^exp(s) and e2m1 * s lie in
// [2^-10, 2688] with at most 6 significant bits, so both are exact in fp16 and
// the values equal decode8<true>'s (NaN scales give NaN either way).
typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));
struct HalfScale {
    float cvt;    // operand of the conversion (its exponent is applied)
    f16x2v f;     // the significand factor, twice
};
__device__ __forceinline__ HalfScale half_scale(float s) {
    float cs, f;
    split_scale(s, cs, f);
    const _Float16 h = (_Float16)f;
    return HalfScale{cs, f16x2v{h, h}};
}
__device__ __forceinline__ uint4 decode8_f16_split(uint32_t codes, const HalfScale& h) {
    const f16x2v a = __builtin_bit_cast(f16x2v, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, h.cvt, 0)) * h.f;
    const f16x2v b = __builtin_bit_cast(f16x2v, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, h.cvt, 1)) * h.f;
    const f16x2v c = __builtin_bit_cast(f16x2v, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, h.cvt, 2)) * h.f;
    const f16x2v d = __builtin_bit_cast(f16x2v, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, h.cvt, 3)) * h.f;
    return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
                      __builtin_bit_cast(uint32_t, d));
}

// The GEMM kernels' decode of one code dword: E8M0 scales (MX) in the
// conversion, E4M3 scales by fp32 multiplies.
template <bool F16, bool MX>
__device__ __forceinline__ uint4 decode8_fmt(uint32_t codes, float scale) {
    if constexpr (MX) return decode8_pow2<F16>(codes, scale);
    else return decode8<F16>(codes, scale);
}

// Four E2M1 codes (bytes BYTE, BYTE + 1) times 2^exp(cvt_scale) -> four values, exact.
template <bool F16, int BYTE>
__device__ __forceinline__ s16x4 decode4_pow2(uint32_t codes, float cvt_scale) {
    if constexpr (!F16) return decode4_bf16_pow2<BYTE>(codes, cvt_scale);
    const uint32_t ua = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, cvt_scale, BYTE));
    const uint32_t ub =
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, cvt_scale, BYTE + 1));
    return dwords_to_s16x4(ua, ub);
}

// acc + A . B for one 16 x 16 x 32 step; a and b hold eight values each.
template <bool F16>
__device__ __forceinline__ f32x4 mma16(uint4 a, uint4 b, f32x4 acc) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc,
                                                      0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(uint4_to_bf16x8(a), uint4_to_bf16x8(b), acc, 0, 0, 0);
}

// acc + A . B in the 16-block 4 x 4 x 4 form (cbsz / abid broadcast controls).
template <bool F16, int CBSZ, int ABID>
__device__ __forceinline__ f32x4 mma4(s16x4 a, s16x4 b, f32x4 acc) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), acc, CBSZ,
                                                  ABID, 0);
    else
        return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, b, acc, CBSZ, ABID, 0);
}

// fp32 -> 16-bit output pattern, round to nearest even (NaN stays NaN;
// fp16 overflows to infinity).
template <bool F16>
__device__ __forceinline__ uint32_t round_out(float v) {
    if constexpr (F16) return __builtin_bit_cast(uint16_t, (_Float16)v);
    else return f32_to_bf16_rne(v);
}

// 16-bit activation pattern -> fp32 (exact).
template <bool F16>
__device__ __forceinline__ float act_to_f32(uint32_t h) {
    if constexpr (F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
    else return bf16_to_f32(h);
}

// MoE activations between FC1 and FC2, on values already rounded to the
// activation type (FC1's outputs), in fp32.  The standalone glue kernels and
// the FC1 epilogue (act below) share these, so the two paths agree bitwise.
//   gated SiLU: silu(gate) * up, silu(v) = v / (1 + e^-v);
//   squared ReLU (experts without a gate): max(h, 0)^2.
//
// Products that are then rounded to the output type pass through an empty
// asm statement as fp32 values: the backend otherwise folds a multiply and
// the following conversion to fp16 into one mixed-precision FMA
// (v_fma_mixlo_f16, which rounds the exact product once; contraction off
// does not stop it), in some kernels and not in others, so that two paths
// computing the same output would differ in the last bit now and then.
// Every output path thus rounds the fp32 product.
__device__ __forceinline__ float fp32_value(float v) {
    asm volatile("" : "+v"(v));
    return v;
}
__device__ __forceinline__ float silu_times(float gate, float up) {
    return fp32_value(gate / (1.0f + expf(-gate)) * up);
}
__device__ __forceinline__ float relu_squared(float h) {
    const float r = fmaxf(h, 0.0f);
    return fp32_value(r * r);
}
// g * acc of an epilogue, as an fp32 value (see above)
__device__ __forceinline__ float scale_acc(float g, float acc) { return fp32_value(g * acc); }

// What a grouped GEMM's epilogue writes (template parameter ACT):
//   kActNone     Y = RNE(g * acc);
//   kActSiluGlu  the blob's 16-row units alternate gate / up (nvfp4_repack_gated),
//                and output column 16 j + c is RNE(silu_times(h(2j, c), h(2j+1, c)))
//                with h(u, c) = RNE(g * acc) of unit u, column c: N / 2 columns;
//   kActRelu2    RNE(relu_squared(RNE(g * acc))).
constexpr int kActNone = 0, kActSiluGlu = 1, kActRelu2 = 2;

// fp32 pair -> bf16 (fp16 with F16) pair, round to nearest even with the
// hardware conversion (one instruction per pair; a NaN stays NaN), first
// value in the low half.
template <bool F16>
__device__ __forceinline__ uint32_t pack_round2(float a, float b) {
    if constexpr (F16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
    else return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// The pre-quant (AWQ) scale applied where an activation piece is loaded:
// eight activation values (a 16-byte piece, k ascending) times the eight
// scale values of the same k, each product rounded once to the activation
// type.  A product of two bf16 values, or of two fp16 values, is exact in
// fp32, so this is the correctly rounded RNE(X * s) of the definition.
template <bool F16>
__device__ __forceinline__ uint4 prescale8(uint4 x, uint4 s) {
    const uint32_t xd[4] = {x.x, x.y, x.z, x.w}, sd[4] = {s.x, s.y, s.z, s.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float a0, a1;
        if constexpr (F16) {
            a0 = act_to_f32<true>(xd[i] & 0xFFFFu) * act_to_f32<true>(sd[i] & 0xFFFFu);
            a1 = act_to_f32<true>(xd[i] >> 16) * act_to_f32<true>(sd[i] >> 16);
        } else {
            a0 = __uint_as_float(xd[i] << 16) * __uint_as_float(sd[i] << 16);
            a1 = __uint_as_float(xd[i] & 0xFFFF0000u) * __uint_as_float(sd[i] & 0xFFFF0000u);
        }
        o[i] = pack_round2<F16>(a0, a1);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// Streaming loads of weight codes and scales: every byte is read exactly
// once, so the loads are marked non-temporal and do not displace the
// activations (which are reused) from the caches.
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream_u4(const uint8_t* p) {
    const u32x4v t = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
    return make_uint4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ uint32_t load_stream_u16(const uint8_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
}
// Scale bytes of a 128-byte scale block: lanes 2i and 2i + 1 load the same
// dword (a dword load needs no zero extension, which spares the register
// copies the compiler otherwise inserts around 16-bit loads kept in flight
// across a loop).  The raw dword is kept in the prefetch ring and the lane's
// two bytes are selected only when the chunk is used (scale_pair), so no
// arithmetic touches a load result before its slot is consumed.
__device__ __forceinline__ uint32_t load_scale_dword(const uint8_t* block, int lane) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(block + ((lane >> 1) << 2)));
}
// The lane's two scale bytes (low byte = lower k) in bits 0..15 of the result.
__device__ __forceinline__ uint32_t scale_pair(uint32_t raw, int lane) { return raw >> ((lane & 1) << 4); }

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding:
// vmcnt in bits 3..0 and 15..14, expcnt 6..4, lgkmcnt 11..8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is six bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0) with the other counters left alone.
__device__ __forceinline__ void wait_lgkmcnt0() {
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

// A pointer the compiler must keep in scalar registers: every lane holds the
// same value, and passing it through readfirstlane stops the compiler from
// folding a per-lane offset into a loop-invariant 64-bit vector address.
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}

// Global scale as used in the epilogue: the stored value, or its correctly
// rounded fp32 reciprocal when it is stored as a divisor.
__device__ __forceinline__ float effective_global_scale(float stored, int is_divisor) {
    return is_divisor ? __fdiv_rn(1.0f, stored) : stored;
}

// Global scale of expert e; formats without one (MXFP4) pass no pointer: 1.
__device__ __forceinline__ float global_scale_at(const float* gs, int e, int is_divisor) {
    return gs ? effective_global_scale(gs[e], is_divisor) : 1.0f;
}

}  // namespace nvfp4
