/*
 * CPU oracle for the W4A16 NVFP4 matrix multiply.  TEST INFRASTRUCTURE ONLY:
 * nothing on the product path may include, link or call this file; only the
 * tests, the smoke check and the benchmark's CPU-baseline leg use it.
 *
 * What it computes (plain definitions, fp64, no blocking or reordering):
 *
 *   T[n,k]  = e2m1(code(n,k)) * e4m3(S[n, k/16])                 (weight tile)
 *   g       = flag ? fp32(1/stored) : stored                      (global scale)
 *   X'[m,k] = pre ? RNE_bf16(X[m,k] * s[k]) : X[m,k]              (pre-quant scale)
 *   Y[m,n]  = g * sum_{k=0..K-1} X'[m,k] * T[n,k]                 (never rounded)
 *
 * Sources (all on the pages "Support nvfp4 w4a16 on sm120", "Support
 * Nemotron-H nvfp4 ckpt on Hopper", the SGLang compressed-tensors NVFP4
 * weight-only page and "Apply the NVFP4_AWQ pre-quant scale in MegaMoE
 * CuteDSL"):
 *  - packed FP4 weights with one FP8 scale per group of 16 along K and a
 *    per-tensor global scale: sm120 page, Summary; Hopper page, Walkthrough
 *    table row "Triton NVFP4 dequantization kernels" (E2M1 codebook lookup,
 *    per-block FP8 scale); SGLang page, Motivation (group size 16, E4M3 group
 *    scales, NVFP4 always has a real global scale).
 *  - the global scale stored as a divisor must be inverted: SGLang page,
 *    Modifications, the note on global-scale inversion.
 *  - the per-channel pre-quant scale multiplies the BF16 activation before
 *    the GEMM and the product stays BF16: MegaMoE page, Description ("Fix")
 *    and its commit messages.
 *  - the active-expert-only MoE form: Hopper page, Walkthrough table rows
 *    for the MoE path.
 * The E2M1 value set and bit layout follow the OCP Microscaling (MX) format
 * specification v1.0, section 5.3.3 (FP4 E2M1); E4M3 follows the OCP 8-bit
 * floating point specification (OFP8) v1.0, E4M3 column of its format table.
 * Nibble order (low nibble = even k) is a reading the pages leave open.
 *
 * MXFP4 weight-only (the *_fmt functions with fmt = 1): the same E2M1 codes
 * with one E8M0 scale per group of 32 along K and no global scale (SGLang
 * page, Modifications: the paragraph on MXFP4 names group_blocks == 2, E8M0
 * scales and the missing global_scale as what sets it apart from NVFP4).
 *   T[n,k] = e2m1(code(n,k)) * e8m0(S[n, k/32]),  Y[m,n] = sum_k X'[m,k] T[n,k]
 * E8M0 follows the OCP MX specification v1.0 (section 5.4.1): 2^(e-127) for
 * e = 0..254, NaN for 255, no sign and no zero.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (fp contraction off
 * so every product and sum is a separately rounded fp64 operation).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>

/* E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
 * exponent 0 is subnormal: value = m * 2^-1; otherwise 2^(e-1) * (1 + m/2). */
double oracle_e2m1(int code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? ldexp((double)m, -1) : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* E4M3 (OCP "FN" variant): bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0
 * mantissa.  exponent 0 is subnormal: m * 2^-9.  Exponent 15 with mantissa 7
 * is NaN; there is no infinity. */
double oracle_e4m3(int byte) {
    int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp((double)m, -9);
    else mag = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* E8M0 (OCP MX scale): an unsigned biased exponent, 2^(e-127); 0xFF is NaN. */
double oracle_e8m0(int byte) {
    if ((byte & 255) == 255) return NAN;
    return ldexp(1.0, (byte & 255) - 127);
}

/* Weight (n, k) of one expert in format fmt: 0 = NVFP4 (E4M3 scale per 16 k),
 * 1 = MXFP4 (E8M0 scale per 32 k). */
static double weight_value(const uint8_t* w, int64_t ld_w, const uint8_t* s, int64_t ld_s, int64_t n, int64_t k,
                           int fmt);

/* bf16 bit pattern -> value (bf16 is the upper half of an IEEE binary32). */
double oracle_bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round an fp64 value to the nearest bf16 value, ties to even (8 significant
 * bits, binary32 exponent range incl. subnormals down to 2^-133; overflow to
 * infinity).  Returned as the fp64 value of that bf16. */
double oracle_round_bf16(double v) {
    if (v == 0.0 || isnan(v) || isinf(v)) return v;
    int e;
    frexp(v, &e);                 /* |v| = f * 2^e, f in [0.5, 1) */
    int q = e - 8;                /* spacing of bf16 values near v */
    if (q < -133) q = -133;       /* subnormal spacing */
    double r = ldexp(nearbyint(ldexp(v, -q)), q);   /* default mode: ties-to-even */
    double maxbf = ldexp(255.0, 120);               /* (2 - 2^-7) * 2^127 */
    if (fabs(r) > maxbf) return v > 0 ? INFINITY : -INFINITY;
    return r;
}

/* Global scale: the multiplier as the GEMM uses it.  When the stored value is
 * a divisor it is inverted and rounded to fp32 (round to nearest even). */
double oracle_global_scale(float stored, int is_divisor) {
    if (!is_divisor) return (double)stored;
    return (double)(float)(1.0 / (double)stored);
}

/* Code of weight (n, k): low nibble of byte k/2 holds the even k. */
static int code_at(const uint8_t* w, int64_t ld_w, int64_t n, int64_t k) {
    return (w[n * ld_w + (k >> 1)] >> (4 * (k & 1))) & 15;
}

static double weight_value(const uint8_t* w, int64_t ld_w, const uint8_t* s, int64_t ld_s, int64_t n, int64_t k,
                           int fmt) {
    if (fmt == 1) return oracle_e2m1(code_at(w, ld_w, n, k)) * oracle_e8m0(s[n * ld_s + (k >> 5)]);
    return oracle_e2m1(code_at(w, ld_w, n, k)) * oracle_e4m3(s[n * ld_s + (k >> 4)]);
}

/* Weight tile T[n,k] in fp64 for one expert, written to out[N*K]. */
void oracle_dequant_fmt(const uint8_t* w, int64_t ld_w, const uint8_t* s, int64_t ld_s,
                        int64_t N, int64_t K, int fmt, double* out) {
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            out[n * K + k] = weight_value(w, ld_w, s, ld_s, n, k, fmt);
}

void oracle_dequant(const uint8_t* w, int64_t ld_w, const uint8_t* s, int64_t ld_s,
                    int64_t N, int64_t K, double* out) {
    oracle_dequant_fmt(w, ld_w, s, ld_s, N, K, 0, out);
}

/* X'[m,k] in fp64: the activation, times the pre-quant scale rounded back to
 * bf16 when a pre-scale is given.  out[M*K]. */
void oracle_activation(const uint16_t* x, int64_t ld_x, const uint16_t* pre, int64_t M, int64_t K,
                       double* out) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            double v = oracle_bf16_value(x[m * ld_x + k]);
            if (pre) v = oracle_round_bf16(v * oracle_bf16_value(pre[k]));
            out[m * K + k] = v;
        }
}

/* Dense: Y[m,n] = g * sum_k X'[m,k] T[n,k], k ascending, fp64, out[M*N].
 * Parallel over n: each thread decodes row n of T once into tbuf, then forms
 * one plain sequential sum per output.  xbuf[M*K] and tbuf[threads*K] are
 * caller-provided scratch. */
/* fmt as for oracle_dequant_fmt; MXFP4 has no global scale (g = 1). */
void oracle_gemm_fmt(const uint16_t* x, int64_t ld_x, const uint16_t* pre,
                     const uint8_t* w, int64_t ld_w, const uint8_t* s, int64_t ld_s,
                     float g_stored, int g_is_divisor, int fmt,
                     int64_t M, int64_t N, int64_t K, double* xbuf, double* tbuf, int threads,
                     double* out) {
    double g = fmt == 1 ? 1.0 : oracle_global_scale(g_stored, g_is_divisor);
    oracle_activation(x, ld_x, pre, M, K, xbuf);
#pragma omp parallel num_threads(threads)
    {
        double* t = tbuf + (int64_t)omp_get_thread_num() * K;
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < K; ++k)
                t[k] = weight_value(w, ld_w, s, ld_s, n, k, fmt);
            for (int64_t m = 0; m < M; ++m) {
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k) acc += xbuf[m * K + k] * t[k];
                out[m * N + n] = g * acc;
            }
        }
    }
}

void oracle_gemm(const uint16_t* x, int64_t ld_x, const uint16_t* pre,
                 const uint8_t* w, int64_t ld_w, const uint8_t* s, int64_t ld_s,
                 float g_stored, int g_is_divisor,
                 int64_t M, int64_t N, int64_t K, double* xbuf, double* tbuf, int threads,
                 double* out) {
    oracle_gemm_fmt(x, ld_x, pre, w, ld_w, s, ld_s, g_stored, g_is_divisor, 0, M, N, K, xbuf, tbuf, threads, out);
}

int oracle_max_threads(void) { return omp_get_max_threads(); }

/* One output of the dense form, computed on its own from the raw inputs. */
static double gemm_one(const uint16_t* x, int64_t ld_x, const uint16_t* pre,
                       const uint8_t* w, int64_t ld_w, const uint8_t* s, int64_t ld_s,
                       float g_stored, int g_is_divisor, int fmt, int64_t K, int64_t m, int64_t n) {
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double xv = oracle_bf16_value(x[m * ld_x + k]);
        if (pre) xv = oracle_round_bf16(xv * oracle_bf16_value(pre[k]));
        acc += xv * weight_value(w, ld_w, s, ld_s, n, k, fmt);
    }
    return (fmt == 1 ? 1.0 : oracle_global_scale(g_stored, g_is_divisor)) * acc;
}

double oracle_gemm_one(const uint16_t* x, int64_t ld_x, const uint16_t* pre,
                       const uint8_t* w, int64_t ld_w, const uint8_t* s, int64_t ld_s,
                       float g_stored, int g_is_divisor, int64_t K, int64_t m, int64_t n) {
    return gemm_one(x, ld_x, pre, w, ld_w, s, ld_s, g_stored, g_is_divisor, 0, K, m, n);
}

/* Sampled dense outputs: out[i] = Y[rows[i], cols[i]]. */
void oracle_gemm_sampled_fmt(const uint16_t* x, int64_t ld_x, const uint16_t* pre,
                             const uint8_t* w, int64_t ld_w, const uint8_t* s, int64_t ld_s,
                             float g_stored, int g_is_divisor, int fmt, int64_t K,
                             const int64_t* rows, const int64_t* cols, int64_t count, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        out[i] = gemm_one(x, ld_x, pre, w, ld_w, s, ld_s, g_stored, g_is_divisor, fmt, K, rows[i], cols[i]);
}

void oracle_gemm_sampled(const uint16_t* x, int64_t ld_x, const uint16_t* pre,
                         const uint8_t* w, int64_t ld_w, const uint8_t* s, int64_t ld_s,
                         float g_stored, int g_is_divisor, int64_t K,
                         const int64_t* rows, const int64_t* cols, int64_t count, double* out) {
    oracle_gemm_sampled_fmt(x, ld_x, pre, w, ld_w, s, ld_s, g_stored, g_is_divisor, 0, K, rows, cols, count, out);
}

/* Expert owning row r: the e with offsets[e] <= r < offsets[e+1] (-1 if none). */
static int64_t expert_of_row(const int32_t* offsets, int64_t E, int64_t r) {
    for (int64_t e = 0; e < E; ++e)
        if (offsets[e] <= r && r < offsets[e + 1]) return e;
    return -1;
}

/* Grouped (MoE) form.  Rows [offsets[e], offsets[e+1]) of X belong to expert e
 * and use that expert's weights w + e*N*ld_w, scales s + e*N*ld_s and global
 * scale g_stored[e]; the pre-scale (if any) is shared by all experts.
 * out[R*N]; rows outside every expert's range are left untouched. */
void oracle_grouped_gemm_fmt(const uint16_t* x, int64_t ld_x, const int32_t* offsets, const uint16_t* pre,
                             const uint8_t* w, int64_t ld_w, const uint8_t* s, int64_t ld_s,
                             const float* g_stored, int g_is_divisor, int fmt,
                             int64_t R, int64_t E, int64_t N, int64_t K, double* out) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < R; ++r) {
        int64_t e = expert_of_row(offsets, E, r);
        if (e < 0) continue;
        const uint8_t* we = w + e * N * ld_w;
        const uint8_t* se = s + e * N * ld_s;
        for (int64_t n = 0; n < N; ++n)
            out[r * N + n] = gemm_one(x, ld_x, pre, we, ld_w, se, ld_s, fmt == 1 ? 1.0f : g_stored[e], g_is_divisor,
                                      fmt, K, r, n);
    }
}

void oracle_grouped_gemm(const uint16_t* x, int64_t ld_x, const int32_t* offsets, const uint16_t* pre,
                         const uint8_t* w, int64_t ld_w, const uint8_t* s, int64_t ld_s,
                         const float* g_stored, int g_is_divisor,
                         int64_t R, int64_t E, int64_t N, int64_t K, double* out) {
    oracle_grouped_gemm_fmt(x, ld_x, offsets, pre, w, ld_w, s, ld_s, g_stored, g_is_divisor, 0, R, E, N, K, out);
}

/* Sampled grouped outputs: out[i] = Y[rows[i], cols[i]] (NaN if the row has no expert). */
void oracle_grouped_gemm_sampled(const uint16_t* x, int64_t ld_x, const int32_t* offsets, const uint16_t* pre,
                                 const uint8_t* w, int64_t ld_w, const uint8_t* s, int64_t ld_s,
                                 const float* g_stored, int g_is_divisor, int64_t E, int64_t N, int64_t K,
                                 const int64_t* rows, const int64_t* cols, int64_t count, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        int64_t e = expert_of_row(offsets, E, rows[i]);
        if (e < 0) { out[i] = NAN; continue; }
        out[i] = gemm_one(x, ld_x, pre, w + e * N * ld_w, ld_w, s + e * N * ld_s, ld_s,
                          g_stored[e], g_is_divisor, 0, K, rows[i], cols[i]);
    }
}
