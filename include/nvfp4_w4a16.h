/*
 * nvfp4_w4a16.h -- C ABI of the MI355X (gfx950) W4A16 NVFP4 GEMM library.
 *
 * The operation (dense form):
 *
 *     Y[M,N] = g * (X[M,K] (.) s_pre[K]) . dequant(W)^T,
 *     dequant(W)[n,k] = e2m1(code(n,k)) * e4m3(S[n, k/16])
 *
 * W is packed FP4 (E2M1, two codes per byte along K) with one FP8 (E4M3)
 * scale per 16 consecutive K of a row and one fp32 global scale g; the
 * activation X and the output Y stay bf16 (fp16 in the *_f16 calls at the
 * end of this file).  Where the operation is defined:
 *   - packed FP4 weights + per-group FP8 scales + bf16/fp16 activations:
 *     "Support nvfp4 w4a16 on sm120", Summary;
 *   - E2M1 codebook lookup times a per-block FP8 scale and a per-tensor
 *     global scale (linear and active-expert-only MoE dequant):
 *     "Support Nemotron-H nvfp4 ckpt on Hopper", Walkthrough, Changes table;
 *   - group size 16 with E4M3 group scales and a real global scale, and the
 *     divisor-stored global scale that must be inverted: SGLang
 *     compressed-tensors NVFP4 weight-only page, Motivation and Modifications;
 *   - the per-channel pre-quant scale multiplies the bf16 activation before
 *     the GEMM (product kept in bf16), and a zero-token call launches no
 *     kernel: "Apply the NVFP4_AWQ pre-quant scale in MegaMoE CuteDSL",
 *     Description.
 * The E2M1 values and the low-nibble-is-even-k order follow the OCP MX
 * format; E4M3 is the OCP E4M3FN encoding (bias 7, max 448, NaN = 0x7F/0xFF).
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library allocates nothing and keeps no pointer after it returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *     Every call is asynchronous on that stream and never synchronises the
 *     host, so it can be captured into a HIP graph.
 *   - Arguments are checked on the host before anything is launched; on an
 *     error nothing has been enqueued and nvfp4_last_error() (thread-local)
 *     names the argument and the violated constraint.
 *   - Device-resident values (global scales, expert offsets) are not read by
 *     the host and are not checked: offsets that are not a non-decreasing
 *     sequence from 0 to R are undefined behaviour; a stored divisor of 0
 *     gives non-finite outputs.
 *   - bf16 values are IEEE binary32 upper halves; all rounding to bf16 is
 *     round-to-nearest-even.
 */
#ifndef NVFP4_W4A16_H
#define NVFP4_W4A16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NVFP4_OK = 0,
    NVFP4_ERR_INVALID_ARG = 1,     /* a size, pointer or flag is invalid */
    NVFP4_ERR_ALIGNMENT = 2,       /* a pointer or leading dimension is misaligned */
    NVFP4_ERR_BUFFER_TOO_SMALL = 3,/* out_bytes / workspace_bytes below the size query */
    NVFP4_ERR_HIP = 4              /* the HIP runtime reported an error at launch */
} nvfp4_status;

/* Message of the last failed call on this thread ("" if none). */
const char* nvfp4_last_error(void);

/* Zero sizes: a call with no rows (M, R or T == 0) or no output columns
 * (N == 0) checks its other arguments, returns NVFP4_OK and launches nothing
 * (a zero-token chunk launches no kernel: "Apply the NVFP4_AWQ pre-quant
 * scale in MegaMoE CuteDSL", Description). */

/* ---------------------------------------------------------------- repack --
 * One-time re-tiling of canonical weights into the layout the GEMM kernels
 * stream (a step the pages perform as the Marlin weight transformation with
 * K/N padding: "Support nvfp4 w4a16 on sm120", Changes, Linear).
 *
 * Canonical input, E experts (E = 1 for a dense layer):
 *   w_packed : uint8 [E][N][ld_w], row (e,n) at w_packed + (e*N + n)*ld_w;
 *              byte j holds codes k = 2j (low nibble) and k = 2j+1 (high
 *              nibble); ld_w >= K/2.
 *   w_scale  : uint8 [E][N][ld_s] E4M3 bytes, row (e,n) at w_scale +
 *              (e*N + n)*ld_s; byte b scales k in [16b, 16b+16); ld_s >= K/16.
 * Output: `out`, nvfp4_repack_bytes(E,N,K) bytes, 16-byte aligned.  The blob
 * is pure derived state: repacking the same input again gives the same bytes,
 * and the canonical input is never modified.  N is padded to a multiple of
 * 16 and K to a multiple of 128 with zero codes and zero scales.  N == 0
 * needs 0 bytes and launches nothing.
 * Errors: E < 1, N < 0, K < 16, K % 16 != 0, ld_w < K/2, ld_s < K/16, NULL
 * pointer (N > 0) -> INVALID_ARG; out not 16-byte aligned -> ALIGNMENT;
 * out_bytes too small -> BUFFER_TOO_SMALL. */
int64_t nvfp4_repack_bytes(int64_t E, int64_t N, int64_t K); /* < 0 if invalid */
nvfp4_status nvfp4_repack(const uint8_t* w_packed, int64_t ld_w, const uint8_t* w_scale, int64_t ld_s,
                          int64_t E, int64_t N, int64_t K, void* out, int64_t out_bytes, void* stream);

/* ------------------------------------------------------------ dense GEMM --
 * Y = RNE_bf16(g * sum_k X'[m,k] * dequant(W)[n,k]) with
 *   X'[m,k] = pre_scale ? RNE_bf16(X[m,k] * pre_scale[k]) : X[m,k]
 *   g       = global_scale_is_divisor ? fp32(1 / *global_scale) : *global_scale
 * (the inversion happens at use, in the epilogue; *global_scale is never
 * rewritten).  The pre-quant scale is applied where the kernels load the
 * activation; X' is never written to memory.  Accumulation is fp32; the
 * summation order is fixed, so results are bitwise reproducible run to run.
 *   x         : bf16 [M][ld_x] (16-byte aligned, K <= ld_x <= 2^23, ld_x % 8 == 0)
 *   pre_scale : bf16 [K] (16-byte aligned) or NULL
 *   w_repacked: output of nvfp4_repack with E = 1 and the same N, K
 *   global_scale: device pointer to one fp32
 *   y         : bf16 [M][ld_y] (2-byte aligned, ld_y >= N)
 *   workspace : device scratch of nvfp4_w4a16_gemm_workspace_bytes(M,N,K)
 *               bytes, 256-byte aligned (may be NULL when that is 0; it is 0
 *               unless the call's kernel splits K across workgroups).  It
 *               holds split-K partial sums and arrival counters; it must be
 *               zero-filled before its first use; every call leaves the
 *               counters zero again, so one workspace can serve any number
 *               of calls issued one after another.  Calls that may overlap
 *               in time (other streams) need their own workspace.  The size
 *               covers every kernel variant that takes the shape.
 * M == 0 or N == 0 returns NVFP4_OK without launching anything.
 * Errors: M < 0, N < 0, K < 16, K % 16 != 0, ld_x < K, ld_x > 2^23, ld_y < N, NULL
 * x / w_repacked / global_scale / y (x and y may be NULL when M == 0) ->
 * INVALID_ARG; misaligned x, pre_scale, w_repacked, y or workspace, or
 * ld_x % 8 != 0 -> ALIGNMENT; workspace smaller than this call needs ->
 * BUFFER_TOO_SMALL. */
int64_t nvfp4_w4a16_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
nvfp4_status nvfp4_w4a16_gemm(const void* x, int64_t ld_x, const void* pre_scale, const void* w_repacked,
                              const float* global_scale, int global_scale_is_divisor,
                              void* y, int64_t ld_y, int64_t M, int64_t N, int64_t K,
                              void* workspace, int64_t workspace_bytes, void* stream);

/* ---------------------------------------------------------- grouped GEMM --
 * Active-expert-only MoE form ("Support Nemotron-H nvfp4 ckpt on Hopper",
 * Walkthrough, Changes table, MoE rows: only experts that received tokens
 * are dequantised).  Rows of x are grouped by expert: rows
 * [expert_offsets[e], expert_offsets[e+1]) use expert e's weights and global
 * scale; every other row of y is left untouched.  Experts with no rows read
 * no weight bytes.  The tile schedule is built on the device from
 * expert_offsets, with no host synchronisation.
 *   x             : bf16 [R][ld_x] (same alignment rules as the dense form)
 *   expert_offsets: device int32 [E+1], offsets[0] = 0, non-decreasing, offsets[E] = R
 *   pre_scale     : bf16 [K] shared by all experts, or NULL
 *   w_repacked    : output of nvfp4_repack with this E, N, K
 *   global_scales : device fp32 [E]
 *   y             : bf16 [R][ld_y]
 *   workspace     : as for the dense form, nvfp4_w4a16_grouped_gemm_workspace_bytes
 *                   bytes (0: the grouped kernels never split K)
 * R == 0 or N == 0 returns NVFP4_OK without launching anything.
 * Errors as for the dense form, plus E < 1 -> INVALID_ARG. */
int64_t nvfp4_w4a16_grouped_gemm_workspace_bytes(int64_t R, int64_t E, int64_t N, int64_t K);
nvfp4_status nvfp4_w4a16_grouped_gemm(const void* x, int64_t ld_x, const int32_t* expert_offsets,
                                      const void* pre_scale, const void* w_repacked,
                                      const float* global_scales, int global_scale_is_divisor,
                                      void* y, int64_t ld_y, int64_t R, int64_t E, int64_t N, int64_t K,
                                      void* workspace, int64_t workspace_bytes, void* stream);

/* ------------------------------------------------------------ MoE glue --
 * The steps either side of the grouped GEMM in a mixture-of-experts layer
 * whose experts take only the tokens routed to them ("Support Nemotron-H
 * nvfp4 ckpt on Hopper", Changes table, MoE W4A16 execution path: the layer
 * dispatches tokens to their active experts and runs a fused MoE over them;
 * the gated FC1 holds the gate and up projections together, the SGLang
 * compressed-tensors NVFP4 weight-only page, review discussion of the w13
 * sizing for gated and non-gated experts).  A layer of T tokens, top-k
 * routing over E experts, hidden size Hd and expert width I runs as
 *   nvfp4_moe_route -> nvfp4_w4a16_grouped_gemm_gather (FC1, N = 2 I)
 *   -> nvfp4_moe_silu_mul -> nvfp4_w4a16_grouped_gemm (FC2, K = I, N = Hd)
 *   -> nvfp4_moe_combine,
 * or with the activation in FC1's epilogue (one step fewer, and FC1 writes
 * I columns instead of 2 I):
 *   nvfp4_moe_route -> nvfp4_moe_fc1 (gated weights from nvfp4_repack_gated)
 *   -> nvfp4_w4a16_grouped_gemm (FC2) -> nvfp4_moe_combine,
 * every step stream-ordered, with no host synchronisation.
 *
 * Routing: topk_ids is device int32 [T][k] (row t: the k experts of token
 * t, values in [0, E); the caller keeps them distinct per token).  The
 * (token, slot) pairs p = t*k + j are ordered by expert, ties in pair order
 * (a stable sort), which defines the grouped rows:
 *   expert_offsets[e] : first grouped row of expert e; [E] = T*k,
 *   row_token[r]      : token of grouped row r,              [T*k]
 *   token_row[p]      : grouped row of pair p = t*k + j,     [T*k]
 * all device int32, 4-byte aligned.  The result does not depend on timing.
 * workspace: nvfp4_moe_route_workspace_bytes(T, k, E) bytes of device
 * scratch (4-byte aligned, no initial contents needed; calls that may
 * overlap in time need their own).  Ids outside [0, E) give undefined (but
 * in-bounds) results.  T == 0 returns NVFP4_OK without launching anything
 * (the outputs are not written).
 * Errors: T < 0, E < 1 or E > 1024, k < 1 or k > E, T*k >= 2^31, a NULL
 * array -> INVALID_ARG; misaligned array or workspace -> ALIGNMENT;
 * workspace too small -> BUFFER_TOO_SMALL. */
int64_t nvfp4_moe_route_workspace_bytes(int64_t T, int64_t k, int64_t E);   /* < 0 if invalid */
nvfp4_status nvfp4_moe_route(const int32_t* topk_ids, int64_t T, int64_t k, int64_t E, int32_t* expert_offsets,
                             int32_t* row_token, int32_t* token_row, void* workspace, int64_t workspace_bytes,
                             void* stream);

/* Grouped GEMM whose activation rows are gathered on the fly: grouped row r
 * reads row row_token[r] of x (bf16 [T][ld_x], the tokens in their own
 * order), so the expert-ordered copy of the activation is never written.
 * Otherwise as nvfp4_w4a16_grouped_gemm (y is in grouped row order; the
 * pre-scale, if any, applies to the T token rows).  row_token values must be
 * in [0, T) (device data, not checked: undefined behaviour otherwise).
 * Errors: as for nvfp4_w4a16_grouped_gemm, plus T < 0, R > 0 with T == 0,
 * T * ld_x >= 2^31, row_token NULL (R > 0) -> INVALID_ARG; row_token not
 * 4-byte aligned -> ALIGNMENT. */
int64_t nvfp4_w4a16_grouped_gemm_gather_workspace_bytes(int64_t T, int64_t R, int64_t E, int64_t N, int64_t K);
nvfp4_status nvfp4_w4a16_grouped_gemm_gather(const void* x, int64_t ld_x, int64_t T, const int32_t* row_token,
                                             const int32_t* expert_offsets, const void* pre_scale,
                                             const void* w_repacked, const float* global_scales,
                                             int global_scale_is_divisor, void* y, int64_t ld_y, int64_t R,
                                             int64_t E, int64_t N, int64_t K, void* workspace,
                                             int64_t workspace_bytes, void* stream);

/* Gated SiLU between FC1 and FC2: h is bf16 [R][ld_h] holding the gate
 * projection in columns [0, I) and the up projection in [I, 2I) (the w13
 * order, gate first); a[r][i] = RNE_bf16(silu(h[r][i]) * h[r][I + i]) with
 * silu(v) = v / (1 + exp(-v)) evaluated in fp32.  a is bf16 [R][ld_a].
 * Errors: R < 0, I < 1, ld_h < 2I, ld_a < I, NULL (R > 0) -> INVALID_ARG;
 * odd addresses -> ALIGNMENT. */
nvfp4_status nvfp4_moe_silu_mul(const void* h, int64_t ld_h, int64_t R, int64_t I, void* a, int64_t ld_a,
                                void* stream);

/* Non-gated squared ReLU for experts without a gate projection (the SGLang
 * compressed-tensors NVFP4 weight-only page, review discussion: non-gated
 * relu2 experts hold one FC1 projection): a[r][i] = RNE_bf16(max(h[r][i], 0)^2)
 * evaluated in fp32; h is bf16 [R][ld_h] with I columns, a bf16 [R][ld_a].
 * Errors: R < 0, I < 1, ld_h < I, ld_a < I, NULL (R > 0) -> INVALID_ARG; odd
 * addresses -> ALIGNMENT. */
nvfp4_status nvfp4_moe_relu2(const void* h, int64_t ld_h, int64_t R, int64_t I, void* a, int64_t ld_a, void* stream);

/* Gated FC1 weights in the layout the fused FC1 reads.  The pages name two
 * orders for the fused gate / up weight: gate first (SGLang's w13, the w1
 * rows then the w3 rows: the SGLang compressed-tensors NVFP4 weight-only page,
 * review discussion) and up first (TensorRT-LLM's w3_w1 / fc31: the inline
 * review comments on "Support Nemotron-H nvfp4 ckpt on Hopper" and the
 * Description of "Apply the NVFP4_AWQ pre-quant scale in MegaMoE CuteDSL").
 * Input: canonical NVFP4 weights of E experts with 2 I rows each (as
 * nvfp4_repack, N = 2 I), rows [0, I) the gate projection and [I, 2 I) the
 * up projection when up_first = 0, the other way round when up_first = 1.
 * Output: nvfp4_repack_gated_bytes(E, I, K) bytes (= nvfp4_repack_bytes(E,
 * 2 I, K)), 16-byte aligned, whose 16-row units alternate gate / up: unit 2 j
 * holds gate rows 16 j .. 16 j + 15 and unit 2 j + 1 the up rows of the same
 * columns.  It is meant for nvfp4_moe_fc1 only.
 * Errors: as nvfp4_repack, plus I < 0 or I not a multiple of 16, up_first not
 * 0 or 1 -> INVALID_ARG. */
int64_t nvfp4_repack_gated_bytes(int64_t E, int64_t I, int64_t K); /* < 0 if invalid */
nvfp4_status nvfp4_repack_gated(const uint8_t* w_packed, int64_t ld_w, const uint8_t* w_scale, int64_t ld_s,
                                int64_t E, int64_t I, int64_t K, int up_first, void* out, int64_t out_bytes,
                                void* stream);

/* FC1 with its activation applied in the GEMM's epilogue, so the 2 I-wide
 * FC1 output is never written:
 *   NVFP4_MOE_SILU_GLU: w_fc1 from nvfp4_repack_gated (E experts, I, K);
 *     a[r][i] = RNE_bf16(silu(h_gate) * h_up) with h = RNE_bf16(g_e * acc)
 *     of the gate and up columns i: bitwise what nvfp4_w4a16_grouped_gemm
 *     (gather) followed by nvfp4_moe_silu_mul gives on the canonical weights;
 *   NVFP4_MOE_RELU2: w_fc1 from nvfp4_repack (E, N = I, K); a[r][i] =
 *     RNE_bf16(max(h, 0)^2), h = RNE_bf16(g_e * acc): bitwise the grouped GEMM
 *     followed by nvfp4_moe_relu2.
 * Rows: with row_token, grouped row r reads token row row_token[r] of x
 * (bf16 [T][ld_x]) as in nvfp4_w4a16_grouped_gemm_gather; with row_token
 * NULL, x holds the R grouped rows (T must equal R).  a is bf16 [R][ld_a] in
 * grouped row order; expert_offsets, pre_scale, global_scales and the
 * divisor flag as in nvfp4_w4a16_grouped_gemm.  No workspace.
 * Errors: as nvfp4_w4a16_grouped_gemm_gather (with N = 2 I or I), plus an
 * unknown activation, I < 0, I not a multiple of 16 (gated), ld_a < I,
 * row_token NULL with T != R -> INVALID_ARG. */
enum { NVFP4_MOE_SILU_GLU = 1, NVFP4_MOE_RELU2 = 2 };
nvfp4_status nvfp4_moe_fc1(const void* x, int64_t ld_x, int64_t T, const int32_t* row_token,
                           const int32_t* expert_offsets, const void* pre_scale, const void* w_fc1,
                           const float* global_scales, int global_scale_is_divisor, int activation, void* a,
                           int64_t ld_a, int64_t R, int64_t E, int64_t I, int64_t K, void* stream);

/* Test export: one grouped GEMM (activation 0: plain output, N columns) or
 * fused FC1 (activation NVFP4_MOE_SILU_GLU on a gated blob, N = 2 I and I
 * output columns; NVFP4_MOE_RELU2) on a chosen kernel, so that the kernels
 * can be checked against each other on the same inputs: variant 0 the
 * automatic choice, 1 the small-M kernel, 2 the tile kernel (64-row tiles),
 * 3 the MFMA-bound kernel (256-row tiles per expert).  Rows as in
 * nvfp4_moe_fc1 (row_token NULL: x holds the R grouped rows, T = R); f16:
 * fp16 activations and output; mx: an MXFP4 blob (mxfp4_repack; the global
 * scales are then not read and may be NULL); no workspace.  Errors: as the grouped GEMM,
 * plus an unknown activation or variant, N not a multiple of 32 with the
 * gated activation, mx not 0 or 1, and for variant 3 a blob of 2 GiB of
 * codes or more or NVFP4_MOE_RELU2 (the tile kernel serves it) -> INVALID_ARG. */
nvfp4_status nvfp4_w4a16_grouped_gemm_variant(const void* x, int64_t ld_x, int64_t T, const int32_t* row_token,
                                              const int32_t* expert_offsets, const void* pre_scale, const void* w,
                                              const float* global_scales, int global_scale_is_divisor, int activation,
                                              void* y, int64_t ld_y, int64_t R, int64_t E, int64_t N, int64_t K,
                                              int variant, int f16, int mx, void* stream);

/* Top-k weighted combine back to token order: out[t][c] =
 * RNE_bf16(sum_{j=0..k-1} topk_weights[t*k + j] * y[token_row[t*k + j]][c]),
 * accumulated in fp32 in slot order.  y: bf16 [R][ld_y] (FC2 output in
 * grouped row order), token_row: from nvfp4_moe_route, topk_weights: device
 * fp32 [T][k], out: bf16 [T][ld_o].
 * Errors: T < 0, k < 1, H < 1, ld_y < H, ld_o < H, NULL (T > 0) ->
 * INVALID_ARG; misaligned pointer -> ALIGNMENT. */
nvfp4_status nvfp4_moe_combine(const void* y, int64_t ld_y, const int32_t* token_row, const float* topk_weights,
                               int64_t T, int64_t k, int64_t H, void* out, int64_t ld_o, void* stream);

/* --------------------------------------------------------- test exports --
 * Decode a repacked blob back to bf16 [E][N][ld_out] in canonical order with
 * the same device decode the GEMM kernels use (no global scale applied):
 * out[e][n][k] = RNE_bf16(e2m1(code) * e4m3(scale)), which is exact.
 * Errors: as for repack, ld_out < K -> INVALID_ARG. */
nvfp4_status nvfp4_dequant_bf16(const void* w_repacked, int64_t E, int64_t N, int64_t K,
                                void* out, int64_t ld_out, void* stream);

/* Dense GEMM with the kernel variant forced instead of chosen from M:
 *   variant 0 = automatic (same as nvfp4_w4a16_gemm),
 *   variant 1 = small-M kernel (M <= 16 only; larger M -> INVALID_ARG),
 *   variant 2 = tile kernel (any M),
 *   variant 3 = MFMA-bound kernel (any M; launched as one or two kernels),
 *   variant 4 = activation-resident kernel: M <= 16, K <= 32768 (K split
 *               across workgroups beyond 4096) and
 *               ceil(N / 16) * ceil(K / 4096) <= 2048; otherwise INVALID_ARG,
 *   variant 5 = MFMA-bound kernel with every 256 x 256 tile run as four
 *               64-row workgroups (several then share a compute unit).
 * The automatic choice takes the small-M kernel up to 4 rows, the
 * activation-resident kernel for 5..16 rows where it applies, the MFMA-bound
 * kernel for large M and the tile kernel otherwise (nvfp4_w4a16_gemm_plan).
 * Used to check that the variants agree on the same inputs. */
nvfp4_status nvfp4_w4a16_gemm_variant(const void* x, int64_t ld_x, const void* pre_scale, const void* w_repacked,
                                      const float* global_scale, int global_scale_is_divisor,
                                      void* y, int64_t ld_y, int64_t M, int64_t N, int64_t K,
                                      void* workspace, int64_t workspace_bytes, int variant, void* stream);

/* The variant (1..4 above) that nvfp4_w4a16_gemm runs for an M x N x K call,
 * 0 when it launches nothing (M == 0 or N == 0), -1 for invalid sizes.  A
 * pure host function of the sizes (bf16 and fp16 calls choose alike). */
int nvfp4_w4a16_gemm_plan(int64_t M, int64_t N, int64_t K);

/* 1 if nvfp4_w4a16_gemm_variant accepts `variant` for an M x N x K call, 0 if
 * it rejects the shape (INVALID_ARG), -1 for invalid sizes or variants.  A
 * pure host function of the sizes. */
int nvfp4_w4a16_gemm_variant_takes(int64_t M, int64_t N, int64_t K, int variant);

/* ------------------------------------------------- no-allocation entry --
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  nvfp4_w4a16_gemm without the workspace arguments: the split-K
 * partial sums and arrival counters that some shapes need live in a static
 * device array of the library, nvfp4_w4a16_gemm_noalloc_max_scratch_bytes()
 * bytes (4 MiB) on every GPU the library runs on, held until the process
 * ends.  The call allocates nothing (no hipMalloc, no allocating library
 * routine); the caller still passes the inputs and the output.  The first
 * call on a device looks up the array's device address and clears its
 * counters on `stream` (a fill kernel); every call leaves the counters it
 * used at zero.  All calls on one GPU share that GPU's array: calls that may
 * overlap in time on one GPU (other streams, other threads) race and give
 * undefined results; issue them one after another.
 * Arguments, kernel choice, results (bitwise those of nvfp4_w4a16_gemm) and
 * errors as for nvfp4_w4a16_gemm, plus: a call whose kernel needs more
 * scratch than the array holds (nvfp4_w4a16_gemm_workspace_bytes above the
 * maximum) -> BUFFER_TOO_SMALL, before anything is launched; the address
 * lookup failing -> HIP. */
int64_t nvfp4_w4a16_gemm_noalloc_max_scratch_bytes(void);
nvfp4_status nvfp4_w4a16_gemm_noalloc(const void* x, int64_t ld_x, const void* pre_scale, const void* w_repacked,
                                      const float* global_scale, int global_scale_is_divisor, void* y, int64_t ld_y,
                                      int64_t M, int64_t N, int64_t K, void* stream);

/* Measurement export: a plain read of `bytes` (a multiple of 16) at p
 * (16-byte aligned), the bandwidth reference the GEMMs are measured against.
 * `workgroups` workgroups of 256 threads each read a contiguous share with
 * non-temporal 16-byte loads, `unroll` (1, 2, 4 or 8) loads per thread in
 * flight; out (uint32 [workgroups], 4-byte aligned) is written only in the
 * practically impossible case that a workgroup's data folds to a fixed value
 * (it keeps the loads alive).  Errors: bad sizes or unroll -> INVALID_ARG,
 * misaligned pointers -> ALIGNMENT. */
nvfp4_status nvfp4_bench_stream_read(const void* p, int64_t bytes, uint32_t* out, int64_t workgroups, int unroll,
                                     void* stream);

/* ---- MXFP4 weights -----------------------------------------------------------
 *
 * Weight-only MXFP4: the same packed E2M1 codes with one E8M0 scale per 32
 * consecutive K of a row and no global scale (SGLang compressed-tensors
 * NVFP4 weight-only page, Modifications: the paragraph on MXFP4 names group
 * size 32 (group_blocks == 2), E8M0 scales and the missing global scale as
 * what sets it apart from NVFP4).  E8M0 is the OCP MX scale: byte e decodes
 * to 2^(e-127), 0xFF is NaN.
 *
 *     Y = RNE(sum_k X'[m,k] * e2m1(code(n,k)) * e8m0(S[n, k/32]))
 *
 *   w_scale : uint8 E8M0 [E][N][ld_s], ld_s >= K/32; K must be a multiple of
 *             32 (INVALID_ARG otherwise).
 * The repacked blob has the size mxfp4_repack_bytes(E,N,K) (equal to
 * nvfp4_repack_bytes) and may only be passed to the mxfp4_* calls.  The
 * GEMMs take the arguments, kernel choice, workspace sizes
 * (nvfp4_w4a16_gemm_workspace_bytes, nvfp4_w4a16_grouped_gemm_workspace_bytes),
 * pre-quant scale, ownership, zero sizes and errors of the NVFP4 calls, minus
 * the global scale; the _f16 forms take fp16 activations and outputs.
 * Decoded weights are exact in bf16 while |e2m1 * 2^(e-127)| stays in bf16's
 * normal range (scale bytes 2..252; the kernels may flush smaller ones to
 * zero and larger ones overflow to infinity), in fp16 while it stays in
 * fp16's (bytes 114..140 for every code). */
int64_t mxfp4_repack_bytes(int64_t E, int64_t N, int64_t K); /* < 0 if invalid */
nvfp4_status mxfp4_repack(const uint8_t* w_packed, int64_t ld_w, const uint8_t* w_scale, int64_t ld_s,
                          int64_t E, int64_t N, int64_t K, void* out, int64_t out_bytes, void* stream);
nvfp4_status mxfp4_w4a16_gemm(const void* x, int64_t ld_x, const void* pre_scale, const void* w_repacked, void* y,
                              int64_t ld_y, int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                              void* stream);
nvfp4_status mxfp4_w4a16_gemm_f16(const void* x, int64_t ld_x, const void* pre_scale, const void* w_repacked, void* y,
                                  int64_t ld_y, int64_t M, int64_t N, int64_t K, void* workspace,
                                  int64_t workspace_bytes, void* stream);
nvfp4_status mxfp4_w4a16_grouped_gemm(const void* x, int64_t ld_x, const int32_t* expert_offsets, const void* pre_scale,
                                      const void* w_repacked, void* y, int64_t ld_y, int64_t R, int64_t E, int64_t N,
                                      int64_t K, void* workspace, int64_t workspace_bytes, void* stream);
nvfp4_status mxfp4_w4a16_grouped_gemm_f16(const void* x, int64_t ld_x, const int32_t* expert_offsets,
                                          const void* pre_scale, const void* w_repacked, void* y, int64_t ld_y,
                                          int64_t R, int64_t E, int64_t N, int64_t K, void* workspace,
                                          int64_t workspace_bytes, void* stream);
/* The fused MoE FC1 on MXFP4 weights (the weight format of the section above,
 * in the MoE FC1 that nvfp4_moe_fc1 cites): mxfp4_repack_gated is
 * nvfp4_repack_gated with E8M0 scales [E][2 I][ld_s], ld_s >= K/32 (K a
 * multiple of 32), and mxfp4_moe_fc1 is nvfp4_moe_fc1 without global scales,
 * on a blob from mxfp4_repack_gated (NVFP4_MOE_SILU_GLU) or mxfp4_repack
 * (NVFP4_MOE_RELU2): bitwise mxfp4_w4a16_grouped_gemm (with the row gather)
 * followed by nvfp4_moe_silu_mul or nvfp4_moe_relu2.  Errors as those calls. */
int64_t mxfp4_repack_gated_bytes(int64_t E, int64_t I, int64_t K); /* < 0 if invalid */
nvfp4_status mxfp4_repack_gated(const uint8_t* w_packed, int64_t ld_w, const uint8_t* w_scale, int64_t ld_s,
                                int64_t E, int64_t I, int64_t K, int up_first, void* out, int64_t out_bytes,
                                void* stream);
nvfp4_status mxfp4_moe_fc1(const void* x, int64_t ld_x, int64_t T, const int32_t* row_token,
                           const int32_t* expert_offsets, const void* pre_scale, const void* w_fc1, int activation,
                           void* a, int64_t ld_a, int64_t R, int64_t E, int64_t I, int64_t K, void* stream);
nvfp4_status mxfp4_moe_fc1_f16(const void* x, int64_t ld_x, int64_t T, const int32_t* row_token,
                               const int32_t* expert_offsets, const void* pre_scale, const void* w_fc1, int activation,
                               void* a, int64_t ld_a, int64_t R, int64_t E, int64_t I, int64_t K, void* stream);
/* Test exports: the decoded tile (as nvfp4_dequant_bf16, E8M0 scales) and the
 * dense GEMM with a forced kernel variant (as nvfp4_w4a16_gemm_variant; f16
 * selects fp16 activations and outputs). */
nvfp4_status mxfp4_dequant_bf16(const void* w_repacked, int64_t E, int64_t N, int64_t K, void* out, int64_t ld_out,
                                void* stream);
nvfp4_status mxfp4_w4a16_gemm_variant(const void* x, int64_t ld_x, const void* pre_scale, const void* w_repacked,
                                      void* y, int64_t ld_y, int64_t M, int64_t N, int64_t K, void* workspace,
                                      int64_t workspace_bytes, int variant, int f16, void* stream);

/* ---- FP16 activations and outputs ------------------------------------------
 *
 * The same operations with X, the pre-quant scale and Y in IEEE binary16
 * instead of bf16 (weight-only FP4 serves bf16 or fp16 activations: "Support
 * nvfp4 w4a16 on sm120", Summary; SGLang compressed-tensors NVFP4
 * weight-only page, Motivation).  Arguments, layouts, workspace sizes
 * (nvfp4_w4a16_gemm_workspace_bytes / nvfp4_w4a16_grouped_gemm_workspace_bytes),
 * kernel choice, ownership and errors are those of the bf16 calls above.
 * The decoded weights are exact in fp16 (e2m1 * e4m3 lies in [2^-10, 2688]
 * with at most 6 significant bits), the MFMAs take fp16 with fp32
 * accumulation, the pre-scaled activation is RNE_fp16(X * s) and
 * Y = RNE_fp16(g * acc); outputs beyond the fp16 range become +-infinity. */
nvfp4_status nvfp4_w4a16_gemm_f16(const void* x, int64_t ld_x, const void* pre_scale, const void* w_repacked,
                                  const float* global_scale, int global_scale_is_divisor, void* y, int64_t ld_y,
                                  int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                                  void* stream);

/* nvfp4_w4a16_gemm_variant with fp16 activations and outputs. */
nvfp4_status nvfp4_w4a16_gemm_variant_f16(const void* x, int64_t ld_x, const void* pre_scale, const void* w_repacked,
                                          const float* global_scale, int global_scale_is_divisor, void* y,
                                          int64_t ld_y, int64_t M, int64_t N, int64_t K, void* workspace,
                                          int64_t workspace_bytes, int variant, void* stream);

/* nvfp4_w4a16_grouped_gemm with fp16 activations and outputs. */
nvfp4_status nvfp4_w4a16_grouped_gemm_f16(const void* x, int64_t ld_x, const int32_t* expert_offsets,
                                          const void* pre_scale, const void* w_repacked, const float* global_scales,
                                          int global_scale_is_divisor, void* y, int64_t ld_y, int64_t R, int64_t E,
                                          int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                                          void* stream);

/* The MoE glue steps with fp16 activations (the routing is type-free): the
 * gathering grouped GEMM, the gated SiLU, the squared ReLU and the top-k
 * combine, each as its bf16 form above with every 16-bit array in IEEE
 * binary16 and every rounding RNE to fp16 (overflow to +-infinity). */
nvfp4_status nvfp4_w4a16_grouped_gemm_gather_f16(const void* x, int64_t ld_x, int64_t T, const int32_t* row_token,
                                                 const int32_t* expert_offsets, const void* pre_scale,
                                                 const void* w_repacked, const float* global_scales,
                                                 int global_scale_is_divisor, void* y, int64_t ld_y, int64_t R,
                                                 int64_t E, int64_t N, int64_t K, void* workspace,
                                                 int64_t workspace_bytes, void* stream);
nvfp4_status nvfp4_moe_silu_mul_f16(const void* h, int64_t ld_h, int64_t R, int64_t I, void* a, int64_t ld_a,
                                    void* stream);
nvfp4_status nvfp4_moe_relu2_f16(const void* h, int64_t ld_h, int64_t R, int64_t I, void* a, int64_t ld_a,
                                 void* stream);
nvfp4_status nvfp4_moe_combine_f16(const void* y, int64_t ld_y, const int32_t* token_row, const float* topk_weights,
                                   int64_t T, int64_t k, int64_t H, void* out, int64_t ld_o, void* stream);
/* nvfp4_moe_fc1 with fp16 activations and output (RNE to fp16 throughout). */
nvfp4_status nvfp4_moe_fc1_f16(const void* x, int64_t ld_x, int64_t T, const int32_t* row_token,
                               const int32_t* expert_offsets, const void* pre_scale, const void* w_fc1,
                               const float* global_scales, int global_scale_is_divisor, int activation, void* a,
                               int64_t ld_a, int64_t R, int64_t E, int64_t I, int64_t K, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_W4A16_H */
