/*
 * qkvmx.h -- C ABI of the MI355X (gfx950) fused MXFP8 QKV projection library.
 *
 * The operations follow two source pages:
 *   [QKV-CTE]    "Kernel reference: qkv_cte -- Wan2.2 additions to the NKI Library QKV CTE MXFP8
 *                projection" (sections "Upstream behavior", "Design 1)" .. "Design 5)",
 *                "Interface").
 *   [RMSNORM-MX] "RMSNorm MX Prefill Kernel API Reference" (parameters residual, eps,
 *                unpadded_hidden_size, qmx_output_dtype, emit_norm_bf16).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library never frees or
 *     retains them past the call.  Nothing is allocated on any call.
 *   - Work is enqueued asynchronously on `stream` (NULL = the legacy default stream).  Calls on
 *     one stream are ordered; the library keeps no mutable global state, so distinct streams may
 *     call concurrently on distinct buffers.
 *   - Every argument is validated on the host BEFORE any HIP call; a failed validation returns a
 *     status and touches nothing.  qkvmx_last_error() then gives a one-line reason (per thread).
 *   - A HIP launch error returns QKVMX_ERR_HIP.  Faults inside a kernel surface at the caller's
 *     next synchronisation, as for any asynchronous HIP work.
 *   - bf16 tensors are passed as uint16_t bit patterns; fp32 scales are IEEE binary32.
 *   - T = B * S tokens: [B, S, ...] tensors of the pages are flattened to [T, ...].
 */
#ifndef QKVMX_H
#define QKVMX_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QKVMX_OK = 0,
  QKVMX_ERR_NULL = 1,         /* a required pointer is NULL                                  */
  QKVMX_ERR_SHAPE = 2,        /* sizes inconsistent or outside the supported range           */
  QKVMX_ERR_ALIGN = 3,        /* a pointer or stride violates the stated alignment           */
  QKVMX_ERR_ARG = 4,          /* invalid flag / optional-argument combination                */
  QKVMX_ERR_WORKSPACE = 5,    /* workspace missing or smaller than qkvmx_workspace_bytes()   */
  QKVMX_ERR_UNSUPPORTED = 6,  /* well-formed request this build does not implement           */
  QKVMX_ERR_HIP = 7           /* a HIP runtime call (launch) failed                          */
} qkvmx_status;

/* Pass-2 flags ([QKV-CTE] "Interface": qk_norm_pre_rope q_norm / k_norm, fused_rope). */
enum {
  QKVMX_NORM_Q = 1,       /* across-heads RMSNorm of the first (Q) segment                 */
  QKVMX_NORM_K = 2,       /* across-heads RMSNorm of the K segment (needs num_kv_heads > 0)  */
  QKVMX_FUSED_ROPE = 4    /* rotate-half RoPE on Q and K after the norm                      */
};

/* Output layouts ([QKV-CTE] "Interface": output_layout, BSD [B, S, I] or NBSd
 * [num_heads, B, S, d_head]; B = 1 here, T = S).  With I / d heads in column order (the
 * num_heads Q heads, then the num_kv_heads K heads, then the V heads), BSD column h * d + j of
 * token t and NBSd element (h, t, j) hold the same value. */
enum {
  QKVMX_LAYOUT_BSD = 0,   /* [T, I] row-major, I = (num_heads + 2 * num_kv_heads) * head_dim  */
  QKVMX_LAYOUT_NBSD = 1   /* [I / head_dim, T, head_dim]: (h, t, j) at (h * T + t) * d + j    */
};

/* Per-head qk-norm kinds of qkv_rowmx_project_headnorm ([QKV-CTE] "Upstream behavior":
 * RMS_NORM / LAYER_NORM). */
enum { QKVMX_HEAD_RMS_NORM = 1, QKVMX_HEAD_LAYER_NORM = 2 };

/* Element types of the plain row quantiser's input. */
enum { QKVMX_DTYPE_F32 = 0, QKVMX_DTYPE_BF16 = 1 };

/* Static name of a status code. */
const char* qkvmx_status_string(qkvmx_status s);

/* Reason for the last non-OK status returned on the calling thread ("" if none). */
const char* qkvmx_last_error(void);

/* ------------------------------------------------------------------------------------------
 * Weight preparation (one-time, like weight loading; not part of the per-token path).
 * ------------------------------------------------------------------------------------------ */

/* MX block-32 FP8 encoding of a natural-orientation fp32 weight W[H, I] (row-major).
 * Writes the pages' layout ([QKV-CTE] "Interface", weight: "[H // 4, I, 4] FP8, MX-contiguous"):
 * element (h, i) at byte ((h / 4) * I + i) * 4 + h % 4 of `w_h4_i_4` (H * I bytes), and one
 * E8M0 exponent per 32 consecutive h of a column in `w_e8m0` ([H / 32, I] bytes).
 * Exponent rule (OCP MX shared exponent, the plain reading; the pages do not fix it):
 * X = floor(log2(max |w| of the block)) - 8, E = clamp(X + 127, 0, 254); code =
 * E4M3 round-to-nearest-even, saturating, of w / 2^(E - 127); an all-zero block gets E = 0.
 * Requires H % 32 == 0, H, I > 0.  Non-finite weights give unspecified codes. */
qkvmx_status mx_weight_quantize(const float* w, int64_t H, int64_t I,
                                uint8_t* w_h4_i_4, uint8_t* w_e8m0, hipStream_t stream);

/* Bytes of the device-side packed weight for an [H, I] projection. */
size_t qkv_weight_packed_bytes(int64_t H, int64_t I);

/* Re-lays the pages' weight ([H / 4, I, 4] E4M3 codes + [H / 32, I] E8M0 exponents) into the
 * layout the projection kernel reads: K-contiguous rows per output channel plus the exponents
 * grouped per MFMA step.  `w_packed` (>= qkv_weight_packed_bytes(H, I) bytes, 256-byte aligned)
 * is opaque; it depends only on (H, I).  Requires H % 32 == 0. */
qkvmx_status qkv_weight_prepack(const uint8_t* w_h4_i_4, const uint8_t* w_e8m0, int64_t H,
                                int64_t I, void* w_packed, size_t w_packed_bytes,
                                hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Activation producers.
 * ------------------------------------------------------------------------------------------ */

/* ROW_MX row quantisation, the role of the pages' row_quantize_packed ([QKV-CTE] "Interface",
 * packed_hidden: "[B, S, H + 4] FP8: H FP8 codes plus a 4-byte fp32 dequant scale tail").
 * x: [T, H] fp32 or bf16 (x_dtype), row-major.  packed_out: [T, H + 4] bytes; per row
 * s = fl32(max_h |x_h| / 448) (IEEE division), code_h = E4M3 round-to-nearest-even saturating of
 * fl32(x_h / s), then s as little-endian fp32 at byte offset H.  A zero row gets s = 0 and zero
 * codes.  Requires H % 32 == 0, H <= 16384; packed_out 4-byte aligned. */
qkvmx_status row_quantize_packed(const void* x, int32_t x_dtype, int64_t T, int64_t H,
                                 uint8_t* packed_out, hipStream_t stream);

/* Fused residual add + RMSNorm + ROW_MX quantisation of bf16 hidden states
 * ([RMSNORM-MX]; output in the ROW_MX packed layout the projection consumes).
 *   r    = bf16_RNE(fp32(hidden) + fp32(residual))   -> residual_out   (r = hidden if no residual)
 *   inv  = fp32(1 / sqrt(sum_h r_h^2 / Hu + eps))     (sum, sqrt and divide in fp64)
 *   y_h  = fl32(fl32(r_h * inv) * gamma_h)            -> ROW_MX encode as row_quantize_packed
 * hidden, residual, residual_out: [T, H] bf16; gamma: [H] bf16; packed_out: [T, H + 4].
 * residual_out is required iff residual is given.  unpadded_H (Hu) in (0, H], 0 means H: the
 * sum runs over all H columns, the mean divides by Hu.  Requires H % 32 == 0, H <= 16384. */
qkvmx_status rmsnorm_mx_quantize(const uint16_t* hidden, const uint16_t* residual,
                                 const uint16_t* gamma, float eps, int64_t T, int64_t H,
                                 int64_t unpadded_H, uint16_t* residual_out, uint8_t* packed_out,
                                 hipStream_t stream);

/* Staged ROW_MX activations.  [RMSNORM-MX] lays its quantised output out for the consumer
 * that reads it next (its scale packing and H-swizzle serve the other machine's transposes);
 * the counterpart here is the projection's own operand layout, so the projection DMA-copies
 * the codes into LDS without re-laying them per call.  The arithmetic (scale, codes) is exactly
 * that of the packed-row producers; only the placement of the bytes differs:
 *   act_image  [ceil(T / 256)][KS][256][64] bytes, KS = 4 * ceil(H / 256): the code of row t,
 *              element h sits at ((t / 256 * KS + h / 64) * 256 + t % 256) * 64
 *              + ((((h / 16) % 4) ^ sw(t % 256)) << 4) + h % 16,
 *              sw(r) = ((r >> 1) & 3) ^ ((r >> 3) & 1).  Codes for h in [H, 64 KS) and every
 *              code of rows t in [T, 256 ceil(T / 256)) are written as 0x00.
 *              qkv_act_image_bytes(T, H) bytes, 16-byte aligned.
 *   row_scale  [T] fp32: the row scale s of the packed layout's 4-byte tail. */
size_t qkv_act_image_bytes(int64_t T, int64_t H);

/* row_quantize_packed with the staged output (act_image, row_scale as above).  image_bytes
 * must be >= qkv_act_image_bytes(T, H).  Requires H % 32 == 0, H <= 16384; x 16-byte,
 * act_image 16-byte, row_scale 4-byte aligned. */
qkvmx_status row_quantize_staged(const void* x, int32_t x_dtype, int64_t T, int64_t H,
                                 uint8_t* act_image, size_t image_bytes, float* row_scale,
                                 hipStream_t stream);

/* rmsnorm_mx_quantize with the staged output: the same r, inv, y, scale and codes; codes into
 * act_image, scales into row_scale (layouts above).  image_bytes >= qkv_act_image_bytes(T, H).
 * Other arguments and requirements as rmsnorm_mx_quantize; act_image 16-byte, row_scale 4-byte
 * aligned. */
qkvmx_status rmsnorm_mx_quantize_staged(const uint16_t* hidden, const uint16_t* residual,
                                        const uint16_t* gamma, float eps, int64_t T, int64_t H,
                                        int64_t unpadded_H, uint16_t* residual_out,
                                        uint8_t* act_image, size_t image_bytes, float* row_scale,
                                        hipStream_t stream);

/* MX block-32 encoding of activation rows ([RMSNORM-MX] qmx_output_dtype: E4M3 codes with one
 * E8M0 scale per 32 elements of a row; the other machine's packing and swizzle of the scales are
 * not reproduced).  x: [T, H] fp32 or bf16 (x_dtype).  codes_out: [T, H] bytes, natural H order;
 * e8m0_out: [T, H / 32] bytes, byte b of row t the exponent of elements [32 b, 32 b + 32).
 * Per block: E = clamp(floor(log2(max |x| of the block)) - 8 + 127, 0, 254), codes = E4M3
 * round-to-nearest-even saturating of x / 2^(E - 127) (the rule the weight encoder uses); an
 * all-zero block stores E = 0 and zero codes.  Requires H % 32 == 0, H <= 16384; x 16-byte,
 * codes_out 8-byte, e8m0_out 4-byte aligned. */
qkvmx_status mx_block_quantize(const void* x, int32_t x_dtype, int64_t T, int64_t H,
                               uint8_t* codes_out, uint8_t* e8m0_out, hipStream_t stream);

/* Fused residual add + RMSNorm + MX block-32 quantisation ([RMSNORM-MX]: residual, eps,
 * unpadded_hidden_size, qmx_output_dtype, emit_norm_bf16).  r, inv and y are those of
 * rmsnorm_mx_quantize; y is then encoded as mx_block_quantize does, and when norm_out is not
 * NULL y is also stored there rounded to bf16 (round to nearest even): emit_norm_bf16.
 * hidden, residual, residual_out, norm_out: [T, H] bf16; gamma: [H] bf16; codes_out [T, H];
 * e8m0_out [T, H / 32].  residual_out is required iff residual is given.  Requires H % 32 == 0,
 * H <= 16384; bf16 tensors 16-byte, codes_out 8-byte, e8m0_out 4-byte aligned. */
qkvmx_status rmsnorm_mx_block_quantize(const uint16_t* hidden, const uint16_t* residual,
                                       const uint16_t* gamma, float eps, int64_t T, int64_t H,
                                       int64_t unpadded_H, uint16_t* residual_out,
                                       uint8_t* codes_out, uint8_t* e8m0_out, uint16_t* norm_out,
                                       hipStream_t stream);

/* Staged MX block-32 activations: the codes in the act_image layout of the staged ROW_MX
 * producers, the exponents in the exponent image the projection's K-loop reads:
 *   exp_image  [ceil(T / 256)][S][256][2] uint32, S = ceil(H / 256): byte q of dword g of row
 *              t % 256 in superstep s of tile t / 256 is the E8M0 exponent of elements
 *              [32 (8 s + 2 q + g), 32 (8 s + 2 q + g) + 32) of row t; 127 (2^0) for blocks
 *              past H / 32 and for rows past T (whose codes are 0x00).
 *              qkv_act_exp_image_bytes(T, H) bytes, 16-byte aligned.
 * Codes and exponents are exactly those of mx_block_quantize / rmsnorm_mx_block_quantize. */
size_t qkv_act_exp_image_bytes(int64_t T, int64_t H);

/* mx_block_quantize with the staged outputs (act_image, exp_image above). */
qkvmx_status mx_block_quantize_staged(const void* x, int32_t x_dtype, int64_t T, int64_t H,
                                      uint8_t* act_image, size_t image_bytes, uint32_t* exp_image,
                                      size_t exp_image_bytes, hipStream_t stream);

/* rmsnorm_mx_block_quantize with the staged outputs (act_image, exp_image above); residual_out
 * and norm_out as there. */
qkvmx_status rmsnorm_mx_block_quantize_staged(const uint16_t* hidden, const uint16_t* residual,
                                              const uint16_t* gamma, float eps, int64_t T,
                                              int64_t H, int64_t unpadded_H,
                                              uint16_t* residual_out, uint8_t* act_image,
                                              size_t image_bytes, uint32_t* exp_image,
                                              size_t exp_image_bytes, uint16_t* norm_out,
                                              hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Pass 1: the projection ([QKV-CTE] "Upstream behavior", O[S, I] = A[S, H] @ W[H, I] + bias,
 * I = (num_heads + 2 * num_kv_heads) * head_dim; "Design 1)" step a).
 * ------------------------------------------------------------------------------------------ */

/* Workspace bytes qkv_rowmx_project needs for a [T, H] x [H, I] call: the activation codes
 * re-laid in the kernel's LDS stage images (about T * H bytes) plus per-tile sums of squares
 * and, for calls with few output tiles (see qkvmx_projection_k_chunks), k fp32 [T, I] planes
 * of the split contraction, k = min(3, 256 / tiles), tiles = ceil(T / 256) * ceil(I / 256)
 * <= 128.  0 for invalid sizes. */
size_t qkvmx_workspace_bytes(int64_t T, int64_t H, int64_t I);

/* Number of K chunks the projections (qkv_rowmx_project[_staged], qkv_mx_project[_staged])
 * cut a [T, H] x [H, I] call into.  A call with at most 128 output tiles of 256 x 256 leaves
 * most compute units idle, so its 256-byte K supersteps are split into up to
 * min(3, 256 / tiles) chunks of ceil(supersteps / that) supersteps; each (tile, chunk) unit
 * writes its fp32 partial sums to a plane of the workspace, and a per-token pass adds the
 * planes in chunk order and applies the epilogue (scales, bias, bf16 rounding, sums of
 * squares; BSD or NBSd store).  The result is the same function of the inputs, accumulated in
 * a different fp32 order, and identical for both layouts.  1 = no split; 0 for invalid sizes
 * or layout.  Host only. */
int32_t qkvmx_projection_k_chunks(int64_t T, int64_t H, int64_t I, int32_t layout);

/* out[t, i] = bf16_RNE( a_scale[t] * c[i] * sum_h dec(a[t, h]) * dec(W[h, i]) * 2^(E[h/32, i]-127)
 *                       + bias[i] )
 * and, when ssq != NULL, ssq[t] = { sum over the Q columns of X^2, sum over the K columns of X^2 }
 * over the fp32 values before rounding (V excluded; the K entry is 0 when num_kv_heads == 0).
 *   a_codes       E4M3 codes of row t at a_codes + t * a_row_stride (H bytes).
 *   a_scales      fp32 row scale of row t at a_scales + t * a_scale_stride (4-byte aligned).
 *                 The pages' packed rows: a_scales = a_codes + H, both strides = H + 4.
 *   w_packed      output of qkv_weight_prepack for this (H, I).
 *   w_channel_scale  fp32 [I] per-output-channel scale ("weight_scales [1, I]"), NULL = 1.
 *   bias          bf16 [I] or NULL.
 *   layout        QKVMX_LAYOUT_BSD: out is [T, I] row-major bf16; QKVMX_LAYOUT_NBSD: out is
 *                 [I / head_dim, T, head_dim] bf16 (needs 2 ((256 + d) T + 257 d) < 2^31).
 *                 Any other value is QKVMX_ERR_ARG.
 *   workspace     >= qkvmx_workspace_bytes(T, H, I) bytes, 256-byte aligned, required; its
 *                 contents are scratch (overwritten by every call; calls sharing one workspace
 *                 must be ordered on one stream).
 * Requires T >= 1, H % 32 == 0, head_dim % 16 == 0, num_heads >= 1, num_kv_heads >= 0,
 * a_row_stride >= H and a multiple of 4, a_codes 4-byte aligned, out 16-byte aligned. */
qkvmx_status qkv_rowmx_project(const uint8_t* a_codes, int64_t a_row_stride,
                               const uint8_t* a_scales, int64_t a_scale_stride,
                               const void* w_packed, const float* w_channel_scale,
                               const uint16_t* bias, int64_t T, int64_t H, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t layout,
                               uint16_t* out, float* ssq, void* workspace, size_t ws_bytes,
                               hipStream_t stream);

/* Workspace bytes qkv_rowmx_project_staged (and qkv_mx_project_staged) needs: the per-tile
 * sums of squares, the tile counters (no activation re-layout) and, for calls with few tiles,
 * the split contraction's planes (as for qkvmx_workspace_bytes).  0 for invalid sizes. */
size_t qkv_staged_workspace_bytes(int64_t T, int64_t I);

/* qkv_rowmx_project on staged activations (act_image, row_scale written by
 * row_quantize_staged or rmsnorm_mx_quantize_staged for the same T and H): the same out and
 * ssq, bit for bit, as qkv_rowmx_project on the packed rows of the same codes and scales.
 *   image_bytes  >= qkv_act_image_bytes(T, H); act_image 256-byte aligned.
 *   workspace    >= qkv_staged_workspace_bytes(T, I) bytes, 256-byte aligned, required;
 *                scratch, as for qkv_rowmx_project.
 * Other arguments, layouts and errors as qkv_rowmx_project. */
qkvmx_status qkv_rowmx_project_staged(const uint8_t* act_image, size_t image_bytes,
                                      const float* row_scale, const void* w_packed,
                                      const float* w_channel_scale, const uint16_t* bias,
                                      int64_t T, int64_t H, int32_t num_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t layout,
                                      uint16_t* out, float* ssq, void* workspace,
                                      size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, serving loops
 * or harnesses that forbid hipMalloc): qkv_rowmx_project_staged without the workspace
 * argument.  The projection's scratch (tile counters, sum-of-squares partials, split planes)
 * lives in a static device array of qkvmx_noalloc_scratch_bytes() bytes (80 MiB) that every
 * GPU the library runs on holds until the process ends; the call allocates nothing (no
 * hipMalloc / hipFree, no allocating library routine) and launches the same kernels, so out
 * and ssq are bit for bit those of qkv_rowmx_project_staged.  The counters the kernels need
 * zeroed are cleared by a kernel on every call; nothing else is read before it is written.
 *   Errors: QKVMX_ERR_WORKSPACE when qkv_staged_workspace_bytes(T, I) exceeds the scratch
 *   (checked on the host before any HIP call); QKVMX_ERR_HIP if the scratch's device address
 *   cannot be obtained (looked up once per device, with that device current, on its first
 *   call).  Other arguments, layouts and errors as qkv_rowmx_project_staged.
 *   All calls on one GPU share its scratch: calls that overlap on one GPU (concurrent streams)
 *   race and must not be issued. */
size_t qkvmx_noalloc_scratch_bytes(void);
qkvmx_status qkv_rowmx_project_staged_noalloc(const uint8_t* act_image, size_t image_bytes,
                                              const float* row_scale, const void* w_packed,
                                              const float* w_channel_scale, const uint16_t* bias,
                                              int64_t T, int64_t H, int32_t num_heads,
                                              int32_t num_kv_heads, int32_t head_dim,
                                              int32_t layout, uint16_t* out, float* ssq,
                                              hipStream_t stream);

/* Pass 1 with the upstream per-head qk-norm and rotate-half RoPE fused into the epilogue
 * ([QKV-CTE] "Upstream behavior": an optional per-head qk-norm (RMS_NORM / LAYER_NORM) and
 * rotate-half RoPE applied as each finished result leaves the accumulators, with the dequant
 * scaling and the bias add, so no second pass over Q and K is needed; "Design 1)": each head's
 * d_head slice normalised by its own statistics).  With X the dequantised, bias-added fp32 value
 * of qkv_rowmx_project (before rounding), for every Q and K head h of token t:
 *   RMS_NORM:   y = X / sqrt(mean_h(X^2) + eps) * gamma
 *   LAYER_NORM: y = (X - mean_h(X)) / sqrt(mean_h((X - mean_h(X))^2) + eps) * gamma + beta
 * (statistics over the head's d values), then, with cos_tab / sin_tab, rotate-half RoPE of each
 * pair (j, j + d/2), j < d/2, by the angle of position j of row t:
 *   out_j = y_j cos[t, j] - y_{j+d/2} sin[t, j],  out_{j+d/2} = y_{j+d/2} cos[t, j] + y_j sin[t, j]
 * (rotate-half tables hold the same angle in both halves; the second half is not read).  V is
 * stored as X.  The result is rounded to bf16 once, in `layout` (as qkv_rowmx_project).
 *   q_gamma, k_gamma   bf16 [head_dim], one per segment, shared by its heads; k_gamma required
 *                      iff num_kv_heads > 0.
 *   q_beta, k_beta     bf16 [head_dim] or NULL (0); QKVMX_HEAD_LAYER_NORM only.
 *   cos_tab, sin_tab   fp32 [T, head_dim], both or neither (NULL: no RoPE).
 *   workspace          >= qkvmx_workspace_bytes(T, H, I) bytes, 256-byte aligned; scratch.
 * Activation arguments as qkv_rowmx_project; no channel scale, no sums of squares.  Requires
 * head_dim 64 or 128 and num_heads * head_dim, num_kv_heads * head_dim multiples of 128
 * (QKVMX_ERR_UNSUPPORTED otherwise); gamma/beta 8-byte, tables 16-byte aligned. */
qkvmx_status qkv_rowmx_project_headnorm(const uint8_t* a_codes, int64_t a_row_stride,
                                         const uint8_t* a_scales, int64_t a_scale_stride,
                                         const void* w_packed, const uint16_t* bias, int64_t T,
                                         int64_t H, int32_t num_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t layout, int32_t norm_kind,
                                         const uint16_t* q_gamma, const uint16_t* k_gamma,
                                         const uint16_t* q_beta, const uint16_t* k_beta,
                                         float eps, const float* cos_tab, const float* sin_tab,
                                         uint16_t* out, void* workspace, size_t ws_bytes,
                                         hipStream_t stream);

/* qkv_rowmx_project_headnorm on staged activations (act_image, row_scale written by
 * row_quantize_staged or rmsnorm_mx_quantize_staged for the same T and H): the same out, bit for
 * bit, as qkv_rowmx_project_headnorm on the packed rows of the same codes and scales, without
 * the per-call activation re-layout.
 *   image_bytes  >= qkv_act_image_bytes(T, H); act_image 256-byte aligned.
 *   workspace    >= qkv_staged_workspace_bytes(T, I) bytes, 256-byte aligned, required; scratch.
 * Other arguments, layouts, requirements and errors as qkv_rowmx_project_headnorm. */
qkvmx_status qkv_rowmx_project_headnorm_staged(const uint8_t* act_image, size_t image_bytes,
                                                const float* row_scale, const void* w_packed,
                                                const uint16_t* bias, int64_t T, int64_t H,
                                                int32_t num_heads, int32_t num_kv_heads,
                                                int32_t head_dim, int32_t layout,
                                                int32_t norm_kind, const uint16_t* q_gamma,
                                                const uint16_t* k_gamma, const uint16_t* q_beta,
                                                const uint16_t* k_beta, float eps,
                                                const float* cos_tab, const float* sin_tab,
                                                uint16_t* out, void* workspace, size_t ws_bytes,
                                                hipStream_t stream);

/* Workspace bytes qkv_mx_project needs for a [T, H] x [H, I] call: the activation codes and
 * their exponents re-laid in the kernel's LDS stage images (about T * H * 33 / 32 bytes) plus
 * per-tile sums of squares and, for calls with few tiles, the split contraction's planes (as
 * for qkvmx_workspace_bytes).  0 for invalid sizes. */
size_t qkv_mx_workspace_bytes(int64_t T, int64_t H, int64_t I);

/* Pass 1 on MX block-32 activations ([RMSNORM-MX] qmx_output_dtype feeding [QKV-CTE]'s
 * projection): as qkv_rowmx_project with the row scale replaced by per-block exponents,
 * out[t, i] = bf16_RNE( c[i] * sum_h dec(a[t, h]) * 2^(Ea[t, h/32] - 127)
 *                                  * dec(W[h, i]) * 2^(E[h/32, i] - 127) + bias[i] ),
 * and ssq as there (fp32 values before rounding; V excluded).
 *   a_codes   E4M3 codes of row t at a_codes + t * a_row_stride (H bytes).
 *   a_e8m0    E8M0 exponents of row t at a_e8m0 + t * a_e8m0_stride (H / 32 bytes).
 *   workspace >= qkv_mx_workspace_bytes(T, H, I) bytes, 256-byte aligned, required; its
 *             contents are scratch, as for qkv_rowmx_project.
 * Other arguments, layouts and errors as qkv_rowmx_project.  Requires a_row_stride >= H and a
 * multiple of 4, a_codes 4-byte aligned, a_e8m0_stride >= H / 32. */
qkvmx_status qkv_mx_project(const uint8_t* a_codes, int64_t a_row_stride, const uint8_t* a_e8m0,
                            int64_t a_e8m0_stride, const void* w_packed,
                            const float* w_channel_scale, const uint16_t* bias, int64_t T,
                            int64_t H, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t layout, uint16_t* out, float* ssq, void* workspace,
                            size_t ws_bytes, hipStream_t stream);

/* qkv_mx_project on staged MX activations (act_image, exp_image written by
 * mx_block_quantize_staged or rmsnorm_mx_block_quantize_staged for the same T and H): the same
 * out and ssq, bit for bit, as qkv_mx_project on the natural-order codes and exponents.
 *   act_image, exp_image   256-byte aligned, at least qkv_act_image_bytes(T, H) and
 *                          qkv_act_exp_image_bytes(T, H) bytes.
 *   workspace              >= qkv_staged_workspace_bytes(T, I) bytes, 256-byte aligned; scratch.
 * Other arguments, layouts and errors as qkv_mx_project. */
qkvmx_status qkv_mx_project_staged(const uint8_t* act_image, size_t image_bytes,
                                   const uint32_t* exp_image, size_t exp_image_bytes,
                                   const void* w_packed, const float* w_channel_scale,
                                   const uint16_t* bias, int64_t T, int64_t H, int32_t num_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t layout,
                                   uint16_t* out, float* ssq, void* workspace, size_t ws_bytes,
                                   hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Pass 2: across-heads RMSNorm + rotate-half RoPE, in place on Q and K; V is neither read nor
 * written ([QKV-CTE] "Design 1)" steps b and c, "Design 2)", "Design 5)").
 * ------------------------------------------------------------------------------------------ */

/* For a segment (Q: columns [0, Iq), K: [Iq, Iq + Ik)) with n heads, per token t:
 *   r    = 1 / sqrt(ssq[t, seg] / (n * head_dim) + eps)              (when its NORM flag is set)
 *   y_j  = x_j * gamma_j * r                                          (x_j otherwise)
 *   RoPE: out_j = y_j * cos[t, j'] - y_{j+d/2} * sin[t, j']   for j' = j mod d < d/2,
 *         out_j = y_j * cos[t, j'] + y_{j-d/2} * sin[t, j']   for j' >= d/2  (within each head)
 * and out_j = y_j without QKVMX_FUSED_ROPE.  The result is stored as bf16 in place.
 *   qkv       bf16 output of pass 1 in `layout` (BSD [T, I] or NBSd [I / d, T, d]),
 *             I = (num_heads + 2 * num_kv_heads) * d; heads are addressed per that layout.
 *   ssq       fp32 [T, 2] (pass 1's sums); required iff a NORM flag is set.
 *   q_gamma   bf16 [num_heads * d], segment-wide; required iff QKVMX_NORM_Q.
 *   k_gamma   bf16 [num_kv_heads * d]; required iff QKVMX_NORM_K, must be NULL otherwise.
 *   cos_tab, sin_tab  fp32 [T, d] rotate-half caches; required iff QKVMX_FUSED_ROPE.
 * num_kv_heads == 0 is a single-segment call: QKVMX_NORM_K is then an error.
 * Requires head_dim % 16 == 0 and head_dim <= 1024; qkv, gamma and the tables 16-byte aligned,
 * ssq 8-byte aligned. */
qkvmx_status qk_norm_rope_apply(uint16_t* qkv, const float* ssq, const uint16_t* q_gamma,
                                const uint16_t* k_gamma, const float* cos_tab,
                                const float* sin_tab, int64_t T, int32_t num_heads,
                                int32_t num_kv_heads, int32_t head_dim, float eps,
                                uint32_t flags, int32_t layout, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Roofline calibration (a measurement helper, not a step of the method).
 * ------------------------------------------------------------------------------------------ */

/* Launches `blocks` blocks of 256 threads, each wavefront issuing iters x 16 scaled FP8 MFMAs
 * (V_MFMA_SCALE_F32_32X32X64_F8F6F4, 2 * 32 * 32 * 64 flop each) on register operands: random
 * E4M3 codes (random_operands != 0) or zeros; nothing else touches memory until the end.
 *   sink    [blocks * 256] fp32, written (keeps the results live).
 *   clocks  [blocks][2] uint64: elapsed core-clock cycles and 100 MHz reference ticks of the
 *           loop, per block.
 * flop = blocks * 4 * iters * 16 * 131072; the caller times the launch on `stream`.  Requires
 * 1 <= blocks <= 65535, 1 <= iters <= 1 << 24; sink 4-byte, clocks 8-byte aligned. */
qkvmx_status qkvmx_mfma_rate_probe(int32_t blocks, int32_t iters, int32_t random_operands,
                                   float* sink, uint64_t* clocks, hipStream_t stream);

/* Check of the producers' E4M3 encoding (a measurement helper, not a step of the method).  The
 * ROW_MX and MX producers form their codes with the hardware's packing conversion after a clamp
 * to [-448, 448]; this launches one kernel that compares that path with the library's software
 * round-to-nearest-even saturating encoder on every finite fp32 value (all 2^32 bit patterns).
 *   counts     device uint64 [3], zeroed by the caller: counts[0] += values whose codes differ,
 *              counts[1] += finite values compared (2^32 - 2^24: every pattern but the 2^24
 *              infinities and NaNs),
 *              counts[2] = number of mismatches recorded (at most 8 kept).
 *   first_bad  device uint32 [8] or NULL: bit patterns of the first mismatching values.
 * Asynchronous on `stream`; QKVMX_ERR_NULL / QKVMX_ERR_ALIGN for bad pointers. */
qkvmx_status qkvmx_e4m3_convert_check(unsigned long long* counts, uint32_t* first_bad,
                                      hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* QKVMX_H */
