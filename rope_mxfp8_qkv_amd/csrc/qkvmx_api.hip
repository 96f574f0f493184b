// C ABI of the library: host-side validation of every argument (before any HIP call), then the
// kernel launches on the caller's stream.  Declared in include/qkvmx.h.
#include <stdarg.h>
#include <stdio.h>

#include "../../include/qkvmx.h"
#include "internal.h"

using namespace qkvmx;

namespace {

thread_local char g_err[256] = "";

qkvmx_status fail(qkvmx_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

qkvmx_status ok() {
  g_err[0] = '\0';
  return QKVMX_OK;
}

qkvmx_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(QKVMX_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int64_t kMaxRowH = 16384;             // row kernels keep a row in registers
constexpr int64_t kMaxOffset = (int64_t)1 << 31; // 32-bit byte offsets in the projection

}  // namespace

extern "C" {

const char* qkvmx_status_string(qkvmx_status s) {
  switch (s) {
    case QKVMX_OK: return "QKVMX_OK";
    case QKVMX_ERR_NULL: return "QKVMX_ERR_NULL";
    case QKVMX_ERR_SHAPE: return "QKVMX_ERR_SHAPE";
    case QKVMX_ERR_ALIGN: return "QKVMX_ERR_ALIGN";
    case QKVMX_ERR_ARG: return "QKVMX_ERR_ARG";
    case QKVMX_ERR_WORKSPACE: return "QKVMX_ERR_WORKSPACE";
    case QKVMX_ERR_UNSUPPORTED: return "QKVMX_ERR_UNSUPPORTED";
    case QKVMX_ERR_HIP: return "QKVMX_ERR_HIP";
  }
  return "QKVMX_UNKNOWN_STATUS";
}

const char* qkvmx_last_error(void) { return g_err; }

qkvmx_status mx_weight_quantize(const float* w, int64_t H, int64_t I, uint8_t* w_h4_i_4,
                                uint8_t* w_e8m0, hipStream_t stream) {
  if (!w || !w_h4_i_4 || !w_e8m0) return fail(QKVMX_ERR_NULL, "mx_weight_quantize: null pointer");
  if (H <= 0 || I <= 0 || H % 32) return fail(QKVMX_ERR_SHAPE, "mx_weight_quantize: need H %% 32 == 0, H, I > 0");
  if (H / 32 > 65535) return fail(QKVMX_ERR_UNSUPPORTED, "mx_weight_quantize: H too large");
  if (!aligned(w, 4) || !aligned(w_h4_i_4, 4)) return fail(QKVMX_ERR_ALIGN, "mx_weight_quantize: w and codes must be 4-byte aligned");
  return hip_status(launch_mx_weight_quantize(w, H, I, w_h4_i_4, w_e8m0, stream), "mx_weight_quantize");
}

size_t qkv_weight_packed_bytes(int64_t H, int64_t I) {
  if (H <= 0 || I <= 0 || H % 32) return 0;
  return packed_total_bytes(H, I);
}

qkvmx_status qkv_weight_prepack(const uint8_t* w_h4_i_4, const uint8_t* w_e8m0, int64_t H,
                                int64_t I, void* w_packed, size_t w_packed_bytes,
                                hipStream_t stream) {
  if (!w_h4_i_4 || !w_e8m0 || !w_packed) return fail(QKVMX_ERR_NULL, "qkv_weight_prepack: null pointer");
  if (H <= 0 || I <= 0 || H % 32) return fail(QKVMX_ERR_SHAPE, "qkv_weight_prepack: need H %% 32 == 0, H, I > 0");
  if (w_packed_bytes < packed_total_bytes(H, I))
    return fail(QKVMX_ERR_SHAPE, "qkv_weight_prepack: w_packed_bytes %zu < %zu", w_packed_bytes, packed_total_bytes(H, I));
  if (!aligned(w_h4_i_4, 4) || !aligned(w_packed, 256)) return fail(QKVMX_ERR_ALIGN, "qkv_weight_prepack: codes 4-byte, w_packed 256-byte aligned");
  return hip_status(launch_weight_prepack(w_h4_i_4, w_e8m0, H, I, (uint8_t*)w_packed, stream), "qkv_weight_prepack");
}

qkvmx_status row_quantize_packed(const void* x, int32_t x_dtype, int64_t T, int64_t H,
                                 uint8_t* packed_out, hipStream_t stream) {
  if (!x || !packed_out) return fail(QKVMX_ERR_NULL, "row_quantize_packed: null pointer");
  if (x_dtype != QKVMX_DTYPE_F32 && x_dtype != QKVMX_DTYPE_BF16) return fail(QKVMX_ERR_ARG, "row_quantize_packed: bad dtype");
  if (T <= 0 || H <= 0 || H % 32) return fail(QKVMX_ERR_SHAPE, "row_quantize_packed: need T > 0, H %% 32 == 0");
  if (H > kMaxRowH) return fail(QKVMX_ERR_UNSUPPORTED, "row_quantize_packed: H > %lld", (long long)kMaxRowH);
  if (!aligned(x, 16) || !aligned(packed_out, 4)) return fail(QKVMX_ERR_ALIGN, "row_quantize_packed: x 16-byte, packed 4-byte aligned");
  return hip_status(launch_row_quantize(x, x_dtype, T, H, packed_out, stream), "row_quantize_packed");
}

qkvmx_status rmsnorm_mx_quantize(const uint16_t* hidden, const uint16_t* residual,
                                 const uint16_t* gamma, float eps, int64_t T, int64_t H,
                                 int64_t unpadded_H, uint16_t* residual_out, uint8_t* packed_out,
                                 hipStream_t stream) {
  if (!hidden || !gamma || !packed_out) return fail(QKVMX_ERR_NULL, "rmsnorm_mx_quantize: null pointer");
  if (residual && !residual_out) return fail(QKVMX_ERR_ARG, "rmsnorm_mx_quantize: residual_out is required with a residual");
  if (!residual && residual_out) return fail(QKVMX_ERR_ARG, "rmsnorm_mx_quantize: residual_out given without a residual");
  if (T <= 0 || H <= 0 || H % 32) return fail(QKVMX_ERR_SHAPE, "rmsnorm_mx_quantize: need T > 0, H %% 32 == 0");
  if (unpadded_H < 0 || unpadded_H > H) return fail(QKVMX_ERR_SHAPE, "rmsnorm_mx_quantize: unpadded_H outside [0, H]");
  if (!(eps >= 0.0f)) return fail(QKVMX_ERR_ARG, "rmsnorm_mx_quantize: eps must be >= 0");
  if (H > kMaxRowH) return fail(QKVMX_ERR_UNSUPPORTED, "rmsnorm_mx_quantize: H > %lld", (long long)kMaxRowH);
  if (!aligned(hidden, 16) || !aligned(gamma, 16) || (residual && !aligned(residual, 16)) ||
      (residual_out && !aligned(residual_out, 16)) || !aligned(packed_out, 4))
    return fail(QKVMX_ERR_ALIGN, "rmsnorm_mx_quantize: bf16 tensors 16-byte, packed 4-byte aligned");
  const int64_t Hu = unpadded_H ? unpadded_H : H;
  return hip_status(launch_rmsnorm_quantize(hidden, residual, gamma, eps, T, H, Hu, residual_out,
                                            packed_out, stream), "rmsnorm_mx_quantize");
}

size_t qkv_act_image_bytes(int64_t T, int64_t H) {
  if (T <= 0 || H <= 0 || H % 32) return 0;
  return act_image_bytes(T, H);
}

qkvmx_status row_quantize_staged(const void* x, int32_t x_dtype, int64_t T, int64_t H,
                                 uint8_t* act_image, size_t image_bytes, float* row_scale,
                                 hipStream_t stream) {
  const char* fn = "row_quantize_staged";
  if (!x || !act_image || !row_scale) return fail(QKVMX_ERR_NULL, "%s: null pointer", fn);
  if (x_dtype != QKVMX_DTYPE_F32 && x_dtype != QKVMX_DTYPE_BF16) return fail(QKVMX_ERR_ARG, "%s: bad dtype", fn);
  if (T <= 0 || H <= 0 || H % 32) return fail(QKVMX_ERR_SHAPE, "%s: need T > 0, H %% 32 == 0", fn);
  if (H > kMaxRowH) return fail(QKVMX_ERR_UNSUPPORTED, "%s: H > %lld", fn, (long long)kMaxRowH);
  if (ceil_div(T, 256) * 256 > INT32_MAX) return fail(QKVMX_ERR_UNSUPPORTED, "%s: T too large", fn);
  if (image_bytes < act_image_bytes(T, H))
    return fail(QKVMX_ERR_SHAPE, "%s: image_bytes %zu < %zu", fn, image_bytes, act_image_bytes(T, H));
  if (!aligned(x, 16) || !aligned(act_image, 16) || !aligned(row_scale, 4))
    return fail(QKVMX_ERR_ALIGN, "%s: x 16-byte, act_image 16-byte, row_scale 4-byte aligned", fn);
  return hip_status(launch_row_quantize_staged(x, x_dtype, T, H, act_image, row_scale, stream), fn);
}

qkvmx_status rmsnorm_mx_quantize_staged(const uint16_t* hidden, const uint16_t* residual,
                                        const uint16_t* gamma, float eps, int64_t T, int64_t H,
                                        int64_t unpadded_H, uint16_t* residual_out,
                                        uint8_t* act_image, size_t image_bytes, float* row_scale,
                                        hipStream_t stream) {
  const char* fn = "rmsnorm_mx_quantize_staged";
  if (!hidden || !gamma || !act_image || !row_scale) return fail(QKVMX_ERR_NULL, "%s: null pointer", fn);
  if (residual && !residual_out) return fail(QKVMX_ERR_ARG, "%s: residual_out is required with a residual", fn);
  if (!residual && residual_out) return fail(QKVMX_ERR_ARG, "%s: residual_out given without a residual", fn);
  if (T <= 0 || H <= 0 || H % 32) return fail(QKVMX_ERR_SHAPE, "%s: need T > 0, H %% 32 == 0", fn);
  if (unpadded_H < 0 || unpadded_H > H) return fail(QKVMX_ERR_SHAPE, "%s: unpadded_H outside [0, H]", fn);
  if (!(eps >= 0.0f)) return fail(QKVMX_ERR_ARG, "%s: eps must be >= 0", fn);
  if (H > kMaxRowH) return fail(QKVMX_ERR_UNSUPPORTED, "%s: H > %lld", fn, (long long)kMaxRowH);
  if (ceil_div(T, 256) * 256 > INT32_MAX) return fail(QKVMX_ERR_UNSUPPORTED, "%s: T too large", fn);
  if (image_bytes < act_image_bytes(T, H))
    return fail(QKVMX_ERR_SHAPE, "%s: image_bytes %zu < %zu", fn, image_bytes, act_image_bytes(T, H));
  if (!aligned(hidden, 16) || !aligned(gamma, 16) || (residual && !aligned(residual, 16)) ||
      (residual_out && !aligned(residual_out, 16)) || !aligned(act_image, 16) || !aligned(row_scale, 4))
    return fail(QKVMX_ERR_ALIGN, "%s: bf16 tensors 16-byte, act_image 16-byte, row_scale 4-byte aligned", fn);
  const int64_t Hu = unpadded_H ? unpadded_H : H;
  return hip_status(launch_rmsnorm_quantize_staged(hidden, residual, gamma, eps, T, H, Hu,
                                                   residual_out, act_image, row_scale, stream), fn);
}

qkvmx_status mx_block_quantize(const void* x, int32_t x_dtype, int64_t T, int64_t H,
                               uint8_t* codes_out, uint8_t* e8m0_out, hipStream_t stream) {
  if (!x || !codes_out || !e8m0_out) return fail(QKVMX_ERR_NULL, "mx_block_quantize: null pointer");
  if (x_dtype != QKVMX_DTYPE_F32 && x_dtype != QKVMX_DTYPE_BF16) return fail(QKVMX_ERR_ARG, "mx_block_quantize: bad dtype");
  if (T <= 0 || H <= 0 || H % 32) return fail(QKVMX_ERR_SHAPE, "mx_block_quantize: need T > 0, H %% 32 == 0");
  if (H > kMaxRowH) return fail(QKVMX_ERR_UNSUPPORTED, "mx_block_quantize: H > %lld", (long long)kMaxRowH);
  if (!aligned(x, 16) || !aligned(codes_out, 8) || !aligned(e8m0_out, 4))
    return fail(QKVMX_ERR_ALIGN, "mx_block_quantize: x 16-byte, codes 8-byte, exponents 4-byte aligned");
  return hip_status(launch_mx_quantize(x, x_dtype, T, H, codes_out, e8m0_out, stream), "mx_block_quantize");
}

qkvmx_status rmsnorm_mx_block_quantize(const uint16_t* hidden, const uint16_t* residual,
                                       const uint16_t* gamma, float eps, int64_t T, int64_t H,
                                       int64_t unpadded_H, uint16_t* residual_out,
                                       uint8_t* codes_out, uint8_t* e8m0_out, uint16_t* norm_out,
                                       hipStream_t stream) {
  if (!hidden || !gamma || !codes_out || !e8m0_out) return fail(QKVMX_ERR_NULL, "rmsnorm_mx_block_quantize: null pointer");
  if (residual && !residual_out) return fail(QKVMX_ERR_ARG, "rmsnorm_mx_block_quantize: residual_out is required with a residual");
  if (!residual && residual_out) return fail(QKVMX_ERR_ARG, "rmsnorm_mx_block_quantize: residual_out given without a residual");
  if (T <= 0 || H <= 0 || H % 32) return fail(QKVMX_ERR_SHAPE, "rmsnorm_mx_block_quantize: need T > 0, H %% 32 == 0");
  if (unpadded_H < 0 || unpadded_H > H) return fail(QKVMX_ERR_SHAPE, "rmsnorm_mx_block_quantize: unpadded_H outside [0, H]");
  if (!(eps >= 0.0f)) return fail(QKVMX_ERR_ARG, "rmsnorm_mx_block_quantize: eps must be >= 0");
  if (H > kMaxRowH) return fail(QKVMX_ERR_UNSUPPORTED, "rmsnorm_mx_block_quantize: H > %lld", (long long)kMaxRowH);
  if (!aligned(hidden, 16) || !aligned(gamma, 16) || (residual && !aligned(residual, 16)) ||
      (residual_out && !aligned(residual_out, 16)) || (norm_out && !aligned(norm_out, 16)) ||
      !aligned(codes_out, 8) || !aligned(e8m0_out, 4))
    return fail(QKVMX_ERR_ALIGN, "rmsnorm_mx_block_quantize: bf16 tensors 16-byte, codes 8-byte, exponents 4-byte aligned");
  const int64_t Hu = unpadded_H ? unpadded_H : H;
  return hip_status(launch_rmsnorm_mx(hidden, residual, gamma, eps, T, H, Hu, residual_out,
                                      codes_out, e8m0_out, norm_out, stream), "rmsnorm_mx_block_quantize");
}

size_t qkv_act_exp_image_bytes(int64_t T, int64_t H) {
  if (T <= 0 || H <= 0 || H % 32) return 0;
  return mx_scale_image_bytes(T, H);
}

qkvmx_status mx_block_quantize_staged(const void* x, int32_t x_dtype, int64_t T, int64_t H,
                                      uint8_t* act_image, size_t image_bytes, uint32_t* exp_image,
                                      size_t exp_image_bytes, hipStream_t stream) {
  const char* fn = "mx_block_quantize_staged";
  if (!x || !act_image || !exp_image) return fail(QKVMX_ERR_NULL, "%s: null pointer", fn);
  if (x_dtype != QKVMX_DTYPE_F32 && x_dtype != QKVMX_DTYPE_BF16) return fail(QKVMX_ERR_ARG, "%s: bad dtype", fn);
  if (T <= 0 || H <= 0 || H % 32) return fail(QKVMX_ERR_SHAPE, "%s: need T > 0, H %% 32 == 0", fn);
  if (H > kMaxRowH) return fail(QKVMX_ERR_UNSUPPORTED, "%s: H > %lld", fn, (long long)kMaxRowH);
  if (ceil_div(T, 256) * 256 > INT32_MAX) return fail(QKVMX_ERR_UNSUPPORTED, "%s: T too large", fn);
  if (image_bytes < act_image_bytes(T, H) || exp_image_bytes < mx_scale_image_bytes(T, H))
    return fail(QKVMX_ERR_SHAPE, "%s: images need %zu and %zu bytes", fn, act_image_bytes(T, H), mx_scale_image_bytes(T, H));
  if (!aligned(x, 16) || !aligned(act_image, 16) || !aligned(exp_image, 16))
    return fail(QKVMX_ERR_ALIGN, "%s: x, act_image and exp_image 16-byte aligned", fn);
  return hip_status(launch_mx_quantize_staged(x, x_dtype, T, H, act_image, exp_image, stream), fn);
}

qkvmx_status rmsnorm_mx_block_quantize_staged(const uint16_t* hidden, const uint16_t* residual,
                                              const uint16_t* gamma, float eps, int64_t T,
                                              int64_t H, int64_t unpadded_H,
                                              uint16_t* residual_out, uint8_t* act_image,
                                              size_t image_bytes, uint32_t* exp_image,
                                              size_t exp_image_bytes, uint16_t* norm_out,
                                              hipStream_t stream) {
  const char* fn = "rmsnorm_mx_block_quantize_staged";
  if (!hidden || !gamma || !act_image || !exp_image) return fail(QKVMX_ERR_NULL, "%s: null pointer", fn);
  if (residual && !residual_out) return fail(QKVMX_ERR_ARG, "%s: residual_out is required with a residual", fn);
  if (!residual && residual_out) return fail(QKVMX_ERR_ARG, "%s: residual_out given without a residual", fn);
  if (T <= 0 || H <= 0 || H % 32) return fail(QKVMX_ERR_SHAPE, "%s: need T > 0, H %% 32 == 0", fn);
  if (unpadded_H < 0 || unpadded_H > H) return fail(QKVMX_ERR_SHAPE, "%s: unpadded_H outside [0, H]", fn);
  if (!(eps >= 0.0f)) return fail(QKVMX_ERR_ARG, "%s: eps must be >= 0", fn);
  if (H > kMaxRowH) return fail(QKVMX_ERR_UNSUPPORTED, "%s: H > %lld", fn, (long long)kMaxRowH);
  if (ceil_div(T, 256) * 256 > INT32_MAX) return fail(QKVMX_ERR_UNSUPPORTED, "%s: T too large", fn);
  if (image_bytes < act_image_bytes(T, H) || exp_image_bytes < mx_scale_image_bytes(T, H))
    return fail(QKVMX_ERR_SHAPE, "%s: images need %zu and %zu bytes", fn, act_image_bytes(T, H), mx_scale_image_bytes(T, H));
  if (!aligned(hidden, 16) || !aligned(gamma, 16) || (residual && !aligned(residual, 16)) ||
      (residual_out && !aligned(residual_out, 16)) || (norm_out && !aligned(norm_out, 16)) ||
      !aligned(act_image, 16) || !aligned(exp_image, 16))
    return fail(QKVMX_ERR_ALIGN, "%s: bf16 tensors, act_image and exp_image 16-byte aligned", fn);
  const int64_t Hu = unpadded_H ? unpadded_H : H;
  return hip_status(launch_rmsnorm_mx_staged(hidden, residual, gamma, eps, T, H, Hu, residual_out,
                                             act_image, exp_image, norm_out, stream), fn);
}

size_t qkvmx_workspace_bytes(int64_t T, int64_t H, int64_t I) {
  if (T <= 0 || H <= 0 || I <= 0 || H % 32) return 0;
  return workspace_total_bytes(T, H, I);
}

qkvmx_status qkv_rowmx_project(const uint8_t* a_codes, int64_t a_row_stride,
                               const uint8_t* a_scales, int64_t a_scale_stride,
                               const void* w_packed, const float* w_channel_scale,
                               const uint16_t* bias, int64_t T, int64_t H, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t layout,
                               uint16_t* out, float* ssq, void* workspace, size_t ws_bytes,
                               hipStream_t stream) {
  if (!a_codes || !a_scales || !w_packed || !out) return fail(QKVMX_ERR_NULL, "qkv_rowmx_project: null pointer");
  if (!workspace) return fail(QKVMX_ERR_WORKSPACE, "qkv_rowmx_project: workspace is required");
  if (T <= 0 || H <= 0 || H % 32) return fail(QKVMX_ERR_SHAPE, "qkv_rowmx_project: need T > 0, H %% 32 == 0");
  if (num_heads < 1 || num_kv_heads < 0 || head_dim <= 0 || head_dim % 16)
    return fail(QKVMX_ERR_SHAPE, "qkv_rowmx_project: need num_heads >= 1, num_kv_heads >= 0, head_dim %% 16 == 0");
  if (layout != QKVMX_LAYOUT_BSD && layout != QKVMX_LAYOUT_NBSD)
    return fail(QKVMX_ERR_ARG, "qkv_rowmx_project: layout must be QKVMX_LAYOUT_BSD or QKVMX_LAYOUT_NBSD");
  if (a_row_stride < H || a_row_stride % 4 || a_scale_stride <= 0 || a_scale_stride % 4)
    return fail(QKVMX_ERR_SHAPE, "qkv_rowmx_project: a_row_stride >= H and strides multiples of 4");
  const int64_t I = (int64_t)(num_heads + 2 * (int64_t)num_kv_heads) * head_dim;
  if ((T - 1) * a_row_stride + H >= kMaxOffset)
    return fail(QKVMX_ERR_UNSUPPORTED, "qkv_rowmx_project: activation span must be < 2^31 bytes");
  if (I * 2 * 256 >= kMaxOffset)     // byte offsets within one 256-token output tile
    return fail(QKVMX_ERR_UNSUPPORTED, "qkv_rowmx_project: I must be < 2^22");
  // NBSd: byte offsets from a tile's first head to the rows it writes
  if (layout == QKVMX_LAYOUT_NBSD && 2 * ((256 + (int64_t)head_dim) * T + 257 * (int64_t)head_dim) >= kMaxOffset)
    return fail(QKVMX_ERR_UNSUPPORTED, "qkv_rowmx_project: NBSd needs 2 ((256 + head_dim) T + 257 head_dim) < 2^31");
  if (ws_bytes < workspace_total_bytes(T, H, I))
    return fail(QKVMX_ERR_WORKSPACE, "qkv_rowmx_project: workspace %zu < %zu bytes", ws_bytes, workspace_total_bytes(T, H, I));
  if (!aligned(a_codes, 4) || !aligned(a_scales, 4) || !aligned(w_packed, 256) ||
      (w_channel_scale && !aligned(w_channel_scale, 16)) || (bias && !aligned(bias, 8)) ||
      !aligned(out, 16) || (ssq && !aligned(ssq, 8)) || !aligned(workspace, 256))
    return fail(QKVMX_ERR_ALIGN, "qkv_rowmx_project: alignment (codes/scales 4, w_packed 256, channel scale 16, bias 8, out 16, ssq 8, workspace 256)");
  const int64_t Iq = (int64_t)num_heads * head_dim, Ik = (int64_t)num_kv_heads * head_dim;
  return hip_status(launch_project(a_codes, a_row_stride, a_scales, a_scale_stride,
                                   (const uint8_t*)w_packed, w_channel_scale, bias, T, H, I, Iq,
                                   Ik, head_dim, layout == QKVMX_LAYOUT_NBSD, out, ssq,
                                   (uint8_t*)workspace, stream), "qkv_rowmx_project");
}

size_t qkv_staged_workspace_bytes(int64_t T, int64_t I) {
  if (T <= 0 || I <= 0) return 0;
  return staged_workspace_total_bytes(T, I);
}

int32_t qkvmx_projection_k_chunks(int64_t T, int64_t H, int64_t I, int32_t layout) {
  if (T <= 0 || H <= 0 || H % 32 || I <= 0 || I % 16) return 0;
  if (layout != QKVMX_LAYOUT_BSD && layout != QKVMX_LAYOUT_NBSD) return 0;
  return split_plan(T, H, I).chunks;
}

qkvmx_status qkv_rowmx_project_staged(const uint8_t* act_image, size_t image_bytes,
                                      const float* row_scale, const void* w_packed,
                                      const float* w_channel_scale, const uint16_t* bias,
                                      int64_t T, int64_t H, int32_t num_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t layout,
                                      uint16_t* out, float* ssq, void* workspace,
                                      size_t ws_bytes, hipStream_t stream) {
  const char* fn = "qkv_rowmx_project_staged";
  if (!act_image || !row_scale || !w_packed || !out) return fail(QKVMX_ERR_NULL, "%s: null pointer", fn);
  if (!workspace) return fail(QKVMX_ERR_WORKSPACE, "%s: workspace is required", fn);
  if (T <= 0 || H <= 0 || H % 32) return fail(QKVMX_ERR_SHAPE, "%s: need T > 0, H %% 32 == 0", fn);
  if (num_heads < 1 || num_kv_heads < 0 || head_dim <= 0 || head_dim % 16)
    return fail(QKVMX_ERR_SHAPE, "%s: need num_heads >= 1, num_kv_heads >= 0, head_dim %% 16 == 0", fn);
  if (layout != QKVMX_LAYOUT_BSD && layout != QKVMX_LAYOUT_NBSD)
    return fail(QKVMX_ERR_ARG, "%s: layout must be QKVMX_LAYOUT_BSD or QKVMX_LAYOUT_NBSD", fn);
  if (image_bytes < act_image_bytes(T, H))
    return fail(QKVMX_ERR_SHAPE, "%s: image_bytes %zu < %zu", fn, image_bytes, act_image_bytes(T, H));
  const int64_t I = (int64_t)(num_heads + 2 * (int64_t)num_kv_heads) * head_dim;
  if (I * 2 * 256 >= kMaxOffset)
    return fail(QKVMX_ERR_UNSUPPORTED, "%s: I must be < 2^22", fn);
  if (layout == QKVMX_LAYOUT_NBSD && 2 * ((256 + (int64_t)head_dim) * T + 257 * (int64_t)head_dim) >= kMaxOffset)
    return fail(QKVMX_ERR_UNSUPPORTED, "%s: NBSd needs 2 ((256 + head_dim) T + 257 head_dim) < 2^31", fn);
  if (ws_bytes < staged_workspace_total_bytes(T, I))
    return fail(QKVMX_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, staged_workspace_total_bytes(T, I));
  if (!aligned(act_image, 256) || !aligned(row_scale, 4) || !aligned(w_packed, 256) ||
      (w_channel_scale && !aligned(w_channel_scale, 16)) || (bias && !aligned(bias, 8)) ||
      !aligned(out, 16) || (ssq && !aligned(ssq, 8)) || !aligned(workspace, 256))
    return fail(QKVMX_ERR_ALIGN, "%s: alignment (act_image 256, row_scale 4, w_packed 256, channel scale 16, bias 8, out 16, ssq 8, workspace 256)", fn);
  const int64_t Iq = (int64_t)num_heads * head_dim, Ik = (int64_t)num_kv_heads * head_dim;
  return hip_status(launch_project_staged(act_image, row_scale, (const uint8_t*)w_packed,
                                          w_channel_scale, bias, T, H, I, Iq, Ik, head_dim,
                                          layout == QKVMX_LAYOUT_NBSD, out, ssq,
                                          (uint8_t*)workspace, stream), fn);
}

size_t qkvmx_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

qkvmx_status qkv_rowmx_project_staged_noalloc(const uint8_t* act_image, size_t image_bytes,
                                              const float* row_scale, const void* w_packed,
                                              const float* w_channel_scale, const uint16_t* bias,
                                              int64_t T, int64_t H, int32_t num_heads,
                                              int32_t num_kv_heads, int32_t head_dim,
                                              int32_t layout, uint16_t* out, float* ssq,
                                              hipStream_t stream) {
  const char* fn = "qkv_rowmx_project_staged_noalloc";
  if (!act_image || !row_scale || !w_packed || !out) return fail(QKVMX_ERR_NULL, "%s: null pointer", fn);
  if (T <= 0 || H <= 0 || H % 32) return fail(QKVMX_ERR_SHAPE, "%s: need T > 0, H %% 32 == 0", fn);
  if (num_heads < 1 || num_kv_heads < 0 || head_dim <= 0 || head_dim % 16)
    return fail(QKVMX_ERR_SHAPE, "%s: need num_heads >= 1, num_kv_heads >= 0, head_dim %% 16 == 0", fn);
  if (layout != QKVMX_LAYOUT_BSD && layout != QKVMX_LAYOUT_NBSD)
    return fail(QKVMX_ERR_ARG, "%s: layout must be QKVMX_LAYOUT_BSD or QKVMX_LAYOUT_NBSD", fn);
  const int64_t I = (int64_t)(num_heads + 2 * (int64_t)num_kv_heads) * head_dim;
  if (I * 2 * 256 >= kMaxOffset)
    return fail(QKVMX_ERR_UNSUPPORTED, "%s: I must be < 2^22", fn);
  if (staged_workspace_total_bytes(T, I) > kNoAllocScratchBytes)
    return fail(QKVMX_ERR_WORKSPACE,
                "%s: T = %lld, I = %lld needs %zu bytes of scratch; the static scratch holds %zu "
                "(use qkv_rowmx_project_staged with a workspace)", fn, (long long)T,
                (long long)I, staged_workspace_total_bytes(T, I), kNoAllocScratchBytes);
  if (image_bytes < act_image_bytes(T, H))
    return fail(QKVMX_ERR_SHAPE, "%s: image_bytes %zu < %zu", fn, image_bytes, act_image_bytes(T, H));
  if (layout == QKVMX_LAYOUT_NBSD && 2 * ((256 + (int64_t)head_dim) * T + 257 * (int64_t)head_dim) >= kMaxOffset)
    return fail(QKVMX_ERR_UNSUPPORTED, "%s: NBSd needs 2 ((256 + head_dim) T + 257 head_dim) < 2^31", fn);
  if (!aligned(act_image, 256) || !aligned(row_scale, 4) || !aligned(w_packed, 256) ||
      (w_channel_scale && !aligned(w_channel_scale, 16)) || (bias && !aligned(bias, 8)) ||
      !aligned(out, 16) || (ssq && !aligned(ssq, 8)))
    return fail(QKVMX_ERR_ALIGN, "%s: alignment (act_image 256, row_scale 4, w_packed 256, channel scale 16, bias 8, out 16, ssq 8)", fn);
  void* scratch = nullptr;
  const qkvmx_status st = hip_status(noalloc_scratch(&scratch), fn);
  if (st != QKVMX_OK) return st;
  const int64_t Iq = (int64_t)num_heads * head_dim, Ik = (int64_t)num_kv_heads * head_dim;
  return hip_status(launch_project_staged(act_image, row_scale, (const uint8_t*)w_packed,
                                          w_channel_scale, bias, T, H, I, Iq, Ik, head_dim,
                                          layout == QKVMX_LAYOUT_NBSD, out, ssq,
                                          (uint8_t*)scratch, stream), fn);
}

// Checks shared by the two per-head qk-norm projections (norm kind, shapes, the head geometry
// the fused epilogue supports, layout, gamma / beta / table pairing, eps); QKVMX_OK if they hold.
static qkvmx_status check_headnorm(const char* fn, int64_t T, int64_t H, int32_t num_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t layout,
                                   int32_t norm_kind, const uint16_t* q_gamma,
                                   const uint16_t* k_gamma, const uint16_t* q_beta,
                                   const uint16_t* k_beta, float eps, const float* cos_tab,
                                   const float* sin_tab) {
  if (norm_kind != QKVMX_HEAD_RMS_NORM && norm_kind != QKVMX_HEAD_LAYER_NORM)
    return fail(QKVMX_ERR_ARG, "%s: norm_kind must be QKVMX_HEAD_RMS_NORM or QKVMX_HEAD_LAYER_NORM", fn);
  if (T <= 0 || H <= 0 || H % 32) return fail(QKVMX_ERR_SHAPE, "%s: need T > 0, H %% 32 == 0", fn);
  if (num_heads < 1 || num_kv_heads < 0) return fail(QKVMX_ERR_SHAPE, "%s: need num_heads >= 1, num_kv_heads >= 0", fn);
  if (head_dim != 64 && head_dim != 128)
    return fail(QKVMX_ERR_UNSUPPORTED, "%s: head_dim must be 64 or 128", fn);
  if (((int64_t)num_heads * head_dim) % 128 || ((int64_t)num_kv_heads * head_dim) % 128)
    return fail(QKVMX_ERR_UNSUPPORTED, "%s: the Q and K segments must be multiples of 128 channels", fn);
  if (layout != QKVMX_LAYOUT_BSD && layout != QKVMX_LAYOUT_NBSD)
    return fail(QKVMX_ERR_ARG, "%s: layout must be QKVMX_LAYOUT_BSD or QKVMX_LAYOUT_NBSD", fn);
  if (!q_gamma || (num_kv_heads > 0) != (k_gamma != nullptr))
    return fail(QKVMX_ERR_ARG, "%s: q_gamma is required, k_gamma iff num_kv_heads > 0", fn);
  if (norm_kind != QKVMX_HEAD_LAYER_NORM && (q_beta || k_beta))
    return fail(QKVMX_ERR_ARG, "%s: beta belongs to QKVMX_HEAD_LAYER_NORM", fn);
  if (k_beta && num_kv_heads == 0) return fail(QKVMX_ERR_ARG, "%s: k_beta without a K segment", fn);
  if ((cos_tab == nullptr) != (sin_tab == nullptr)) return fail(QKVMX_ERR_ARG, "%s: cos_tab and sin_tab come together", fn);
  if (!(eps >= 0.0f)) return fail(QKVMX_ERR_ARG, "%s: eps must be >= 0", fn);
  return QKVMX_OK;
}

qkvmx_status qkv_rowmx_project_headnorm(const uint8_t* a_codes, int64_t a_row_stride,
                                         const uint8_t* a_scales, int64_t a_scale_stride,
                                         const void* w_packed, const uint16_t* bias, int64_t T,
                                         int64_t H, int32_t num_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t layout, int32_t norm_kind,
                                         const uint16_t* q_gamma, const uint16_t* k_gamma,
                                         const uint16_t* q_beta, const uint16_t* k_beta,
                                         float eps, const float* cos_tab, const float* sin_tab,
                                         uint16_t* out, void* workspace, size_t ws_bytes,
                                         hipStream_t stream) {
  const char* fn = "qkv_rowmx_project_headnorm";
  if (!a_codes || !a_scales || !w_packed || !out) return fail(QKVMX_ERR_NULL, "%s: null pointer", fn);
  if (!workspace) return fail(QKVMX_ERR_WORKSPACE, "%s: workspace is required", fn);
  const qkvmx_status hs = check_headnorm(fn, T, H, num_heads, num_kv_heads, head_dim, layout,
                                         norm_kind, q_gamma, k_gamma, q_beta, k_beta, eps,
                                         cos_tab, sin_tab);
  if (hs != QKVMX_OK) return hs;
  if (a_row_stride < H || a_row_stride % 4 || a_scale_stride <= 0 || a_scale_stride % 4)
    return fail(QKVMX_ERR_SHAPE, "%s: a_row_stride >= H and strides multiples of 4", fn);
  const int64_t I = (int64_t)(num_heads + 2 * (int64_t)num_kv_heads) * head_dim;
  if ((T - 1) * a_row_stride + H >= kMaxOffset) return fail(QKVMX_ERR_UNSUPPORTED, "%s: activation span must be < 2^31 bytes", fn);
  if (I * 2 * 256 >= kMaxOffset) return fail(QKVMX_ERR_UNSUPPORTED, "%s: I must be < 2^22", fn);
  if (layout == QKVMX_LAYOUT_NBSD && 2 * ((256 + (int64_t)head_dim) * T + 257 * (int64_t)head_dim) >= kMaxOffset)
    return fail(QKVMX_ERR_UNSUPPORTED, "%s: NBSd needs 2 ((256 + head_dim) T + 257 head_dim) < 2^31", fn);
  if (ws_bytes < workspace_total_bytes(T, H, I))
    return fail(QKVMX_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, workspace_total_bytes(T, H, I));
  if (!aligned(a_codes, 4) || !aligned(a_scales, 4) || !aligned(w_packed, 256) ||
      (bias && !aligned(bias, 8)) || !aligned(out, 16) || !aligned(workspace, 256) ||
      !aligned(q_gamma, 8) || (k_gamma && !aligned(k_gamma, 8)) || (q_beta && !aligned(q_beta, 8)) ||
      (k_beta && !aligned(k_beta, 8)) || (cos_tab && !aligned(cos_tab, 16)) || (sin_tab && !aligned(sin_tab, 16)))
    return fail(QKVMX_ERR_ALIGN, "%s: alignment (codes/scales 4, w_packed 256, bias/gamma/beta 8, out/tables 16, workspace 256)", fn);
  const int64_t Iq = (int64_t)num_heads * head_dim, Ik = (int64_t)num_kv_heads * head_dim;
  return hip_status(launch_project_headnorm(a_codes, a_row_stride, a_scales, a_scale_stride,
                                            (const uint8_t*)w_packed, bias, T, H, I, Iq, Ik,
                                            head_dim, layout == QKVMX_LAYOUT_NBSD, norm_kind,
                                            q_gamma, k_gamma, q_beta, k_beta, eps, cos_tab,
                                            sin_tab, out, (uint8_t*)workspace, stream), fn);
}

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
                                                hipStream_t stream) {
  const char* fn = "qkv_rowmx_project_headnorm_staged";
  if (!act_image || !row_scale || !w_packed || !out) return fail(QKVMX_ERR_NULL, "%s: null pointer", fn);
  if (!workspace) return fail(QKVMX_ERR_WORKSPACE, "%s: workspace is required", fn);
  const qkvmx_status hs = check_headnorm(fn, T, H, num_heads, num_kv_heads, head_dim, layout,
                                         norm_kind, q_gamma, k_gamma, q_beta, k_beta, eps,
                                         cos_tab, sin_tab);
  if (hs != QKVMX_OK) return hs;
  if (image_bytes < act_image_bytes(T, H))
    return fail(QKVMX_ERR_SHAPE, "%s: image_bytes %zu < %zu", fn, image_bytes, act_image_bytes(T, H));
  const int64_t I = (int64_t)(num_heads + 2 * (int64_t)num_kv_heads) * head_dim;
  if (I * 2 * 256 >= kMaxOffset) return fail(QKVMX_ERR_UNSUPPORTED, "%s: I must be < 2^22", fn);
  if (layout == QKVMX_LAYOUT_NBSD && 2 * ((256 + (int64_t)head_dim) * T + 257 * (int64_t)head_dim) >= kMaxOffset)
    return fail(QKVMX_ERR_UNSUPPORTED, "%s: NBSd needs 2 ((256 + head_dim) T + 257 head_dim) < 2^31", fn);
  if (ws_bytes < staged_workspace_total_bytes(T, I))
    return fail(QKVMX_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, staged_workspace_total_bytes(T, I));
  if (!aligned(act_image, 256) || !aligned(row_scale, 4) || !aligned(w_packed, 256) ||
      (bias && !aligned(bias, 8)) || !aligned(out, 16) || !aligned(workspace, 256) ||
      !aligned(q_gamma, 8) || (k_gamma && !aligned(k_gamma, 8)) || (q_beta && !aligned(q_beta, 8)) ||
      (k_beta && !aligned(k_beta, 8)) || (cos_tab && !aligned(cos_tab, 16)) || (sin_tab && !aligned(sin_tab, 16)))
    return fail(QKVMX_ERR_ALIGN, "%s: alignment (act_image/w_packed/workspace 256, row_scale 4, bias/gamma/beta 8, out/tables 16)", fn);
  const int64_t Iq = (int64_t)num_heads * head_dim, Ik = (int64_t)num_kv_heads * head_dim;
  return hip_status(launch_project_headnorm_staged(act_image, row_scale, (const uint8_t*)w_packed,
                                                   bias, T, H, I, Iq, Ik, head_dim,
                                                   layout == QKVMX_LAYOUT_NBSD, norm_kind,
                                                   q_gamma, k_gamma, q_beta, k_beta, eps,
                                                   cos_tab, sin_tab, out, (uint8_t*)workspace,
                                                   stream), fn);
}

size_t qkv_mx_workspace_bytes(int64_t T, int64_t H, int64_t I) {
  if (T <= 0 || H <= 0 || I <= 0 || H % 32) return 0;
  return mx_workspace_total_bytes(T, H, I);
}

qkvmx_status qkv_mx_project(const uint8_t* a_codes, int64_t a_row_stride, const uint8_t* a_e8m0,
                            int64_t a_e8m0_stride, const void* w_packed,
                            const float* w_channel_scale, const uint16_t* bias, int64_t T,
                            int64_t H, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t layout, uint16_t* out, float* ssq, void* workspace,
                            size_t ws_bytes, hipStream_t stream) {
  if (!a_codes || !a_e8m0 || !w_packed || !out) return fail(QKVMX_ERR_NULL, "qkv_mx_project: null pointer");
  if (!workspace) return fail(QKVMX_ERR_WORKSPACE, "qkv_mx_project: workspace is required");
  if (T <= 0 || H <= 0 || H % 32) return fail(QKVMX_ERR_SHAPE, "qkv_mx_project: need T > 0, H %% 32 == 0");
  if (num_heads < 1 || num_kv_heads < 0 || head_dim <= 0 || head_dim % 16)
    return fail(QKVMX_ERR_SHAPE, "qkv_mx_project: need num_heads >= 1, num_kv_heads >= 0, head_dim %% 16 == 0");
  if (layout != QKVMX_LAYOUT_BSD && layout != QKVMX_LAYOUT_NBSD)
    return fail(QKVMX_ERR_ARG, "qkv_mx_project: layout must be QKVMX_LAYOUT_BSD or QKVMX_LAYOUT_NBSD");
  if (a_row_stride < H || a_row_stride % 4 || a_e8m0_stride < H / 32)
    return fail(QKVMX_ERR_SHAPE, "qkv_mx_project: a_row_stride >= H and a multiple of 4, a_e8m0_stride >= H / 32");
  const int64_t I = (int64_t)(num_heads + 2 * (int64_t)num_kv_heads) * head_dim;
  if ((T - 1) * a_row_stride + H >= kMaxOffset || (T - 1) * a_e8m0_stride + H / 32 >= kMaxOffset)
    return fail(QKVMX_ERR_UNSUPPORTED, "qkv_mx_project: activation spans must be < 2^31 bytes");
  if (I * 2 * 256 >= kMaxOffset)
    return fail(QKVMX_ERR_UNSUPPORTED, "qkv_mx_project: I must be < 2^22");
  if (layout == QKVMX_LAYOUT_NBSD && 2 * ((256 + (int64_t)head_dim) * T + 257 * (int64_t)head_dim) >= kMaxOffset)
    return fail(QKVMX_ERR_UNSUPPORTED, "qkv_mx_project: NBSd needs 2 ((256 + head_dim) T + 257 head_dim) < 2^31");
  if (ws_bytes < mx_workspace_total_bytes(T, H, I))
    return fail(QKVMX_ERR_WORKSPACE, "qkv_mx_project: workspace %zu < %zu bytes", ws_bytes, mx_workspace_total_bytes(T, H, I));
  if (!aligned(a_codes, 4) || !aligned(w_packed, 256) ||
      (w_channel_scale && !aligned(w_channel_scale, 16)) || (bias && !aligned(bias, 8)) ||
      !aligned(out, 16) || (ssq && !aligned(ssq, 8)) || !aligned(workspace, 256))
    return fail(QKVMX_ERR_ALIGN, "qkv_mx_project: alignment (codes 4, w_packed 256, channel scale 16, bias 8, out 16, ssq 8, workspace 256)");
  const int64_t Iq = (int64_t)num_heads * head_dim, Ik = (int64_t)num_kv_heads * head_dim;
  return hip_status(launch_project_mx(a_codes, a_row_stride, a_e8m0, a_e8m0_stride,
                                      (const uint8_t*)w_packed, w_channel_scale, bias, T, H, I,
                                      Iq, Ik, head_dim, layout == QKVMX_LAYOUT_NBSD, out, ssq,
                                      (uint8_t*)workspace, stream), "qkv_mx_project");
}

qkvmx_status qkv_mx_project_staged(const uint8_t* act_image, size_t image_bytes,
                                   const uint32_t* exp_image, size_t exp_image_bytes,
                                   const void* w_packed, const float* w_channel_scale,
                                   const uint16_t* bias, int64_t T, int64_t H, int32_t num_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t layout,
                                   uint16_t* out, float* ssq, void* workspace, size_t ws_bytes,
                                   hipStream_t stream) {
  const char* fn = "qkv_mx_project_staged";
  if (!act_image || !exp_image || !w_packed || !out) return fail(QKVMX_ERR_NULL, "%s: null pointer", fn);
  if (!workspace) return fail(QKVMX_ERR_WORKSPACE, "%s: workspace is required", fn);
  if (T <= 0 || H <= 0 || H % 32) return fail(QKVMX_ERR_SHAPE, "%s: need T > 0, H %% 32 == 0", fn);
  if (num_heads < 1 || num_kv_heads < 0 || head_dim <= 0 || head_dim % 16)
    return fail(QKVMX_ERR_SHAPE, "%s: need num_heads >= 1, num_kv_heads >= 0, head_dim %% 16 == 0", fn);
  if (layout != QKVMX_LAYOUT_BSD && layout != QKVMX_LAYOUT_NBSD)
    return fail(QKVMX_ERR_ARG, "%s: layout must be QKVMX_LAYOUT_BSD or QKVMX_LAYOUT_NBSD", fn);
  if (image_bytes < act_image_bytes(T, H) || exp_image_bytes < mx_scale_image_bytes(T, H))
    return fail(QKVMX_ERR_SHAPE, "%s: images need %zu and %zu bytes", fn, act_image_bytes(T, H), mx_scale_image_bytes(T, H));
  const int64_t I = (int64_t)(num_heads + 2 * (int64_t)num_kv_heads) * head_dim;
  if (I * 2 * 256 >= kMaxOffset) return fail(QKVMX_ERR_UNSUPPORTED, "%s: I must be < 2^22", fn);
  if (layout == QKVMX_LAYOUT_NBSD && 2 * ((256 + (int64_t)head_dim) * T + 257 * (int64_t)head_dim) >= kMaxOffset)
    return fail(QKVMX_ERR_UNSUPPORTED, "%s: NBSd needs 2 ((256 + head_dim) T + 257 head_dim) < 2^31", fn);
  if (ws_bytes < staged_workspace_total_bytes(T, I))
    return fail(QKVMX_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, staged_workspace_total_bytes(T, I));
  if (!aligned(act_image, 256) || !aligned(exp_image, 256) || !aligned(w_packed, 256) ||
      (w_channel_scale && !aligned(w_channel_scale, 16)) || (bias && !aligned(bias, 8)) ||
      !aligned(out, 16) || (ssq && !aligned(ssq, 8)) || !aligned(workspace, 256))
    return fail(QKVMX_ERR_ALIGN, "%s: alignment (images 256, w_packed 256, channel scale 16, bias 8, out 16, ssq 8, workspace 256)", fn);
  const int64_t Iq = (int64_t)num_heads * head_dim, Ik = (int64_t)num_kv_heads * head_dim;
  return hip_status(launch_project_mx_staged(act_image, exp_image, (const uint8_t*)w_packed,
                                             w_channel_scale, bias, T, H, I, Iq, Ik, head_dim,
                                             layout == QKVMX_LAYOUT_NBSD, out, ssq,
                                             (uint8_t*)workspace, stream), fn);
}

qkvmx_status qk_norm_rope_apply(uint16_t* qkv, const float* ssq, const uint16_t* q_gamma,
                                const uint16_t* k_gamma, const float* cos_tab,
                                const float* sin_tab, int64_t T, int32_t num_heads,
                                int32_t num_kv_heads, int32_t head_dim, float eps,
                                uint32_t flags, int32_t layout, hipStream_t stream) {
  if (!qkv) return fail(QKVMX_ERR_NULL, "qk_norm_rope_apply: null qkv");
  if (flags & ~(uint32_t)(QKVMX_NORM_Q | QKVMX_NORM_K | QKVMX_FUSED_ROPE))
    return fail(QKVMX_ERR_ARG, "qk_norm_rope_apply: unknown flag bits");
  if (T <= 0 || num_heads < 1 || num_kv_heads < 0 || head_dim <= 0 || head_dim % 16)
    return fail(QKVMX_ERR_SHAPE, "qk_norm_rope_apply: need T > 0, num_heads >= 1, num_kv_heads >= 0, head_dim %% 16 == 0");
  if (layout != QKVMX_LAYOUT_BSD && layout != QKVMX_LAYOUT_NBSD)
    return fail(QKVMX_ERR_ARG, "qk_norm_rope_apply: layout must be QKVMX_LAYOUT_BSD or QKVMX_LAYOUT_NBSD");
  if (head_dim > 1024) return fail(QKVMX_ERR_UNSUPPORTED, "qk_norm_rope_apply: head_dim > 1024");
  if ((flags & QKVMX_FUSED_ROPE) && (!cos_tab || !sin_tab))
    return fail(QKVMX_ERR_ARG, "qk_norm_rope_apply: QKVMX_FUSED_ROPE needs cos_tab and sin_tab");
  if (num_kv_heads == 0 && ((flags & QKVMX_NORM_K) || k_gamma))
    return fail(QKVMX_ERR_ARG, "qk_norm_rope_apply: no K segment when num_kv_heads == 0 (omit k_gamma and QKVMX_NORM_K)");
  if ((flags & QKVMX_NORM_Q) && !q_gamma) return fail(QKVMX_ERR_ARG, "qk_norm_rope_apply: QKVMX_NORM_Q needs q_gamma");
  if ((flags & QKVMX_NORM_K) && !k_gamma) return fail(QKVMX_ERR_ARG, "qk_norm_rope_apply: QKVMX_NORM_K needs k_gamma");
  if (!(flags & QKVMX_NORM_K) && k_gamma) return fail(QKVMX_ERR_ARG, "qk_norm_rope_apply: k_gamma given without QKVMX_NORM_K");
  if ((flags & (QKVMX_NORM_Q | QKVMX_NORM_K)) && !ssq) return fail(QKVMX_ERR_ARG, "qk_norm_rope_apply: the norm needs ssq");
  if (!(eps >= 0.0f)) return fail(QKVMX_ERR_ARG, "qk_norm_rope_apply: eps must be >= 0");
  if (!aligned(qkv, 16) || (ssq && !aligned(ssq, 8)) || (q_gamma && !aligned(q_gamma, 16)) ||
      (k_gamma && !aligned(k_gamma, 16)) || (cos_tab && !aligned(cos_tab, 16)) ||
      (sin_tab && !aligned(sin_tab, 16)))
    return fail(QKVMX_ERR_ALIGN, "qk_norm_rope_apply: qkv/gamma/tables 16-byte, ssq 8-byte aligned");
  return hip_status(launch_norm_rope(qkv, ssq, q_gamma, k_gamma, cos_tab, sin_tab, T, num_heads,
                                     num_kv_heads, head_dim, eps, flags,
                                     layout == QKVMX_LAYOUT_NBSD, stream), "qk_norm_rope_apply");
}

qkvmx_status qkvmx_e4m3_convert_check(unsigned long long* counts, uint32_t* first_bad,
                                      hipStream_t stream) {
  const char* fn = "qkvmx_e4m3_convert_check";
  if (!counts) return fail(QKVMX_ERR_NULL, "%s: counts is required", fn);
  if (!aligned(counts, 8) || (first_bad && !aligned(first_bad, 4)))
    return fail(QKVMX_ERR_ALIGN, "%s: counts 8-byte, first_bad 4-byte aligned", fn);
  return hip_status(launch_e4m3_check(counts, first_bad, stream), fn);
}

qkvmx_status qkvmx_mfma_rate_probe(int32_t blocks, int32_t iters, int32_t random_operands,
                                   float* sink, uint64_t* clocks, hipStream_t stream) {
  const char* fn = "qkvmx_mfma_rate_probe";
  if (!sink || !clocks) return fail(QKVMX_ERR_NULL, "%s: null pointer", fn);
  if (blocks < 1 || blocks > 65535 || iters < 1 || iters > (1 << 24))
    return fail(QKVMX_ERR_SHAPE, "%s: need 1 <= blocks <= 65535, 1 <= iters <= 2^24", fn);
  if (!aligned(sink, 4) || !aligned(clocks, 8)) return fail(QKVMX_ERR_ALIGN, "%s: sink 4-byte, clocks 8-byte aligned", fn);
  return hip_status(launch_mfma_rate(blocks, iters, random_operands != 0, sink, clocks, stream), fn);
}

}  // extern "C"
