// Launchers of the projection on ROW_MX activations: from the pages' packed rows
// (qkv_rowmx_project: per-call activation repack, the persistent projection kernel, the
// fixed-order sum of the sum-of-squares partials) and from staged activations
// (qkv_rowmx_project_staged: the codes already in the stage-image layout, so no repack).
#include "project_kernel.h"

namespace qkvmx {

hipError_t launch_project(const uint8_t* a_codes, int64_t a_stride, const uint8_t* a_scales,
                          int64_t s_stride, const uint8_t* w_packed, const float* chan_scale,
                          const uint16_t* bias, int64_t T, int64_t H, int64_t I, int64_t Iq,
                          int64_t Ik, int64_t d, bool nbsd, uint16_t* out, float* ssq,
                          uint8_t* ws, hipStream_t s) {
  ProjectArgs a = common_args(w_packed, chan_scale, bias, T, H, I, Iq, Ik, d, out);
  a.a_codes = a_codes; a.a_stride = a_stride; a.a_scales = a_scales; a.s_stride = s_stride;
  a.x_img = ws;
  float* partials = reinterpret_cast<float*>(ws + act_image_bytes(T, H));
  a.ws = ssq ? partials : nullptr;
  a.ctr = reinterpret_cast<unsigned*>(ws + counters_offset(T, H, I));
  // the activation rows re-laid as stage images (this kernel also resets the tile counters)
  dim3 rg(kStageImage / 16 / 256, (unsigned)a.KS, (unsigned)a.tiles_m);
  hipLaunchKernelGGL(act_repack_kernel, rg, dim3(256), 0, s, a_codes, a_stride, T, H, a.KS, ws,
                     a.ctr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_core<false>(a, chan_scale, bias, nbsd, ssq, s,
                            ws + counters_offset(T, H, I) + kCounterBytes);
}

hipError_t launch_project_staged(const uint8_t* img, const float* row_scale,
                                 const uint8_t* w_packed, const float* chan_scale,
                                 const uint16_t* bias, int64_t T, int64_t H, int64_t I, int64_t Iq,
                                 int64_t Ik, int64_t d, bool nbsd, uint16_t* out, float* ssq,
                                 uint8_t* ws, hipStream_t s) {
  ProjectArgs a = common_args(w_packed, chan_scale, bias, T, H, I, Iq, Ik, d, out);
  a.a_scales = reinterpret_cast<const uint8_t*>(row_scale); a.s_stride = sizeof(float);
  a.x_img = img;
  a.ws = ssq ? reinterpret_cast<float*>(ws) : nullptr;
  a.ctr = reinterpret_cast<unsigned*>(ws + staged_counters_offset(T, I));
  hipLaunchKernelGGL(reset_counters_kernel, dim3(1), dim3(64), 0, s, a.ctr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_core<false>(a, chan_scale, bias, nbsd, ssq, s,
                            ws + staged_counters_offset(T, I) + kCounterBytes);
}

}  // namespace qkvmx
