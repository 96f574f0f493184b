// Launchers of the projection on MX block-32 activations: from natural-order codes and
// exponents (qkv_mx_project: both re-laid per call, then the persistent projection kernel with
// per-block activation exponents) and from staged ones (qkv_mx_project_staged: written by a
// staged producer in the kernel's layouts, so no re-layout).
#include "project_kernel.h"

namespace qkvmx {

hipError_t launch_project_mx(const uint8_t* a_codes, int64_t a_stride, const uint8_t* a_e8,
                             int64_t e_stride, const uint8_t* w_packed, const float* chan_scale,
                             const uint16_t* bias, int64_t T, int64_t H, int64_t I, int64_t Iq,
                             int64_t Ik, int64_t d, bool nbsd, uint16_t* out, float* ssq,
                             uint8_t* ws, hipStream_t s) {
  ProjectArgs a = common_args(w_packed, chan_scale, bias, T, H, I, Iq, Ik, d, out);
  a.a_codes = a_codes; a.a_stride = a_stride;
  a.x_img = ws;
  a.x_scales = ws + mx_scale_image_offset(T, H);
  float* partials = reinterpret_cast<float*>(ws + mx_partials_offset(T, H));
  a.ws = ssq ? partials : nullptr;
  a.ctr = reinterpret_cast<unsigned*>(ws + mx_counters_offset(T, H, I));
  // the activation codes re-laid as stage images (this kernel also resets the tile counters),
  // their exponents in the weight exponents' format
  dim3 rg(kStageImage / 16 / 256, (unsigned)a.KS, (unsigned)a.tiles_m);
  hipLaunchKernelGGL(act_repack_kernel, rg, dim3(256), 0, s, a_codes, a_stride, T, H, a.KS, ws,
                     a.ctr);
  dim3 sg(2, (unsigned)(a.KS / 4), (unsigned)a.tiles_m);
  hipLaunchKernelGGL(act_scale_repack_kernel, sg, dim3(256), 0, s, a_e8, e_stride, T, H,
                     reinterpret_cast<uint32_t*>(ws + mx_scale_image_offset(T, H)));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_core<true>(a, chan_scale, bias, nbsd, ssq, s,
                           ws + mx_counters_offset(T, H, I) + kCounterBytes);
}

hipError_t launch_project_mx_staged(const uint8_t* img, const uint32_t* eimg,
                                    const uint8_t* w_packed, const float* chan_scale,
                                    const uint16_t* bias, int64_t T, int64_t H, int64_t I,
                                    int64_t Iq, int64_t Ik, int64_t d, bool nbsd, uint16_t* out,
                                    float* ssq, uint8_t* ws, hipStream_t s) {
  ProjectArgs a = common_args(w_packed, chan_scale, bias, T, H, I, Iq, Ik, d, out);
  a.x_img = img;
  a.x_scales = reinterpret_cast<const uint8_t*>(eimg);
  a.ws = ssq ? reinterpret_cast<float*>(ws) : nullptr;
  a.ctr = reinterpret_cast<unsigned*>(ws + staged_counters_offset(T, I));
  hipLaunchKernelGGL(reset_counters_kernel, dim3(1), dim3(64), 0, s, a.ctr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_core<true>(a, chan_scale, bias, nbsd, ssq, s,
                           ws + staged_counters_offset(T, I) + kCounterBytes);
}

}  // namespace qkvmx
