// Launchers of the projection with the per-head qk-norm (and rotate-half RoPE) fused into the
// epilogue: from the pages' packed rows (qkv_rowmx_project_headnorm, per-call activation
// repack) and from staged activations (qkv_rowmx_project_headnorm_staged, no repack).
#include "project_kernel.h"

namespace qkvmx {

namespace {

// The persistent project_kernel with the per-head epilogue, on prepared arguments.
hipError_t launch_headnorm_core(const ProjectArgs& a, int norm_kind, bool bias, bool nbsd,
                                hipStream_t s) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const unsigned nblocks = (unsigned)std::min<int64_t>((int64_t)a.tiles_m * a.tiles_n,
                                                       std::max(cus, 1));
  const dim3 grid(nblocks), block(kThreads);
  const int v = (norm_kind == 2 ? 8 : 0) | (a.cos_tab ? 4 : 0) | (bias ? 2 : 0) | (nbsd ? 1 : 0);
#define QKVMX_HN(K, R, B, N) hipLaunchKernelGGL((project_kernel<false, B, N, false, K, R>), grid, block, 0, s, a)
  switch (v) {
    case 0: QKVMX_HN(1, false, false, false); break;
    case 1: QKVMX_HN(1, false, false, true); break;
    case 2: QKVMX_HN(1, false, true, false); break;
    case 3: QKVMX_HN(1, false, true, true); break;
    case 4: QKVMX_HN(1, true, false, false); break;
    case 5: QKVMX_HN(1, true, false, true); break;
    case 6: QKVMX_HN(1, true, true, false); break;
    case 7: QKVMX_HN(1, true, true, true); break;
    case 8: QKVMX_HN(2, false, false, false); break;
    case 9: QKVMX_HN(2, false, false, true); break;
    case 10: QKVMX_HN(2, false, true, false); break;
    case 11: QKVMX_HN(2, false, true, true); break;
    case 12: QKVMX_HN(2, true, false, false); break;
    case 13: QKVMX_HN(2, true, false, true); break;
    case 14: QKVMX_HN(2, true, true, false); break;
    default: QKVMX_HN(2, true, true, true); break;
  }
#undef QKVMX_HN
  return hipGetLastError();
}

void set_head_args(ProjectArgs& a, const uint16_t* q_gamma, const uint16_t* k_gamma,
                   const uint16_t* q_beta, const uint16_t* k_beta, float eps,
                   const float* cos_tab, const float* sin_tab) {
  a.ws = nullptr;
  a.hq_gamma = q_gamma; a.hk_gamma = k_gamma; a.hq_beta = q_beta; a.hk_beta = k_beta;
  a.h_eps = eps; a.cos_tab = cos_tab; a.sin_tab = sin_tab;
}

}  // namespace

hipError_t launch_project_headnorm(const uint8_t* a_codes, int64_t a_stride,
                                   const uint8_t* a_scales, int64_t s_stride,
                                   const uint8_t* w_packed, const uint16_t* bias, int64_t T,
                                   int64_t H, int64_t I, int64_t Iq, int64_t Ik, int64_t d,
                                   bool nbsd, int norm_kind, const uint16_t* q_gamma,
                                   const uint16_t* k_gamma, const uint16_t* q_beta,
                                   const uint16_t* k_beta, float eps, const float* cos_tab,
                                   const float* sin_tab, uint16_t* out, uint8_t* ws,
                                   hipStream_t s) {
  ProjectArgs a = common_args(w_packed, nullptr, bias, T, H, I, Iq, Ik, d, out);
  a.a_codes = a_codes; a.a_stride = a_stride; a.a_scales = a_scales; a.s_stride = s_stride;
  a.x_img = ws;
  a.ctr = reinterpret_cast<unsigned*>(ws + counters_offset(T, H, I));
  set_head_args(a, q_gamma, k_gamma, q_beta, k_beta, eps, cos_tab, sin_tab);
  // the activation rows re-laid as stage images (this kernel also resets the tile counters)
  const dim3 rg(kStageImage / 16 / 256, (unsigned)a.KS, (unsigned)a.tiles_m);
  hipLaunchKernelGGL(act_repack_kernel, rg, dim3(256), 0, s, a_codes, a_stride, T, H, a.KS, ws,
                     a.ctr);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_headnorm_core(a, norm_kind, bias != nullptr, nbsd, s);
}

hipError_t launch_project_headnorm_staged(const uint8_t* img, const float* row_scale,
                                          const uint8_t* w_packed, const uint16_t* bias,
                                          int64_t T, int64_t H, int64_t I, int64_t Iq,
                                          int64_t Ik, int64_t d, bool nbsd, int norm_kind,
                                          const uint16_t* q_gamma, const uint16_t* k_gamma,
                                          const uint16_t* q_beta, const uint16_t* k_beta,
                                          float eps, const float* cos_tab, const float* sin_tab,
                                          uint16_t* out, uint8_t* ws, hipStream_t s) {
  ProjectArgs a = common_args(w_packed, nullptr, bias, T, H, I, Iq, Ik, d, out);
  a.a_scales = reinterpret_cast<const uint8_t*>(row_scale); a.s_stride = sizeof(float);
  a.x_img = img;
  a.ctr = reinterpret_cast<unsigned*>(ws + staged_counters_offset(T, I));
  set_head_args(a, q_gamma, k_gamma, q_beta, k_beta, eps, cos_tab, sin_tab);
  hipLaunchKernelGGL(reset_counters_kernel, dim3(1), dim3(64), 0, s, a.ctr);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_headnorm_core(a, norm_kind, bias != nullptr, nbsd, s);
}

}  // namespace qkvmx
