// Internal launch interface between the validated C ABI (qkvmx_api.hip) and the kernels.
// Every launcher assumes its arguments were validated by the caller and returns the
// hipGetLastError() status of its launch(es).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qkvmx {

// Projection tile geometry (tokens x channels x K bytes per LDS stage).
constexpr int kTileM = 256;      // tokens per block
constexpr int kTileN = 256;      // output channels per block
constexpr int kStageK = 128;     // K bytes per LDS stage
constexpr int kSuperK = 256;     // K bytes per scale dword (4 MFMA steps of 64)
constexpr int kPartialN = 128;   // channels covered by one sum-of-squares partial

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Packed weight: codes [I][H] then, at a 256-byte aligned offset, the exponent dwords
// [I][ceil(H / 256)][2].
inline size_t packed_codes_bytes(int64_t H, int64_t I) { return (size_t)(H * I); }
inline size_t packed_scales_offset(int64_t H, int64_t I) {
  return (packed_codes_bytes(H, I) + 255) & ~(size_t)255;
}
inline size_t packed_total_bytes(int64_t H, int64_t I) {
  return packed_scales_offset(H, I) + (size_t)I * (size_t)ceil_div(H, kSuperK) * 2 * 4;
}
inline int64_t ssq_partials(int64_t I) { return ceil_div(I, kTileN) * (kTileN / kPartialN); }
inline size_t workspace_total_bytes(int64_t T, int64_t I) {
  return (size_t)ssq_partials(I) * (size_t)T * 2 * sizeof(float);
}

hipError_t launch_mx_weight_quantize(const float* w, int64_t H, int64_t I, uint8_t* codes,
                                     uint8_t* e8m0, hipStream_t s);
hipError_t launch_weight_prepack(const uint8_t* codes, const uint8_t* e8m0, int64_t H, int64_t I,
                                 uint8_t* packed, hipStream_t s);
hipError_t launch_row_quantize(const void* x, int dtype, int64_t T, int64_t H, uint8_t* packed,
                               hipStream_t s);
hipError_t launch_rmsnorm_quantize(const uint16_t* hid, const uint16_t* res, const uint16_t* gamma,
                                   float eps, int64_t T, int64_t H, int64_t Hu, uint16_t* res_out,
                                   uint8_t* packed, hipStream_t s);
hipError_t launch_project(const uint8_t* a_codes, int64_t a_stride, const uint8_t* a_scales,
                          int64_t s_stride, const uint8_t* w_packed, const float* chan_scale,
                          const uint16_t* bias, int64_t T, int64_t H, int64_t I, int64_t Iq,
                          int64_t Ik, uint16_t* out, float* ssq, float* ws, hipStream_t s);
hipError_t launch_norm_rope(uint16_t* qkv, const float* ssq, const uint16_t* q_gamma,
                            const uint16_t* k_gamma, const float* cos_tab, const float* sin_tab,
                            int64_t T, int nq, int nkv, int d, float eps, uint32_t flags,
                            hipStream_t s);

}  // namespace qkvmx
