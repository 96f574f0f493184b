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
constexpr int kStage = 64;       // K bytes per LDS stage (one MFMA K-step)
constexpr int kSuperK = 256;     // K bytes per exponent dword (4 MFMA K-steps)
constexpr int kPartialN = 128;   // channels covered by one sum-of-squares partial
constexpr int kStageImage = kTileN * kStage;   // 16 KiB: one operand stage as stored in LDS
constexpr int kZeroPage = 16384;               // zero bytes read in place of K past H

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Chunk swizzle of a stage image row (four 16-byte chunks of K per 64-byte row).  Rows r and
// r + 4 k (k = 1, 2, 3) get distinct values, and so do rows r and r + 2 k: the 16 rows one
// ds_read_b128 serves fall into 16 distinct 16-byte bank groups of a 256-byte LDS window.
__host__ __device__ inline int stage_swizzle(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }

// Packed weight, for an [H, I] projection with NT = ceil(I / 256) channel tiles and
// KS = 4 * ceil(H / 256) K-stages:
//   codes   [NT][KS][16 KiB]  each block the LDS image of one stage of one channel tile
//                             (256 rows x 64 K-bytes, 16-byte chunk c of row r stored at
//                             chunk position c ^ stage_swizzle(r)); zero past I and H
//   scales  [KS / 4][NT * 256][2] dwords: byte q of dword g of channel n in superstep s is the
//                             E8M0 exponent of K-block 8 s + 2 q + g (127 past I / H)
//   zero    16 KiB of zeros (read in place of activation bytes past H)
inline int64_t packed_tiles_n(int64_t I) { return ceil_div(I, kTileN); }
inline int64_t packed_stages(int64_t H) { return 4 * ceil_div(H, kSuperK); }
inline size_t packed_codes_bytes(int64_t H, int64_t I) {
  return (size_t)packed_tiles_n(I) * packed_stages(H) * kStageImage;
}
inline size_t packed_scales_offset(int64_t H, int64_t I) { return packed_codes_bytes(H, I); }
inline size_t packed_scales_bytes(int64_t H, int64_t I) {
  return (size_t)(packed_stages(H) / 4) * packed_tiles_n(I) * kTileN * 2 * 4;
}
inline size_t packed_zero_offset(int64_t H, int64_t I) {
  return packed_scales_offset(H, I) + packed_scales_bytes(H, I);
}
inline size_t packed_total_bytes(int64_t H, int64_t I) {
  return packed_zero_offset(H, I) + kZeroPage;
}
inline int64_t ssq_partials(int64_t I) { return ceil_div(I, kTileN) * (kTileN / kPartialN); }
// Split contraction for calls with few output tiles (at most kSplitMaxTiles 256 x 256 tiles,
// e.g. a 512-token context projection): the K range is cut into up to kMaxSplit chunks (and
// at most kSplitUnits units in all), each (tile, chunk) unit stores its fp32 partial tile into
// its own [T, I] plane, and a per-token pass sums the planes and applies the epilogue.  Each
// unit streams 512 bytes of operands per K-byte but writes a 256 KiB plane tile whatever its
// K range, so deeper splits trade idle compute units for plane traffic: on the 512 x 5120 ->
// 5120 context calls 2, 3, 4 and 5 chunks measured 58.9, 56.0, 59.1 and 63.0 us against
// 66.1 us unsplit.  The factor depends on T and I only, so the workspace queries can size the
// planes.
constexpr int64_t kSplitMaxTiles = 128;
constexpr int64_t kSplitUnits = 256;
constexpr int64_t kMaxSplit = 3;
inline int split_factor(int64_t T, int64_t I) {
  const int64_t tiles = ceil_div(T, kTileM) * ceil_div(I, kTileN);
  if (tiles > kSplitMaxTiles) return 1;
  const int64_t s = kSplitUnits / tiles;
  return (int)(s < kMaxSplit ? s : kMaxSplit);
}
inline size_t split_planes_bytes(int64_t T, int64_t I) {
  const int s = split_factor(T, I);
  return s > 1 ? (size_t)s * (size_t)T * (size_t)I * sizeof(float) : 0;
}
// The K chunks a BSD call actually uses: ceil(supersteps / factor) supersteps each, so the
// last chunk may be shorter; {1, all stages} when the call does not split.
struct SplitPlan {
  int chunks;
  int stages_per_chunk;
};
inline SplitPlan split_plan(int64_t T, int64_t H, int64_t I) {
  const int64_t nsup = ceil_div(H, kSuperK);
  const int sf = split_factor(T, I);
  const SplitPlan whole{1, (int)(4 * nsup)};
  if (sf < 2) return whole;
  const int64_t chunk = ceil_div(nsup, sf);
  const int used = (int)ceil_div(nsup, chunk);
  return used < 2 ? whole : SplitPlan{used, (int)(4 * chunk)};
}
// Projection workspace: the activation codes re-laid as stage images [MT][KS][16 KiB]
// (MT = ceil(T / 256) token tiles), then the sum-of-squares partials [P][T][2] fp32, then a
// 256-byte block holding the per-XCD tile counters of the projection's tile scheduler.
inline size_t act_image_bytes(int64_t T, int64_t H) {
  return (size_t)ceil_div(T, kTileM) * packed_stages(H) * kStageImage;
}
inline size_t partials_bytes(int64_t T, int64_t I) {
  return (size_t)ssq_partials(I) * (size_t)T * 2 * sizeof(float);
}
constexpr size_t kCounterBytes = 256;
inline size_t counters_offset(int64_t T, int64_t H, int64_t I) {
  return (act_image_bytes(T, H) + partials_bytes(T, I) + 255) / 256 * 256;
}
// the split-contraction planes (when the call has few tiles) follow the counter block
inline size_t workspace_total_bytes(int64_t T, int64_t H, int64_t I) {
  return counters_offset(T, H, I) + kCounterBytes + split_planes_bytes(T, I);
}
// MX-activation projection workspace: the activation code stage images (as above), their
// exponents re-laid per (token tile, superstep) as [256][2] dwords, the sum-of-squares
// partials, then the 256-byte counter block.
inline size_t mx_scale_image_offset(int64_t T, int64_t H) { return act_image_bytes(T, H); }
inline size_t mx_scale_image_bytes(int64_t T, int64_t H) {
  return (size_t)ceil_div(T, kTileM) * (packed_stages(H) / 4) * kTileM * 2 * 4;
}
inline size_t mx_partials_offset(int64_t T, int64_t H) {
  return mx_scale_image_offset(T, H) + mx_scale_image_bytes(T, H);
}
inline size_t mx_counters_offset(int64_t T, int64_t H, int64_t I) {
  return (mx_partials_offset(T, H) + partials_bytes(T, I) + 255) / 256 * 256;
}
inline size_t mx_workspace_total_bytes(int64_t T, int64_t H, int64_t I) {
  return mx_counters_offset(T, H, I) + kCounterBytes + split_planes_bytes(T, I);
}

// Projection on staged activations (codes already in the stage-image layout, written by a
// staged producer): the workspace holds only the sum-of-squares partials [P][T][2] fp32,
// after them the 256-byte counter block, then the split-contraction planes (few tiles only).
inline size_t staged_counters_offset(int64_t T, int64_t I) {
  return (partials_bytes(T, I) + 255) / 256 * 256;
}
inline size_t staged_workspace_total_bytes(int64_t T, int64_t I) {
  return staged_counters_offset(T, I) + kCounterBytes + split_planes_bytes(T, I);
}

// The entry point that allocates nothing (qkv_rowmx_project_staged_noalloc) keeps the staged
// projection's workspace in a static device array of this size (one per GPU, held until the
// process ends): 80 MiB holds the full-video call's 69.2 MB (120 partials x 75600 tokens) and
// a split 512-token context call's planes (30.2 MB).
constexpr size_t kNoAllocScratchBytes = (size_t)80 << 20;
// Device address of the current device's static scratch array (project_noalloc.hip).
hipError_t noalloc_scratch(void** out);

hipError_t launch_e4m3_check(unsigned long long* counts, uint32_t* first_bad, hipStream_t s);
hipError_t launch_mx_weight_quantize(const float* w, int64_t H, int64_t I, uint8_t* codes,
                                     uint8_t* e8m0, hipStream_t s);
hipError_t launch_weight_prepack(const uint8_t* codes, const uint8_t* e8m0, int64_t H, int64_t I,
                                 uint8_t* packed, hipStream_t s);
hipError_t launch_row_quantize(const void* x, int dtype, int64_t T, int64_t H, uint8_t* packed,
                               hipStream_t s);
hipError_t launch_rmsnorm_quantize(const uint16_t* hid, const uint16_t* res, const uint16_t* gamma,
                                   float eps, int64_t T, int64_t H, int64_t Hu, uint16_t* res_out,
                                   uint8_t* packed, hipStream_t s);
hipError_t launch_row_quantize_staged(const void* x, int dtype, int64_t T, int64_t H,
                                      uint8_t* img, float* row_scale, hipStream_t s);
hipError_t launch_rmsnorm_quantize_staged(const uint16_t* hid, const uint16_t* res,
                                          const uint16_t* gamma, float eps, int64_t T, int64_t H,
                                          int64_t Hu, uint16_t* res_out, uint8_t* img,
                                          float* row_scale, hipStream_t s);
hipError_t launch_mx_quantize_staged(const void* x, int dtype, int64_t T, int64_t H,
                                     uint8_t* img, uint32_t* eimg, hipStream_t s);
hipError_t launch_rmsnorm_mx_staged(const uint16_t* hid, const uint16_t* res,
                                    const uint16_t* gamma, float eps, int64_t T, int64_t H,
                                    int64_t Hu, uint16_t* res_out, uint8_t* img, uint32_t* eimg,
                                    uint16_t* norm_out, hipStream_t s);
hipError_t launch_project_mx_staged(const uint8_t* img, const uint32_t* eimg,
                                    const uint8_t* w_packed, const float* chan_scale,
                                    const uint16_t* bias, int64_t T, int64_t H, int64_t I,
                                    int64_t Iq, int64_t Ik, int64_t d, bool nbsd, uint16_t* out,
                                    float* ssq, uint8_t* ws, hipStream_t s);
hipError_t launch_project_staged(const uint8_t* img, const float* row_scale,
                                 const uint8_t* w_packed, const float* chan_scale,
                                 const uint16_t* bias, int64_t T, int64_t H, int64_t I, int64_t Iq,
                                 int64_t Ik, int64_t d, bool nbsd, uint16_t* out, float* ssq,
                                 uint8_t* ws, hipStream_t s);
hipError_t launch_project(const uint8_t* a_codes, int64_t a_stride, const uint8_t* a_scales,
                          int64_t s_stride, const uint8_t* w_packed, const float* chan_scale,
                          const uint16_t* bias, int64_t T, int64_t H, int64_t I, int64_t Iq,
                          int64_t Ik, int64_t d, bool nbsd, uint16_t* out, float* ssq,
                          uint8_t* ws, hipStream_t s);
hipError_t launch_project_mx(const uint8_t* a_codes, int64_t a_stride, const uint8_t* a_e8,
                             int64_t e_stride, const uint8_t* w_packed, const float* chan_scale,
                             const uint16_t* bias, int64_t T, int64_t H, int64_t I, int64_t Iq,
                             int64_t Ik, int64_t d, bool nbsd, uint16_t* out, float* ssq,
                             uint8_t* ws, hipStream_t s);
hipError_t launch_project_headnorm(const uint8_t* a_codes, int64_t a_stride,
                                   const uint8_t* a_scales, int64_t s_stride,
                                   const uint8_t* w_packed, const uint16_t* bias, int64_t T,
                                   int64_t H, int64_t I, int64_t Iq, int64_t Ik, int64_t d,
                                   bool nbsd, int norm_kind, const uint16_t* q_gamma,
                                   const uint16_t* k_gamma, const uint16_t* q_beta,
                                   const uint16_t* k_beta, float eps, const float* cos_tab,
                                   const float* sin_tab, uint16_t* out, uint8_t* ws,
                                   hipStream_t s);
hipError_t launch_project_headnorm_staged(const uint8_t* img, const float* row_scale,
                                          const uint8_t* w_packed, const uint16_t* bias,
                                          int64_t T, int64_t H, int64_t I, int64_t Iq,
                                          int64_t Ik, int64_t d, bool nbsd, int norm_kind,
                                          const uint16_t* q_gamma, const uint16_t* k_gamma,
                                          const uint16_t* q_beta, const uint16_t* k_beta,
                                          float eps, const float* cos_tab, const float* sin_tab,
                                          uint16_t* out, uint8_t* ws, hipStream_t s);
hipError_t launch_mx_quantize(const void* x, int dtype, int64_t T, int64_t H, uint8_t* codes,
                              uint8_t* e8, hipStream_t s);
hipError_t launch_rmsnorm_mx(const uint16_t* hid, const uint16_t* res, const uint16_t* gamma,
                             float eps, int64_t T, int64_t H, int64_t Hu, uint16_t* res_out,
                             uint8_t* codes, uint8_t* e8, uint16_t* norm_out, hipStream_t s);
hipError_t launch_mfma_rate(int blocks, int iters, bool random_operands, float* sink,
                            uint64_t* clocks, hipStream_t s);
hipError_t launch_norm_rope(uint16_t* qkv, const float* ssq, const uint16_t* q_gamma,
                            const uint16_t* k_gamma, const float* cos_tab, const float* sin_tab,
                            int64_t T, int nq, int nkv, int d, float eps, uint32_t flags,
                            bool nbsd, hipStream_t s);

}  // namespace qkvmx
