// Weight preparation kernels (one-time, off the per-token path):
//  * mx_weight_quantize: fp32 W[H, I] -> MX block-32 E4M3 codes in the pages' [H/4, I, 4]
//    layout + one E8M0 exponent per 32 h of a column ([QKV-CTE] "Interface", weight).
//  * weight_prepack: pages' layout -> the projection kernel's layout: per (256-channel tile,
//    64-byte K-stage) the exact 16 KiB LDS image the kernel consumes (so one DMA instruction
//    copies 1 KiB contiguous), plus exponent dwords grouped so that each lane of the 32x32x64
//    scaled MFMA finds its block exponent for step q (0..3) of a 256-K superstep in byte q.
#include "device_common.h"
#include "internal.h"

namespace qkvmx {

// One thread per (32-row block b, column i): threads of a wavefront take consecutive columns,
// so every strided row read and every [H/4, I, 4] dword write is coalesced across the wave.
__global__ void __launch_bounds__(256) mx_weight_quantize_kernel(const float* __restrict__ w,
                                                                 int64_t H, int64_t I,
                                                                 uint8_t* __restrict__ codes,
                                                                 uint8_t* __restrict__ e8m0) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t b = blockIdx.y;
  if (i >= I) return;
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    v[r] = w[(b * 32 + r) * I + i];
    amax = fmaxf(amax, fabsf(v[r]));
  }
  int E = 0;
  if (amax > 0.0f) {
    int e2;
    frexpf(amax, &e2);                 // amax = f * 2^e2, 0.5 <= f < 1  => floor(log2) = e2 - 1
    E = (e2 - 1) - 8 + 127;
    E = E < 0 ? 0 : (E > 254 ? 254 : E);
  }
  e8m0[b * I + i] = (uint8_t)E;
  float inv = ldexpf(1.0f, 127 - E);   // exact power of two
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    uint32_t word = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t c = (amax > 0.0f) ? f32_to_e4m3(v[4 * g + q] * inv) : 0u;
      word |= c << (8 * q);
    }
    // element (h, i) lives at byte ((h / 4) * I + i) * 4 + h % 4
    reinterpret_cast<uint32_t*>(codes)[(b * 8 + g) * I + i] = word;
  }
}

// Codes: one thread per 16-byte chunk position p (0..1023) of the stage image (tile tn, stage
// t): position p holds logical chunk c = (p % 4) ^ stage_swizzle(r) of row r = p / 4, i.e. bytes
// [64 t + 16 c, +16) of channel 256 tn + r, gathered from four dwords of the [H/4, I, 4] codes
// (h/4 rows 16 t + 4 c .. +3).  Zero past I or H.
__global__ void __launch_bounds__(256) prepack_codes_kernel(const uint8_t* __restrict__ codes,
                                                            int64_t H, int64_t I, int64_t KS,
                                                            uint8_t* __restrict__ packed) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;   // 0..1023
  const int64_t t = blockIdx.y;
  const int64_t tn = blockIdx.z;
  const int r = p >> 2;
  const int c = (p & 3) ^ stage_swizzle(r);
  const int64_t n = tn * kTileN + r;
  const int64_t k = t * kStage + 16 * c;
  uint4 o = make_uint4(0, 0, 0, 0);
  if (n < I && k < H) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(codes);
    const int64_t h4 = k / 4;
    o.x = src[(h4 + 0) * I + n];
    o.y = src[(h4 + 1) * I + n];
    o.z = src[(h4 + 2) * I + n];
    o.w = src[(h4 + 3) * I + n];
  }
  reinterpret_cast<uint4*>(packed)[(tn * KS + t) * (kStageImage / 16) + p] = o;
}

// Exponents: one thread per (superstep s, channel slot n of the padded NT * 256 channels).
__global__ void __launch_bounds__(256) prepack_scales_kernel(const uint8_t* __restrict__ e8m0,
                                                             int64_t H, int64_t I, int64_t NI,
                                                             uint32_t* __restrict__ sc) {
  const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t s = blockIdx.y;
  if (n >= NI) return;
  const int64_t nblk = H / 32;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    uint32_t word = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t blk = 8 * s + 2 * q + g;
      const uint32_t e = (n < I && blk < nblk) ? e8m0[blk * I + n] : 127u;
      word |= e << (8 * q);
    }
    sc[(s * NI + n) * 2 + g] = word;
  }
}

__global__ void __launch_bounds__(256) zero_fill_kernel(uint4* __restrict__ p, int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n16) p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_mx_weight_quantize(const float* w, int64_t H, int64_t I, uint8_t* codes,
                                     uint8_t* e8m0, hipStream_t s) {
  dim3 grid((unsigned)ceil_div(I, 256), (unsigned)(H / 32));
  hipLaunchKernelGGL(mx_weight_quantize_kernel, grid, dim3(256), 0, s, w, H, I, codes, e8m0);
  return hipGetLastError();
}

hipError_t launch_weight_prepack(const uint8_t* codes, const uint8_t* e8m0, int64_t H, int64_t I,
                                 uint8_t* packed, hipStream_t s) {
  const int64_t NT = packed_tiles_n(I), KS = packed_stages(H);
  dim3 g1(kStageImage / 16 / 256, (unsigned)KS, (unsigned)NT);
  hipLaunchKernelGGL(prepack_codes_kernel, g1, dim3(256), 0, s, codes, H, I, KS, packed);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t NI = NT * kTileN;
  dim3 g2((unsigned)ceil_div(NI, 256), (unsigned)(KS / 4));
  hipLaunchKernelGGL(prepack_scales_kernel, g2, dim3(256), 0, s, e8m0, H, I, NI,
                     reinterpret_cast<uint32_t*>(packed + packed_scales_offset(H, I)));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(zero_fill_kernel, dim3(kZeroPage / 16 / 256), dim3(256), 0, s,
                     reinterpret_cast<uint4*>(packed + packed_zero_offset(H, I)),
                     (int64_t)(kZeroPage / 16));
  return hipGetLastError();
}

}  // namespace qkvmx
