// Weight preparation kernels (one-time, off the per-token path):
//  * mx_weight_quantize: fp32 W[H, I] -> MX block-32 E4M3 codes in the pages' [H/4, I, 4]
//    layout + one E8M0 exponent per 32 h of a column ([QKV-CTE] "Interface", weight).
//  * weight_prepack: pages' layout -> K-contiguous rows per output channel + exponent dwords
//    grouped so that each lane of the 32x32x64 scaled MFMA finds its block exponent for step
//    q (0..3) of a 256-K superstep in byte q of one dword.
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

// Codes: one thread per (channel i, 16-byte K chunk c): gathers 4 dwords (h/4 = 4c..4c+3) of
// column i and writes W^T[i][16c .. 16c+15].  Threads of a wave take consecutive i (coalesced
// dword reads).
__global__ void __launch_bounds__(256) prepack_codes_kernel(const uint8_t* __restrict__ codes,
                                                            int64_t H, int64_t I,
                                                            uint8_t* __restrict__ packed) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t c = blockIdx.y;              // H / 16 chunks (H % 32 == 0)
  if (i >= I) return;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(codes);
  uint4 o;
  o.x = src[(4 * c + 0) * I + i];
  o.y = src[(4 * c + 1) * I + i];
  o.z = src[(4 * c + 2) * I + i];
  o.w = src[(4 * c + 3) * I + i];
  *reinterpret_cast<uint4*>(packed + i * H + 16 * c) = o;
}

// Exponents: dword (i, s, g) holds, in byte q, the exponent of block 8s + 2q + g of column i
// (127, i.e. 2^0, past the end of H; those K positions carry zero codes).
__global__ void __launch_bounds__(256) prepack_scales_kernel(const uint8_t* __restrict__ e8m0,
                                                             int64_t H, int64_t I,
                                                             uint32_t* __restrict__ sc) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t s = blockIdx.y;
  if (i >= I) return;
  int64_t nblk = H / 32;
  int64_t S = ceil_div(H, kSuperK);
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    uint32_t word = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int64_t blk = 8 * s + 2 * q + g;
      uint32_t e = blk < nblk ? e8m0[blk * I + i] : 127u;
      word |= e << (8 * q);
    }
    sc[(i * S + s) * 2 + g] = word;
  }
}

hipError_t launch_mx_weight_quantize(const float* w, int64_t H, int64_t I, uint8_t* codes,
                                     uint8_t* e8m0, hipStream_t s) {
  dim3 grid((unsigned)ceil_div(I, 256), (unsigned)(H / 32));
  hipLaunchKernelGGL(mx_weight_quantize_kernel, grid, dim3(256), 0, s, w, H, I, codes, e8m0);
  return hipGetLastError();
}

hipError_t launch_weight_prepack(const uint8_t* codes, const uint8_t* e8m0, int64_t H, int64_t I,
                                 uint8_t* packed, hipStream_t s) {
  dim3 g1((unsigned)ceil_div(I, 256), (unsigned)(H / 16));
  hipLaunchKernelGGL(prepack_codes_kernel, g1, dim3(256), 0, s, codes, H, I, packed);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2((unsigned)ceil_div(I, 256), (unsigned)ceil_div(H, kSuperK));
  hipLaunchKernelGGL(prepack_scales_kernel, g2, dim3(256), 0, s, e8m0, H, I,
                     reinterpret_cast<uint32_t*>(packed + packed_scales_offset(H, I)));
  return hipGetLastError();
}

}  // namespace qkvmx
