// Roofline calibration (measurement only, not a step of the method): the rate at which this GPU
// issues the projection's instruction, V_MFMA_SCALE_F32_32X32X64_F8F6F4, when nothing but the
// matrix cores is busy.  Every wavefront keeps 16 independent 32x32 accumulators (the
// projection's 4 x 4 fragments per wave) and runs `iters` rounds of 16 MFMAs on operands held in
// registers: no memory traffic, no LDS, no epilogue.  The operands are random E4M3 codes (as
// quantised activations and weights are) or all zero; the two differ in how much the operand
// bits toggle, hence in power, hence in the clock the chip sustains.  Each block also reports
// its elapsed core-clock cycles and 100 MHz reference ticks, from which the clock follows.
#include "internal.h"

namespace qkvmx {

namespace {

typedef int v8i_c __attribute__((ext_vector_type(8)));
typedef float v16f_c __attribute__((ext_vector_type(16)));

template <bool kRandom>
__global__ void __launch_bounds__(256, 1) mfma_rate_kernel(int iters, unsigned seed,
                                                           float* __restrict__ sink,
                                                           uint64_t* __restrict__ clocks) {
  v8i_c a[4], b[4];
  unsigned x = seed ^ (threadIdx.x * 2654435761u) ^ (blockIdx.x * 40503u);
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // linear congruential draws; mask 0xB7 keeps each code's exponent field <= 7 (|v| < 2),
      // so the sums stay finite
      x = x * 1664525u + 1013904223u;
      a[f][j] = (int)(kRandom ? (x & 0xB7B7B7B7u) : 0u);
      x = x * 1664525u + 1013904223u;
      b[f][j] = (int)(kRandom ? (x & 0xB7B7B7B7u) : 0u);
    }
  v16f_c acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f_c{};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int cf = k >> 2, tf = k & 3;
      acc[cf][tf] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          a[cf], b[tf], acc[cf][tf], 0, 0, 0, 0x7F7F7F7F, 0, 0x7F7F7F7F);
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[i][j][e];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clocks[(int64_t)blockIdx.x * 2] = t1 - t0;
    clocks[(int64_t)blockIdx.x * 2 + 1] = r1 - r0;
  }
}

}  // namespace

hipError_t launch_mfma_rate(int blocks, int iters, bool random_operands, float* sink,
                            uint64_t* clocks, hipStream_t s) {
  if (random_operands)
    hipLaunchKernelGGL(mfma_rate_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, iters,
                       12345u, sink, clocks);
  else
    hipLaunchKernelGGL(mfma_rate_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, iters,
                       12345u, sink, clocks);
  return hipGetLastError();
}

}  // namespace qkvmx
