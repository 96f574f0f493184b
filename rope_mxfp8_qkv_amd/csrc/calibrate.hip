// Roofline calibration (measurement only, not a step of the method): the rate at which this GPU
// issues the projection's instruction, V_MFMA_SCALE_F32_32X32X64_F8F6F4, when nothing but the
// matrix cores is busy.  Every wavefront keeps 16 independent 32x32 accumulators (the
// projection's 4 x 4 fragments per wave) and runs `iters` rounds of 16 MFMAs on operands held in
// registers: no memory traffic, no LDS, no epilogue.  The operands are random E4M3 codes (as
// quantised activations and weights are) or all zero; the two differ in how much the operand
// bits toggle, hence in power, hence in the clock the chip sustains.  Each block also reports
// its elapsed core-clock cycles and 100 MHz reference ticks, from which the clock follows.
//
// Also the exhaustive check of the producers' E4M3 encoding: the hardware packing conversion
// after a clamp to +-448 against the software round-to-nearest-even encoder, on every finite
// fp32 value.
#include "device_common.h"
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

// Every 32-bit pattern p (4 consecutive patterns per thread and step): for each finite fp32
// value of the four, the hardware path (e4m3x4) and the software encoder (f32_to_e4m3) must give
// the same code byte.  counts[0] += mismatching values, counts[1] += finite values compared;
// the first 8 mismatching patterns go to first_bad (if given).
__global__ void __launch_bounds__(256) e4m3_check_kernel(unsigned long long* __restrict__ counts,
                                                         uint32_t* __restrict__ first_bad) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x * 4;
  unsigned long long bad = 0, seen = 0;
  for (uint64_t base = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; base < (1ull << 32);
       base += stride) {
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float((uint32_t)(base + i));
    const uint32_t hw = e4m3x4(v[0], v[1], v[2], v[3]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!__builtin_isfinite(v[i])) continue;
      ++seen;
      if (((hw >> (8 * i)) & 0xFFu) != f32_to_e4m3(v[i])) {
        ++bad;
        if (first_bad) {
          const unsigned long long slot = atomicAdd(&counts[2], 1ull);
          if (slot < 8) first_bad[slot] = (uint32_t)(base + i);
        }
      }
    }
  }
  if (bad) atomicAdd(&counts[0], bad);
  atomicAdd(&counts[1], seen);
}

}  // namespace

hipError_t launch_e4m3_check(unsigned long long* counts, uint32_t* first_bad, hipStream_t s) {
  hipLaunchKernelGGL(e4m3_check_kernel, dim3(1024), dim3(256), 0, s, counts, first_bad);
  return hipGetLastError();
}

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
