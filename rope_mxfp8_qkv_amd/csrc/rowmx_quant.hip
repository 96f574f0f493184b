// ROW_MX activation producers ([QKV-CTE] "Interface", packed_hidden: H FP8 codes + 4-byte fp32
// scale tail per row; [RMSNORM-MX] residual / eps / unpadded_hidden_size).
//
// One 256-thread block per row; the row stays in registers between the reduction passes, so
// every input byte is read from HBM once and every output byte written once (HBM-bound: per
// row the producer moves 4H read + 2H + (H + 4) written bytes).
#include "device_common.h"
#include "internal.h"

namespace qkvmx {

namespace {

constexpr int kThreads = 256;
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));

__device__ __forceinline__ float block_max(float v, float* sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  v = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
  return v;
}

__device__ __forceinline__ double block_sum(double v, double* sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  v = (sh[0] + sh[1]) + (sh[2] + sh[3]);
  return v;
}

// Encode the row held as CPT chunks of 8 fp32 per thread and store codes + scale tail.
template <int CPT>
__device__ __forceinline__ void encode_store(float (&y)[CPT][8], float amax, int64_t H,
                                             uint8_t* __restrict__ row_out) {
  const int64_t nchunks = H / 8;
  // s = fl32(amax / 448); a zero row stores s = 0 and zero codes.
  const float s = amax / 448.0f;
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int64_t c = threadIdx.x + (int64_t)k * kThreads;
    if (c < nchunks) {
      uint32_t lo = 0, hi = 0;
      if (s > 0.0f) {
#pragma unroll
        for (int e = 0; e < 4; ++e) lo |= f32_to_e4m3(y[k][e] / s) << (8 * e);
#pragma unroll
        for (int e = 0; e < 4; ++e) hi |= f32_to_e4m3(y[k][4 + e] / s) << (8 * e);
      }
      u32x2_a4 v = {lo, hi};
      *reinterpret_cast<u32x2_a4*>(row_out + c * 8) = v;
    }
  }
  if (threadIdx.x == 0) *reinterpret_cast<float*>(row_out + H) = s;
}

template <int CPT, bool BF16>
__global__ void __launch_bounds__(kThreads) row_quantize_kernel(const void* __restrict__ x,
                                                                int64_t H,
                                                                uint8_t* __restrict__ packed) {
  __shared__ float sh[4];
  const int64_t row = blockIdx.x;
  const int64_t nchunks = H / 8;
  float y[CPT][8];
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int64_t c = threadIdx.x + (int64_t)k * kThreads;
    if (c < nchunks) {
      if (BF16) {
        const uint4 v = reinterpret_cast<const uint4*>(
            reinterpret_cast<const uint16_t*>(x) + row * H)[c];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y[k][2 * e] = bf16_to_f32(w[e] & 0xFFFFu);
          y[k][2 * e + 1] = bf16_to_f32(w[e] >> 16);
        }
      } else {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) +
                                                          row * H) + 2 * c;
        const float4 a = p[0], b = p[1];
        y[k][0] = a.x; y[k][1] = a.y; y[k][2] = a.z; y[k][3] = a.w;
        y[k][4] = b.x; y[k][5] = b.y; y[k][6] = b.z; y[k][7] = b.w;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(y[k][e]));
    }
  }
  amax = block_max(amax, sh);
  encode_store<CPT>(y, amax, H, packed + row * (H + 4));
}

template <int CPT, bool RES>
__global__ void __launch_bounds__(kThreads) rmsnorm_quantize_kernel(
    const uint16_t* __restrict__ hid, const uint16_t* __restrict__ res,
    const uint16_t* __restrict__ gamma, float eps, int64_t H, int64_t Hu,
    uint16_t* __restrict__ res_out, uint8_t* __restrict__ packed) {
  __shared__ double shd[4];
  __shared__ float shf[4];
  const int64_t row = blockIdx.x;
  const int64_t nchunks = H / 8;
  float y[CPT][8];
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int64_t c = threadIdx.x + (int64_t)k * kThreads;
    if (c < nchunks) {
      const uint4 hv = reinterpret_cast<const uint4*>(hid + row * H)[c];
      const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w};
      if (RES) {
        const uint4 rv = reinterpret_cast<const uint4*>(res + row * H)[c];
        const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
        uint32_t ow[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // r = bf16_RNE(fp32 + fp32): one fp32 rounding, then one bf16 rounding
          const uint32_t lo = f32_to_bf16(bf16_to_f32(hw[e] & 0xFFFFu) + bf16_to_f32(rw[e] & 0xFFFFu));
          const uint32_t hi = f32_to_bf16(bf16_to_f32(hw[e] >> 16) + bf16_to_f32(rw[e] >> 16));
          ow[e] = lo | (hi << 16);
          y[k][2 * e] = bf16_to_f32(lo);
          y[k][2 * e + 1] = bf16_to_f32(hi);
        }
        reinterpret_cast<uint4*>(res_out + row * H)[c] = make_uint4(ow[0], ow[1], ow[2], ow[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y[k][2 * e] = bf16_to_f32(hw[e] & 0xFFFFu);
          y[k][2 * e + 1] = bf16_to_f32(hw[e] >> 16);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += (double)y[k][e] * (double)y[k][e];
    }
  }
  ss = block_sum(ss, shd);
  // inv = fp32(1 / sqrt(ss / Hu + eps)), sqrt and divide correctly rounded in fp64
  const float inv = (float)(1.0 / sqrt(ss / (double)Hu + (double)eps));
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int64_t c = threadIdx.x + (int64_t)k * kThreads;
    if (c < nchunks) {
      const uint4 gv = reinterpret_cast<const uint4*>(gamma)[c];
      const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float g0 = bf16_to_f32(gw[e] & 0xFFFFu), g1 = bf16_to_f32(gw[e] >> 16);
        // two separately rounded fp32 products (no fused form exists for mul*mul)
        y[k][2 * e] = (y[k][2 * e] * inv) * g0;
        y[k][2 * e + 1] = (y[k][2 * e + 1] * inv) * g1;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(y[k][e]));
    }
  }
  amax = block_max(amax, shf);
  encode_store<CPT>(y, amax, H, packed + row * (H + 4));
}

int chunks_per_thread(int64_t H) {
  const int64_t need = ceil_div(H / 8, kThreads);
  return need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 8;
}

}  // namespace

hipError_t launch_row_quantize(const void* x, int dtype, int64_t T, int64_t H, uint8_t* packed,
                               hipStream_t s) {
  const int cpt = chunks_per_thread(H);
  const dim3 grid((unsigned)T), block(kThreads);
  const bool bf = dtype == 1;
#define QKVMX_RQ(C)                                                                        \
  case C:                                                                                  \
    if (bf) hipLaunchKernelGGL((row_quantize_kernel<C, true>), grid, block, 0, s, x, H, packed); \
    else hipLaunchKernelGGL((row_quantize_kernel<C, false>), grid, block, 0, s, x, H, packed);   \
    break;
  switch (cpt) { QKVMX_RQ(1) QKVMX_RQ(2) QKVMX_RQ(4) QKVMX_RQ(8) }
#undef QKVMX_RQ
  return hipGetLastError();
}

hipError_t launch_rmsnorm_quantize(const uint16_t* hid, const uint16_t* res, const uint16_t* gamma,
                                   float eps, int64_t T, int64_t H, int64_t Hu, uint16_t* res_out,
                                   uint8_t* packed, hipStream_t s) {
  const int cpt = chunks_per_thread(H);
  const dim3 grid((unsigned)T), block(kThreads);
#define QKVMX_RN(C)                                                                          \
  case C:                                                                                    \
    if (res) hipLaunchKernelGGL((rmsnorm_quantize_kernel<C, true>), grid, block, 0, s, hid, res, \
                                gamma, eps, H, Hu, res_out, packed);                          \
    else hipLaunchKernelGGL((rmsnorm_quantize_kernel<C, false>), grid, block, 0, s, hid, res,    \
                            gamma, eps, H, Hu, res_out, packed);                              \
    break;
  switch (cpt) { QKVMX_RN(1) QKVMX_RN(2) QKVMX_RN(4) QKVMX_RN(8) }
#undef QKVMX_RN
  return hipGetLastError();
}

}  // namespace qkvmx
