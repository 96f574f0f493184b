// ROW_MX activation producers ([QKV-CTE] "Interface", packed_hidden: H FP8 codes + 4-byte fp32
// scale tail per row; [RMSNORM-MX] residual / eps / unpadded_hidden_size).
//
// One block per row, two 8-element chunks per thread (H / 16 threads, rounded up to whole
// wavefronts), the chunks of a thread one block-width apart so each wavefront load covers 1 KiB
// contiguous.  The row stays in registers between the reduction passes, so every input byte is
// read from HBM once and every output byte written once (HBM-bound: per row the fused producer
// moves 4H bytes in and 2H + (H + 4) bytes out).  The packed row is only 4-byte aligned (stride
// H + 4), so its 8-byte code chunks are stored with dword alignment.
#include "device_common.h"
#include "internal.h"

namespace qkvmx {

namespace {

constexpr int kChunk = 8;                  // elements per chunk (one 16-byte bf16 load)
constexpr int kCpt = 2;                    // chunks per thread
constexpr int kMaxWaves = 16;              // H <= 16384
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));

__device__ __forceinline__ float block_max(float v, float* sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  v = sh[0];
  for (int i = 1; i < nw; ++i) v = fmaxf(v, sh[i]);
  return v;
}

// fp64 sum in a fixed order: butterfly within each wavefront, then wavefronts in index order.
__device__ __forceinline__ double block_sum(double v, double* sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  v = sh[0];
  for (int i = 1; i < nw; ++i) v += sh[i];
  return v;
}

__device__ __forceinline__ void unpack8(const uint4 v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = bf16_to_f32(w[e] & 0xFFFFu);
    f[2 * e + 1] = bf16_to_f32(w[e] >> 16);
  }
}

// Chunk k of thread t is chunk c = t + k * blockDim (elements [8 c, 8 c + 8)), so every load
// instruction of a wavefront covers 1 KiB contiguous.
__device__ __forceinline__ int64_t chunk_of(int k) { return threadIdx.x + (int64_t)k * blockDim.x; }

// s = fl32(amax / 448) (IEEE division); codes = E4M3 RNE saturating of fl32(y / s); a zero row
// stores s = 0 and zero codes; thread 0 writes the scale tail.
__device__ __forceinline__ void encode_store(const float (&y)[kCpt][kChunk], float amax,
                                             int64_t H, uint8_t* __restrict__ row_out) {
  const float s = amax / 448.0f;
  const int64_t nchunks = H / kChunk;
#pragma unroll
  for (int k = 0; k < kCpt; ++k) {
    const int64_t c = chunk_of(k);
    if (c < nchunks) {
      uint32_t lo = 0, hi = 0;
      if (s > 0.0f) {
#pragma unroll
        for (int e = 0; e < 4; ++e) lo |= f32_to_e4m3(y[k][e] / s) << (8 * e);
#pragma unroll
        for (int e = 0; e < 4; ++e) hi |= f32_to_e4m3(y[k][4 + e] / s) << (8 * e);
      }
      *reinterpret_cast<u32x2_a4*>(row_out + c * kChunk) = u32x2_a4{lo, hi};
    }
  }
  if (threadIdx.x == 0) *reinterpret_cast<float*>(row_out + H) = s;
}

template <bool BF16>
__global__ void __launch_bounds__(1024) row_quantize_kernel(const void* __restrict__ x, int64_t H,
                                                             uint8_t* __restrict__ packed) {
  __shared__ float sh[kMaxWaves];
  const int64_t row = blockIdx.x;
  const int64_t nchunks = H / kChunk;
  float y[kCpt][kChunk];
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < kCpt; ++k) {
    const int64_t c = chunk_of(k);
#pragma unroll
    for (int e = 0; e < kChunk; ++e) y[k][e] = 0.0f;
    if (c < nchunks) {
      if (BF16) {
        unpack8(reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + row * H)[c],
                y[k]);
      } else {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) +
                                                          row * H) + 2 * c;
        const float4 a = p[0], b = p[1];
        y[k][0] = a.x; y[k][1] = a.y; y[k][2] = a.z; y[k][3] = a.w;
        y[k][4] = b.x; y[k][5] = b.y; y[k][6] = b.z; y[k][7] = b.w;
      }
#pragma unroll
      for (int e = 0; e < kChunk; ++e) amax = fmaxf(amax, fabsf(y[k][e]));
    }
  }
  amax = block_max(amax, sh);
  encode_store(y, amax, H, packed + row * (H + 4));
}

template <bool RES>
__global__ void __launch_bounds__(1024) rmsnorm_quantize_kernel(
    const uint16_t* __restrict__ hid, const uint16_t* __restrict__ res,
    const uint16_t* __restrict__ gamma, float eps, int64_t H, int64_t Hu,
    uint16_t* __restrict__ res_out, uint8_t* __restrict__ packed) {
  __shared__ double shd[kMaxWaves];
  __shared__ float shf[kMaxWaves];
  const int64_t row = blockIdx.x;
  const int64_t nchunks = H / kChunk;
  float y[kCpt][kChunk];
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < kCpt; ++k) {
    const int64_t c = chunk_of(k);
#pragma unroll
    for (int e = 0; e < kChunk; ++e) y[k][e] = 0.0f;
    if (c < nchunks) {
      const uint4 hv = reinterpret_cast<const uint4*>(hid + row * H)[c];
      if (RES) {
        const uint4 rv = reinterpret_cast<const uint4*>(res + row * H)[c];
        const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w};
        const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
        uint32_t ow[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // r = bf16_RNE(fp32 + fp32): one fp32 rounding, then one bf16 rounding
          ow[e] = pack_bf16x2(bf16_to_f32(hw[e] & 0xFFFFu) + bf16_to_f32(rw[e] & 0xFFFFu),
                              bf16_to_f32(hw[e] >> 16) + bf16_to_f32(rw[e] >> 16));
          y[k][2 * e] = bf16_to_f32(ow[e] & 0xFFFFu);
          y[k][2 * e + 1] = bf16_to_f32(ow[e] >> 16);
        }
        reinterpret_cast<uint4*>(res_out + row * H)[c] = make_uint4(ow[0], ow[1], ow[2], ow[3]);
      } else {
        unpack8(hv, y[k]);
      }
#pragma unroll
      for (int e = 0; e < kChunk; ++e) ss += (double)y[k][e] * (double)y[k][e];
    }
  }
  ss = block_sum(ss, shd);
  // inv = fp32(1 / sqrt(ss / Hu + eps)), sqrt and divide correctly rounded in fp64
  const float inv = (float)(1.0 / sqrt(ss / (double)Hu + (double)eps));
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < kCpt; ++k) {
    const int64_t c = chunk_of(k);
    if (c < nchunks) {
      float g[kChunk];
      unpack8(reinterpret_cast<const uint4*>(gamma)[c], g);
#pragma unroll
      for (int e = 0; e < kChunk; ++e) {
        y[k][e] = (y[k][e] * inv) * g[e];    // two separately rounded fp32 products
        amax = fmaxf(amax, fabsf(y[k][e]));
      }
    }
  }
  amax = block_max(amax, shf);
  encode_store(y, amax, H, packed + row * (H + 4));
}

unsigned block_threads(int64_t H) {
  return (unsigned)(ceil_div(ceil_div(H / kChunk, kCpt), 64) * 64);
}

}  // namespace

hipError_t launch_row_quantize(const void* x, int dtype, int64_t T, int64_t H, uint8_t* packed,
                               hipStream_t s) {
  const dim3 grid((unsigned)T), block(block_threads(H));
  if (dtype == 1)
    hipLaunchKernelGGL(row_quantize_kernel<true>, grid, block, 0, s, x, H, packed);
  else
    hipLaunchKernelGGL(row_quantize_kernel<false>, grid, block, 0, s, x, H, packed);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_quantize(const uint16_t* hid, const uint16_t* res, const uint16_t* gamma,
                                   float eps, int64_t T, int64_t H, int64_t Hu, uint16_t* res_out,
                                   uint8_t* packed, hipStream_t s) {
  const dim3 grid((unsigned)T), block(block_threads(H));
  if (res)
    hipLaunchKernelGGL(rmsnorm_quantize_kernel<true>, grid, block, 0, s, hid, res, gamma, eps, H,
                       Hu, res_out, packed);
  else
    hipLaunchKernelGGL(rmsnorm_quantize_kernel<false>, grid, block, 0, s, hid, res, gamma, eps,
                       H, Hu, res_out, packed);
  return hipGetLastError();
}

}  // namespace qkvmx
