// Activation producers: ROW_MX rows ([QKV-CTE] "Interface", packed_hidden: H FP8 codes + 4-byte
// fp32 scale tail per row) and MX block-32 rows ([RMSNORM-MX] qmx_output_dtype: E4M3 codes
// with one E8M0 exponent per 32 elements; emit_norm_bf16), each optionally fused with the
// residual add and RMSNorm ([RMSNORM-MX] residual / eps / unpadded_hidden_size).
//
// Two forms.  The fused producers for rows of up to 8192 elements run one wavefront per row
// (lane l owns the 8-element chunks l, l + 64, ...; both row reductions are exchanges inside
// the wavefront, no LDS, no barrier).  Wider rows and the plain encoders run one block per row,
// two 8-element chunks per thread (H / 16 threads, rounded up to whole wavefronts), the chunks
// of a thread one block-width apart.  Either way each wavefront load covers 1 KiB contiguous and
// the row stays in registers between the reduction passes, so every input byte is read from HBM
// once and every output byte written once (HBM-bound: per row the fused producer moves 4H bytes
// in and 2H + (H + 4) bytes out).  The packed row is only 4-byte aligned (stride H + 4), so its
// 8-byte code chunks are stored with dword alignment.
#include "device_common.h"
#include "internal.h"

namespace qkvmx {

namespace {

constexpr int kChunk = 8;                  // elements per chunk (one 16-byte bf16 load)
constexpr int kCpt = 2;                    // chunks per thread
constexpr int kMaxWaves = 16;              // H <= 16384
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// 8 bf16 values read once (streaming load: the producer's inputs are not re-read).
__device__ __forceinline__ uint4 ntload16(const uint16_t* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

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

// Destinations of an encoded ROW_MX row.
// PackedRow: the pages' packed row, H codes then the fp32 scale (4-byte tail at byte H).
struct PackedRow {
  uint8_t* row;
  int64_t H;
  __device__ uint8_t* chunk(int64_t c) const { return row + c * kChunk; }
  __device__ void scale(float s) const { *reinterpret_cast<float*>(row + H) = s; }
  __device__ int64_t pad_chunks() const { return 0; }
};
// StagedRow: the projection's stage-image layout.  Codes of row m, K-byte h go to image offset
// ((m / 256 * KS + h / 64) * 256 + m % 256) * 64 + (((h / 16) % 4 ^ stage_swizzle(m % 256)) << 4)
// + h % 16 (the layout its K-loop DMA-copies into LDS unchanged); K-bytes from H up to KS * 64
// are written as zero codes; the scale goes to a separate fp32 array.
struct StagedRow {
  uint8_t* base;      // image + (m / 256 * KS) * kStageImage + (m % 256) * kStage
  int swz;            // stage_swizzle(m % 256)
  float* scale_p;     // &row_scale[m]
  int64_t padded;     // KS * 64 / kChunk chunks per row in the image
  __device__ uint8_t* chunk(int64_t c) const {
    return base + (c >> 3) * kStageImage + ((((int)(c >> 1) & 3) ^ swz) << 4) + (c & 1) * kChunk;
  }
  __device__ void scale(float s) const { *scale_p = s; }
  __device__ int64_t pad_chunks() const { return padded; }
};

// s = fl32(amax / 448) (IEEE division); codes = E4M3 RNE saturating of fl32(y / s); a zero row
// stores s = 0 and zero codes; thread 0 writes the scale.
// fl32(y / s) is formed as fl32(fl64(y * fl64(1 / s))): the fp64 product is within 2^-52 of
// y / s, while a quotient of two fp32 numbers never is an fp32 rounding midpoint and lies at
// least 2^-49 (relative) away from every one, so rounding the product to fp32 gives exactly the
// IEEE quotient for every normal result (results below 2^-126 encode to a signed zero code
// either way).  One fp64 divide per thread replaces an fp32 divide per element.
template <typename Dst>
__device__ __forceinline__ void encode_store(const float (&y)[kCpt][kChunk], float amax,
                                             int64_t H, const Dst& dst) {
  const float s = amax / 448.0f;
  const double rinv = 1.0 / (double)s;
  const int64_t nchunks = H / kChunk;
#pragma unroll
  for (int k = 0; k < kCpt; ++k) {
    const int64_t c = chunk_of(k);
    if (c < nchunks) {
      uint32_t lo = 0, hi = 0;
      if (s > 0.0f) {
        float q[kChunk];
#pragma unroll
        for (int e = 0; e < kChunk; ++e) q[e] = (float)((double)y[k][e] * rinv);
        lo = e4m3x4(q[0], q[1], q[2], q[3]);
        hi = e4m3x4(q[4], q[5], q[6], q[7]);
      }
      *reinterpret_cast<u32x2_a4*>(dst.chunk(c)) = u32x2_a4{lo, hi};
    } else if (c < dst.pad_chunks()) {
      *reinterpret_cast<u32x2_a4*>(dst.chunk(c)) = u32x2_a4{0u, 0u};
    }
  }
  if (threadIdx.x == 0) dst.scale(s);
}

// The staged destination of row m (KS K-stages per row).
__device__ __forceinline__ StagedRow staged_row(uint8_t* img, float* row_scale, int64_t m, int KS) {
  const int r = (int)(m & (kTileM - 1));
  return StagedRow{img + (m / kTileM) * KS * (int64_t)kStageImage + (int64_t)r * kStage,
                   stage_swizzle(r), row_scale + m, (int64_t)KS * kStage / kChunk};
}

// Rows from T up to the end of the last 256-row tile of a staged image: zero codes (the
// projection multiplies them but never stores their outputs).  One block per row.
__device__ __forceinline__ void staged_zero_row(uint8_t* img, int64_t m, int KS) {
  const StagedRow d = staged_row(img, nullptr, m, KS);
  for (int64_t c = threadIdx.x; c < d.padded; c += blockDim.x)
    *reinterpret_cast<u32x2_a4*>(d.chunk(c)) = u32x2_a4{0u, 0u};
}

// y = x (fp32 or bf16 rows), ROW_MX encoded into packed rows [T, H + 4] or, with STAGED, into
// the stage-image layout plus fp32 row scales (grid: T rows, rounded up to whole 256-row tiles).
template <bool BF16, bool STAGED>
__global__ void __launch_bounds__(1024) row_quantize_kernel(const void* __restrict__ x, int64_t T,
                                                             int64_t H, uint8_t* __restrict__ out,
                                                             float* __restrict__ row_scale,
                                                             int KS) {
  __shared__ float sh[kMaxWaves];
  const int64_t row = blockIdx.x;
  if (STAGED && row >= T) {
    staged_zero_row(out, row, KS);
    return;
  }
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
  if (STAGED)
    encode_store(y, amax, H, staged_row(out, row_scale, row, KS));
  else
    encode_store(y, amax, H, PackedRow{out + row * (H + 4), H});
}

// Steps 1-4 of the fused producer for one row, into registers y (zeros past H):
//   r = bf16_RNE(fp32(hid) + fp32(res)) -> res_out (r = hid without a residual);
//   inv = fp32(1 / sqrt(sum r^2 / Hu + eps)), the sum (fixed order), sqrt and divide in fp64;
//   y = fl32(fl32(r * inv) * gamma).
template <bool RES>
__device__ __forceinline__ void normed_row(const uint16_t* __restrict__ hid,
                                           const uint16_t* __restrict__ res,
                                           const uint16_t* __restrict__ gamma, float eps,
                                           int64_t H, int64_t Hu, uint16_t* __restrict__ res_out,
                                           int64_t row, float (&y)[kCpt][kChunk], double* shd) {
  const int64_t nchunks = H / kChunk;
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < kCpt; ++k) {
    const int64_t c = chunk_of(k);
#pragma unroll
    for (int e = 0; e < kChunk; ++e) y[k][e] = 0.0f;
    if (c < nchunks) {
      const uint4 hv = ntload16(hid + row * H + c * kChunk);
      if (RES) {
        const uint4 rv = ntload16(res + row * H + c * kChunk);
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
        __builtin_nontemporal_store(u32x4_t{ow[0], ow[1], ow[2], ow[3]},
                                    reinterpret_cast<u32x4_t*>(res_out + row * H + c * kChunk));
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
#pragma unroll
  for (int k = 0; k < kCpt; ++k) {
    const int64_t c = chunk_of(k);
    if (c < nchunks) {
      float g[kChunk];
      unpack8(reinterpret_cast<const uint4*>(gamma)[c], g);
#pragma unroll
      for (int e = 0; e < kChunk; ++e) y[k][e] = (y[k][e] * inv) * g[e];   // two fp32 roundings
    }
  }
}

// One wavefront per row (rows of up to 512 NC elements): lane l owns the 8-element chunks
// l, l + 64, .., l + 64 (NC - 1), so each load instruction of the wavefront covers 1 KiB
// contiguous, and both row reductions (the fp64 sum of squares and the maximum) are butterfly
// exchanges inside the wavefront: no LDS, no block barrier between a row's loads and its
// stores.  Arithmetic, rounding and the reduction's fixed order (the same butterfly on every
// lane, so every lane holds the identical sum) follow normed_row / encode_store.
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

constexpr int kRowsPerWaveBlock = 4;       // rows (wavefronts) per 256-thread block

// Steps 1-4 of the fused producer for one row on one wavefront (lane l: chunks l + 64 k), into
// registers y (zeros past H), with the lane's share of max |y| in amax: the arithmetic of
// normed_row, the fp64 sum by a butterfly inside the wavefront.
template <bool RES, int NC>
__device__ __forceinline__ void wave_normed_row(const uint16_t* __restrict__ hid,
                                                const uint16_t* __restrict__ res,
                                                const uint16_t* __restrict__ gamma, float eps,
                                                int64_t H, int64_t Hu,
                                                uint16_t* __restrict__ res_out, int64_t row,
                                                int lane, float (&y)[NC][kChunk], float& amax) {
  const int64_t nchunks = H / kChunk;
  // all of the row's loads first (2 NC x 16 bytes per lane in flight)
  uint4 hv[NC], rv[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int64_t c = lane + 64 * k;
    if (c < nchunks) {
      hv[k] = ntload16(hid + row * H + c * kChunk);
      if (RES) rv[k] = ntload16(res + row * H + c * kChunk);
    }
  }
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int64_t c = lane + 64 * k;
#pragma unroll
    for (int e = 0; e < kChunk; ++e) y[k][e] = 0.0f;
    if (c < nchunks) {
      if (RES) {
        const uint32_t hw[4] = {hv[k].x, hv[k].y, hv[k].z, hv[k].w};
        const uint32_t rw[4] = {rv[k].x, rv[k].y, rv[k].z, rv[k].w};
        uint32_t ow[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // r = bf16_RNE(fp32 + fp32): one fp32 rounding, then one bf16 rounding
          ow[e] = pack_bf16x2(bf16_to_f32(hw[e] & 0xFFFFu) + bf16_to_f32(rw[e] & 0xFFFFu),
                              bf16_to_f32(hw[e] >> 16) + bf16_to_f32(rw[e] >> 16));
          y[k][2 * e] = bf16_to_f32(ow[e] & 0xFFFFu);
          y[k][2 * e + 1] = bf16_to_f32(ow[e] >> 16);
        }
        __builtin_nontemporal_store(u32x4_t{ow[0], ow[1], ow[2], ow[3]},
                                    reinterpret_cast<u32x4_t*>(res_out + row * H + c * kChunk));
      } else {
        unpack8(hv[k], y[k]);
      }
#pragma unroll
      for (int e = 0; e < kChunk; ++e) ss += (double)y[k][e] * (double)y[k][e];
    }
  }
  ss = wave_sum(ss);
  // inv = fp32(1 / sqrt(ss / Hu + eps)), sqrt and divide correctly rounded in fp64
  const float inv = (float)(1.0 / sqrt(ss / (double)Hu + (double)eps));
  amax = 0.0f;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int64_t c = lane + 64 * k;
    if (c < nchunks) {
      float g[kChunk];
      unpack8(reinterpret_cast<const uint4*>(gamma)[c], g);
#pragma unroll
      for (int e = 0; e < kChunk; ++e) {
        y[k][e] = (y[k][e] * inv) * g[e];                       // two fp32 roundings
        amax = fmaxf(amax, fabsf(y[k][e]));
      }
    }
  }
}

template <bool RES, bool STAGED, int NC>
__global__ void __launch_bounds__(64 * kRowsPerWaveBlock) rmsnorm_quantize_wave_kernel(
    const uint16_t* __restrict__ hid, const uint16_t* __restrict__ res,
    const uint16_t* __restrict__ gamma, float eps, int64_t T, int64_t H, int64_t Hu,
    uint16_t* __restrict__ res_out, uint8_t* __restrict__ out, float* __restrict__ row_scale,
    int KS, int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerWaveBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int64_t nchunks = H / kChunk;
  if (STAGED && row >= T) {                 // rows past T up to the tile end: zero codes
    const StagedRow d = staged_row(out, nullptr, row, KS);
    for (int64_t c = lane; c < d.padded; c += 64)
      *reinterpret_cast<u32x2_a4*>(d.chunk(c)) = u32x2_a4{0u, 0u};
    return;
  }
  float y[NC][kChunk];
  float amax;
  wave_normed_row<RES, NC>(hid, res, gamma, eps, H, Hu, res_out, row, lane, y, amax);
  amax = wave_max(amax);
  // s = fl32(amax / 448); codes = E4M3 RNE saturating of fl32(y / s), formed as
  // fl32(fl64(y * fl64(1 / s))) (exact: see encode_store); a zero row stores s = 0, zero codes
  const float s = amax / 448.0f;
  const double rinv = 1.0 / (double)s;
  StagedRow sd{};
  if (STAGED) sd = staged_row(out, row_scale, row, KS);
  uint8_t* const prow = out + row * (H + 4);
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int64_t c = lane + 64 * k;
    if (c < nchunks) {
      uint32_t lo = 0, hi = 0;
      if (s > 0.0f) {
        float q[kChunk];
#pragma unroll
        for (int e = 0; e < kChunk; ++e) q[e] = (float)((double)y[k][e] * rinv);
        lo = e4m3x4(q[0], q[1], q[2], q[3]);
        hi = e4m3x4(q[4], q[5], q[6], q[7]);
      }
      *reinterpret_cast<u32x2_a4*>(STAGED ? sd.chunk(c) : prow + c * kChunk) = u32x2_a4{lo, hi};
    }
  }
  if (STAGED) {                             // K-bytes from H to the stage end: zero codes
    for (int64_t c = nchunks + lane; c < sd.padded; c += 64)
      *reinterpret_cast<u32x2_a4*>(sd.chunk(c)) = u32x2_a4{0u, 0u};
  }
  if (lane == 0) {
    if (STAGED) sd.scale(s);
    else *reinterpret_cast<float*>(prow + H) = s;
  }
}

// The fused MX block-32 producer on one wavefront per row (rows of up to 512 NC elements):
// wave_normed_row, then each 32-element block (4 consecutive chunks on 4 consecutive lanes) as
// in mx_encode_codes, the block maximum by two lane exchanges.  Natural layout: the block's
// first lane stores its exponent byte.  Staged layout: the exponent dword (superstep s, g)
// holds blocks 8 s + 2 q + g, q = 0..3, which sit on lanes L, L + 8, L + 16, L + 24 of the
// superstep's 32-lane half (L = 4 g); lane L gathers them by shuffles and stores the dword, 127
// for blocks past H / 32, as mx_store_exponents_staged does.  Codes go out through ordinary
// (cached) stores, as in the ROW_MX wave kernel: a 128-byte line of the staged image holds the
// 64-byte stage segments of two neighbouring rows, both written by the same 4-row block, so L2
// merges the halves before the line leaves (8-byte streaming stores measured 8% slower at the
// video shape).  The block-per-row kernel below, whose neighbouring row is another block, keeps
// streaming stores: ordinary ones measured 3% slower there (H = 16384).
template <bool RES, bool EMIT, bool STAGED, int NC>
__global__ void __launch_bounds__(64 * kRowsPerWaveBlock) rmsnorm_mx_wave_kernel(
    const uint16_t* __restrict__ hid, const uint16_t* __restrict__ res,
    const uint16_t* __restrict__ gamma, float eps, int64_t T, int64_t H, int64_t Hu,
    uint16_t* __restrict__ res_out, uint8_t* __restrict__ codes, uint8_t* __restrict__ e8,
    uint16_t* __restrict__ norm_out, int KS, int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerWaveBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int64_t nchunks = H / kChunk;
  const int S = KS / 4;                     // staged: supersteps of 256 elements
  uint32_t* const erow = STAGED ? reinterpret_cast<uint32_t*>(e8) +
                                      ((row / kTileM) * S * kTileM + (row & (kTileM - 1))) * 2
                                : nullptr;
  if (STAGED && row >= T) {                 // rows past T up to the tile end
    const StagedRow d = staged_row(codes, nullptr, row, KS);
    for (int64_t c = lane; c < d.padded; c += 64)
      *reinterpret_cast<u32x2_a4*>(d.chunk(c)) = u32x2_a4{0u, 0u};
    for (int i = lane; i < 2 * S; i += 64) erow[(int64_t)(i >> 1) * kTileM * 2 + (i & 1)] = 0x7F7F7F7Fu;
    return;
  }
  float y[NC][kChunk];
  float amax_unused;
  wave_normed_row<RES, NC>(hid, res, gamma, eps, H, Hu, res_out, row, lane, y, amax_unused);
  StagedRow sd{};
  if (STAGED) sd = staged_row(codes, nullptr, row, KS);
  uint8_t* const crow = codes + row * H;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int64_t c = lane + 64 * k;
    if (EMIT && c < nchunks)
      reinterpret_cast<uint4*>(norm_out + row * H)[c] =
          make_uint4(pack_bf16x2(y[k][0], y[k][1]), pack_bf16x2(y[k][2], y[k][3]),
                     pack_bf16x2(y[k][4], y[k][5]), pack_bf16x2(y[k][6], y[k][7]));
    // every lane takes part in the exchanges (a 4-lane group is entirely inside or past H)
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < kChunk; ++e) m = fmaxf(m, fabsf(y[k][e]));
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    const int eb = (int)((__float_as_uint(m) >> 23) & 0xFFu);
    const uint32_t E = (uint32_t)max(eb - 8, 0);
    const float inv = __uint_as_float((254u - E) << 23);          // 2^(127 - E)
    if (c < nchunks) {
      uint32_t lo = 0, hi = 0;
      if (m > 0.0f) {
        lo = e4m3x4(y[k][0] * inv, y[k][1] * inv, y[k][2] * inv, y[k][3] * inv);
        hi = e4m3x4(y[k][4] * inv, y[k][5] * inv, y[k][6] * inv, y[k][7] * inv);
      }
      *reinterpret_cast<u32x2_a4*>(STAGED ? sd.chunk(c) : crow + c * kChunk) = u32x2_a4{lo, hi};
      if (!STAGED && (c & 3) == 0) e8[row * (H / 32) + (c >> 2)] = (uint8_t)E;
    } else if (STAGED && c < sd.padded) {
      *reinterpret_cast<u32x2_a4*>(sd.chunk(c)) = u32x2_a4{0u, 0u};
    }
    if (STAGED) {
      const uint32_t el = c < nchunks ? E : 127u;   // blocks past H / 32: 2^0
      const uint32_t e1 = (uint32_t)__shfl((int)el, lane + 8);
      const uint32_t e2 = (uint32_t)__shfl((int)el, lane + 16);
      const uint32_t e3 = (uint32_t)__shfl((int)el, lane + 24);
      const int in_half = lane & 31;
      const int sidx = 2 * k + (lane >> 5);
      if ((in_half == 0 || in_half == 4) && sidx < S)
        erow[(int64_t)sidx * kTileM * 2 + (in_half >> 2)] = el | (e1 << 8) | (e2 << 16) | (e3 << 24);
    }
  }
  // (every superstep s < S = ceil(H / 256) <= 2 NC has its dwords stored in the loop above)
}

template <bool RES, bool STAGED>
__global__ void __launch_bounds__(1024) rmsnorm_quantize_kernel(
    const uint16_t* __restrict__ hid, const uint16_t* __restrict__ res,
    const uint16_t* __restrict__ gamma, float eps, int64_t T, int64_t H, int64_t Hu,
    uint16_t* __restrict__ res_out, uint8_t* __restrict__ out, float* __restrict__ row_scale,
    int KS) {
  __shared__ double shd[kMaxWaves];
  __shared__ float shf[kMaxWaves];
  const int64_t row = blockIdx.x;
  if (STAGED && row >= T) {
    staged_zero_row(out, row, KS);
    return;
  }
  float y[kCpt][kChunk];
  normed_row<RES>(hid, res, gamma, eps, H, Hu, res_out, row, y, shd);
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < kCpt; ++k)
#pragma unroll
    for (int e = 0; e < kChunk; ++e) amax = fmaxf(amax, fabsf(y[k][e]));
  amax = block_max(amax, shf);
  if (STAGED)
    encode_store(y, amax, H, staged_row(out, row_scale, row, KS));
  else
    encode_store(y, amax, H, PackedRow{out + row * (H + 4), H});
}

// MX block-32 encoding of y (the 4 consecutive chunks of a 32-element block belong to 4
// consecutive lanes, aligned to 4): block maximum by two lane exchanges, shared exponent
// E = max(biased exponent of amax - 8, 0) (floor(log2 amax) - 8 + 127, clamped at 0; amax < 2^-119
// or zero gives 0), codes = E4M3 RNE saturating of y * 2^(127 - E) (a power-of-two scaling,
// exact for every value that does not round to zero); an all-zero block stores zero codes.
// Codes go to chunk_at(c) (8 bytes per chunk; chunks in [H / 8, pad_chunks) get zero codes),
// exponents to sh_e[block] in LDS; the caller stores them after the barrier that ends this.
template <typename ChunkAt>
__device__ __forceinline__ void mx_encode_codes(const float (&y)[kCpt][kChunk], int64_t H,
                                                ChunkAt chunk_at, int64_t pad_chunks,
                                                uint8_t* sh_e) {
  const int64_t nchunks = H / kChunk;
#pragma unroll
  for (int k = 0; k < kCpt; ++k) {
    const int64_t c = chunk_of(k);
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < kChunk; ++e) m = fmaxf(m, fabsf(y[k][e]));
    // every lane of a 4-lane group takes part (a group is entirely inside or past the row)
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    const int eb = (int)((__float_as_uint(m) >> 23) & 0xFFu);
    const uint32_t E = (uint32_t)max(eb - 8, 0);
    const float inv = __uint_as_float((254u - E) << 23);          // 2^(127 - E)
    if (c < nchunks) {
      uint32_t lo = 0, hi = 0;
      if (m > 0.0f) {
        lo = e4m3x4(y[k][0] * inv, y[k][1] * inv, y[k][2] * inv, y[k][3] * inv);
        hi = e4m3x4(y[k][4] * inv, y[k][5] * inv, y[k][6] * inv, y[k][7] * inv);
      }
      __builtin_nontemporal_store(u32x2_t{lo, hi}, reinterpret_cast<u32x2_t*>(chunk_at(c)));
      if ((c & 3) == 0) sh_e[c >> 2] = (uint8_t)E;
    } else if (c < pad_chunks) {
      __builtin_nontemporal_store(u32x2_t{0u, 0u}, reinterpret_cast<u32x2_t*>(chunk_at(c)));
    }
  }
  __syncthreads();
}

// The exponents of one row, natural order: e8_row[b] = exponent of elements [32 b, 32 b + 32).
__device__ __forceinline__ void mx_store_exponents(int64_t H, uint8_t* __restrict__ e8_row,
                                                   const uint8_t* sh_e) {
  if (H % 128 == 0) {                              // whole dwords (the row start is 4-aligned)
    for (int64_t i = threadIdx.x; i < H / 128; i += blockDim.x)
      reinterpret_cast<uint32_t*>(e8_row)[i] = reinterpret_cast<const uint32_t*>(sh_e)[i];
  } else {
    for (int64_t i = threadIdx.x; i < H / 32; i += blockDim.x) e8_row[i] = sh_e[i];
  }
}

// The exponents of row m in the staged exponent image [MT][S][256][2] dwords (S = KS / 4
// supersteps of 256 elements): byte q of dword g of superstep s = exponent of block
// 8 s + 2 q + g, 127 (2^0) for blocks past H / 32; sh_e null: a row past T (all 127).
__device__ __forceinline__ void mx_store_exponents_staged(int64_t H, uint32_t* __restrict__ eimg,
                                                          int64_t m, int S, const uint8_t* sh_e) {
  const int64_t nblocks = H / 32;
  uint32_t* row = eimg + ((m / kTileM) * S * kTileM + (m & (kTileM - 1))) * 2;
  for (int i = threadIdx.x; i < 2 * S; i += blockDim.x) {
    const int sidx = i >> 1, g = i & 1;
    uint32_t w = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t b = 8 * (int64_t)sidx + 2 * q + g;
      const uint32_t e = (sh_e && b < nblocks) ? sh_e[b] : 127u;
      w |= e << (8 * q);
    }
    row[(int64_t)sidx * kTileM * 2 + g] = w;
  }
}

// y = x (fp32 or bf16 rows), MX block-32 encoded: codes [T, H] and exponents [T, H / 32], or
// with STAGED the codes in the stage-image layout and the exponents in the staged exponent
// image (grid: T rows rounded up to whole 256-row tiles; rows past T get zero codes and
// exponents 127).
template <bool BF16, bool STAGED>
__global__ void __launch_bounds__(1024) mx_quantize_kernel(const void* __restrict__ x, int64_t T,
                                                            int64_t H, uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ e8, int KS) {
  __shared__ __attribute__((aligned(4))) uint8_t sh_e[kMaxWaves * 64 * kCpt * kChunk / 32];
  const int64_t row = blockIdx.x;
  if (STAGED && row >= T) {
    staged_zero_row(codes, row, KS);
    mx_store_exponents_staged(H, reinterpret_cast<uint32_t*>(e8), row, KS / 4, nullptr);
    return;
  }
  const int64_t nchunks = H / kChunk;
  float y[kCpt][kChunk];
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
    }
  }
  if (STAGED) {
    const StagedRow d = staged_row(codes, nullptr, row, KS);
    mx_encode_codes(y, H, [&](int64_t c) { return d.chunk(c); }, d.padded, sh_e);
    mx_store_exponents_staged(H, reinterpret_cast<uint32_t*>(e8), row, KS / 4, sh_e);
  } else {
    uint8_t* crow = codes + row * H;
    mx_encode_codes(y, H, [&](int64_t c) { return crow + c * kChunk; }, 0, sh_e);
    mx_store_exponents(H, e8 + row * (H / 32), sh_e);
  }
}

// Residual add + RMSNorm (the steps of rmsnorm_quantize_kernel), then MX block-32 encoding of
// y (natural or, with STAGED, staged layouts as mx_quantize_kernel) and, with EMIT, y rounded
// to bf16 (RNE) into norm_out.
template <bool RES, bool EMIT, bool STAGED>
__global__ void __launch_bounds__(1024) rmsnorm_mx_kernel(
    const uint16_t* __restrict__ hid, const uint16_t* __restrict__ res,
    const uint16_t* __restrict__ gamma, float eps, int64_t T, int64_t H, int64_t Hu,
    uint16_t* __restrict__ res_out, uint8_t* __restrict__ codes, uint8_t* __restrict__ e8,
    uint16_t* __restrict__ norm_out, int KS) {
  __shared__ double shd[kMaxWaves];
  __shared__ __attribute__((aligned(4))) uint8_t sh_e[kMaxWaves * 64 * kCpt * kChunk / 32];
  const int64_t row = blockIdx.x;
  if (STAGED && row >= T) {
    staged_zero_row(codes, row, KS);
    mx_store_exponents_staged(H, reinterpret_cast<uint32_t*>(e8), row, KS / 4, nullptr);
    return;
  }
  float y[kCpt][kChunk];
  normed_row<RES>(hid, res, gamma, eps, H, Hu, res_out, row, y, shd);
  if (EMIT) {
    const int64_t nchunks = H / kChunk;
#pragma unroll
    for (int k = 0; k < kCpt; ++k) {
      const int64_t c = chunk_of(k);
      if (c < nchunks)
        reinterpret_cast<uint4*>(norm_out + row * H)[c] =
            make_uint4(pack_bf16x2(y[k][0], y[k][1]), pack_bf16x2(y[k][2], y[k][3]),
                       pack_bf16x2(y[k][4], y[k][5]), pack_bf16x2(y[k][6], y[k][7]));
    }
  }
  if (STAGED) {
    const StagedRow d = staged_row(codes, nullptr, row, KS);
    mx_encode_codes(y, H, [&](int64_t c) { return d.chunk(c); }, d.padded, sh_e);
    mx_store_exponents_staged(H, reinterpret_cast<uint32_t*>(e8), row, KS / 4, sh_e);
  } else {
    uint8_t* crow = codes + row * H;
    mx_encode_codes(y, H, [&](int64_t c) { return crow + c * kChunk; }, 0, sh_e);
    mx_store_exponents(H, e8 + row * (H / 32), sh_e);
  }
}

unsigned block_threads(int64_t H) {
  return (unsigned)(ceil_div(ceil_div(H / kChunk, kCpt), 64) * 64);
}

}  // namespace

hipError_t launch_row_quantize(const void* x, int dtype, int64_t T, int64_t H, uint8_t* packed,
                               hipStream_t s) {
  const dim3 grid((unsigned)T), block(block_threads(H));
  if (dtype == 1)
    hipLaunchKernelGGL((row_quantize_kernel<true, false>), grid, block, 0, s, x, T, H, packed,
                       nullptr, 0);
  else
    hipLaunchKernelGGL((row_quantize_kernel<false, false>), grid, block, 0, s, x, T, H, packed,
                       nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_row_quantize_staged(const void* x, int dtype, int64_t T, int64_t H,
                                      uint8_t* img, float* row_scale, hipStream_t s) {
  const dim3 grid((unsigned)(ceil_div(T, kTileM) * kTileM)), block(block_threads(H));
  const int KS = (int)packed_stages(H);
  if (dtype == 1)
    hipLaunchKernelGGL((row_quantize_kernel<true, true>), grid, block, 0, s, x, T, H, img,
                       row_scale, KS);
  else
    hipLaunchKernelGGL((row_quantize_kernel<false, true>), grid, block, 0, s, x, T, H, img,
                       row_scale, KS);
  return hipGetLastError();
}

// The fused ROW_MX producer, one wavefront per row, for rows of up to 512 NC elements (NC
// chunks of 8 per lane): false (nothing launched) when H is wider than the widest instance.
template <bool STAGED>
bool launch_rmsnorm_quantize_wave(const uint16_t* hid, const uint16_t* res,
                                  const uint16_t* gamma, float eps, int64_t T, int64_t H,
                                  int64_t Hu, uint16_t* res_out, uint8_t* out, float* row_scale,
                                  int KS, hipStream_t s) {
  const int64_t rows = STAGED ? ceil_div(T, kTileM) * kTileM : T;
  const dim3 grid((unsigned)ceil_div(rows, kRowsPerWaveBlock)), block(64 * kRowsPerWaveBlock);
  const int64_t nc = ceil_div(H, (int64_t)64 * kChunk);
#define QKVMX_WAVE_PRODUCER(N)                                                                   \
  do {                                                                                           \
    if (res)                                                                                     \
      hipLaunchKernelGGL((rmsnorm_quantize_wave_kernel<true, STAGED, N>), grid, block, 0, s,     \
                         hid, res, gamma, eps, T, H, Hu, res_out, out, row_scale, KS, rows);    \
    else                                                                                         \
      hipLaunchKernelGGL((rmsnorm_quantize_wave_kernel<false, STAGED, N>), grid, block, 0, s,    \
                         hid, res, gamma, eps, T, H, Hu, res_out, out, row_scale, KS, rows);    \
  } while (0)
  if (nc <= 2) QKVMX_WAVE_PRODUCER(2);
  else if (nc <= 4) QKVMX_WAVE_PRODUCER(4);
  else if (nc <= 8) QKVMX_WAVE_PRODUCER(8);
  else if (nc <= 10) QKVMX_WAVE_PRODUCER(10);
  else if (nc <= 16) QKVMX_WAVE_PRODUCER(16);
  else return false;
#undef QKVMX_WAVE_PRODUCER
  return true;
}

hipError_t launch_rmsnorm_quantize(const uint16_t* hid, const uint16_t* res, const uint16_t* gamma,
                                   float eps, int64_t T, int64_t H, int64_t Hu, uint16_t* res_out,
                                   uint8_t* packed, hipStream_t s) {
  if (launch_rmsnorm_quantize_wave<false>(hid, res, gamma, eps, T, H, Hu, res_out, packed,
                                          nullptr, 0, s))
    return hipGetLastError();
  const dim3 grid((unsigned)T), block(block_threads(H));
  if (res)
    hipLaunchKernelGGL((rmsnorm_quantize_kernel<true, false>), grid, block, 0, s, hid, res,
                       gamma, eps, T, H, Hu, res_out, packed, nullptr, 0);
  else
    hipLaunchKernelGGL((rmsnorm_quantize_kernel<false, false>), grid, block, 0, s, hid, res,
                       gamma, eps, T, H, Hu, res_out, packed, nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_quantize_staged(const uint16_t* hid, const uint16_t* res,
                                          const uint16_t* gamma, float eps, int64_t T, int64_t H,
                                          int64_t Hu, uint16_t* res_out, uint8_t* img,
                                          float* row_scale, hipStream_t s) {
  const int KS = (int)packed_stages(H);
  if (launch_rmsnorm_quantize_wave<true>(hid, res, gamma, eps, T, H, Hu, res_out, img,
                                         row_scale, KS, s))
    return hipGetLastError();
  const dim3 grid((unsigned)(ceil_div(T, kTileM) * kTileM)), block(block_threads(H));
  if (res)
    hipLaunchKernelGGL((rmsnorm_quantize_kernel<true, true>), grid, block, 0, s, hid, res,
                       gamma, eps, T, H, Hu, res_out, img, row_scale, KS);
  else
    hipLaunchKernelGGL((rmsnorm_quantize_kernel<false, true>), grid, block, 0, s, hid, res,
                       gamma, eps, T, H, Hu, res_out, img, row_scale, KS);
  return hipGetLastError();
}

hipError_t launch_mx_quantize(const void* x, int dtype, int64_t T, int64_t H, uint8_t* codes,
                              uint8_t* e8, hipStream_t s) {
  const dim3 grid((unsigned)T), block(block_threads(H));
  if (dtype == 1)
    hipLaunchKernelGGL((mx_quantize_kernel<true, false>), grid, block, 0, s, x, T, H, codes, e8, 0);
  else
    hipLaunchKernelGGL((mx_quantize_kernel<false, false>), grid, block, 0, s, x, T, H, codes, e8, 0);
  return hipGetLastError();
}

hipError_t launch_mx_quantize_staged(const void* x, int dtype, int64_t T, int64_t H,
                                     uint8_t* img, uint32_t* eimg, hipStream_t s) {
  const dim3 grid((unsigned)(ceil_div(T, kTileM) * kTileM)), block(block_threads(H));
  const int KS = (int)packed_stages(H);
  uint8_t* e = reinterpret_cast<uint8_t*>(eimg);
  if (dtype == 1)
    hipLaunchKernelGGL((mx_quantize_kernel<true, true>), grid, block, 0, s, x, T, H, img, e, KS);
  else
    hipLaunchKernelGGL((mx_quantize_kernel<false, true>), grid, block, 0, s, x, T, H, img, e, KS);
  return hipGetLastError();
}

namespace {

template <bool STAGED>
hipError_t launch_rmsnorm_mx_any(const uint16_t* hid, const uint16_t* res, const uint16_t* gamma,
                                 float eps, int64_t T, int64_t H, int64_t Hu, uint16_t* res_out,
                                 uint8_t* codes, uint8_t* e8, uint16_t* norm_out, hipStream_t s) {
  const int KS = STAGED ? (int)packed_stages(H) : 0;
  const int v = (res ? 2 : 0) | (norm_out ? 1 : 0);
  // rows of up to 8192 elements: one wavefront per row
  const int64_t rows = STAGED ? ceil_div(T, kTileM) * kTileM : T;
  const int64_t nc = ceil_div(H, (int64_t)64 * kChunk);
  const dim3 wgrid((unsigned)ceil_div(rows, kRowsPerWaveBlock)), wblock(64 * kRowsPerWaveBlock);
#define QKVMX_MX_WAVE(N)                                                                          \
  do {                                                                                            \
    switch (v) {                                                                                  \
      case 0: hipLaunchKernelGGL((rmsnorm_mx_wave_kernel<false, false, STAGED, N>), wgrid, wblock, 0, s, hid, res, gamma, eps, T, H, Hu, res_out, codes, e8, norm_out, KS, rows); break; \
      case 1: hipLaunchKernelGGL((rmsnorm_mx_wave_kernel<false, true, STAGED, N>), wgrid, wblock, 0, s, hid, res, gamma, eps, T, H, Hu, res_out, codes, e8, norm_out, KS, rows); break; \
      case 2: hipLaunchKernelGGL((rmsnorm_mx_wave_kernel<true, false, STAGED, N>), wgrid, wblock, 0, s, hid, res, gamma, eps, T, H, Hu, res_out, codes, e8, norm_out, KS, rows); break; \
      default: hipLaunchKernelGGL((rmsnorm_mx_wave_kernel<true, true, STAGED, N>), wgrid, wblock, 0, s, hid, res, gamma, eps, T, H, Hu, res_out, codes, e8, norm_out, KS, rows); break; \
    }                                                                                             \
    return hipGetLastError();                                                                     \
  } while (0)
  if (nc <= 2) QKVMX_MX_WAVE(2);
  if (nc <= 4) QKVMX_MX_WAVE(4);
  if (nc <= 8) QKVMX_MX_WAVE(8);
  if (nc <= 10) QKVMX_MX_WAVE(10);
  if (nc <= 16) QKVMX_MX_WAVE(16);
#undef QKVMX_MX_WAVE
  const dim3 grid((unsigned)(STAGED ? ceil_div(T, kTileM) * kTileM : T)), block(block_threads(H));
  switch (v) {
    case 0: hipLaunchKernelGGL((rmsnorm_mx_kernel<false, false, STAGED>), grid, block, 0, s, hid, res, gamma, eps, T, H, Hu, res_out, codes, e8, norm_out, KS); break;
    case 1: hipLaunchKernelGGL((rmsnorm_mx_kernel<false, true, STAGED>), grid, block, 0, s, hid, res, gamma, eps, T, H, Hu, res_out, codes, e8, norm_out, KS); break;
    case 2: hipLaunchKernelGGL((rmsnorm_mx_kernel<true, false, STAGED>), grid, block, 0, s, hid, res, gamma, eps, T, H, Hu, res_out, codes, e8, norm_out, KS); break;
    default: hipLaunchKernelGGL((rmsnorm_mx_kernel<true, true, STAGED>), grid, block, 0, s, hid, res, gamma, eps, T, H, Hu, res_out, codes, e8, norm_out, KS); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm_mx(const uint16_t* hid, const uint16_t* res, const uint16_t* gamma,
                             float eps, int64_t T, int64_t H, int64_t Hu, uint16_t* res_out,
                             uint8_t* codes, uint8_t* e8, uint16_t* norm_out, hipStream_t s) {
  return launch_rmsnorm_mx_any<false>(hid, res, gamma, eps, T, H, Hu, res_out, codes, e8,
                                      norm_out, s);
}

hipError_t launch_rmsnorm_mx_staged(const uint16_t* hid, const uint16_t* res,
                                    const uint16_t* gamma, float eps, int64_t T, int64_t H,
                                    int64_t Hu, uint16_t* res_out, uint8_t* img, uint32_t* eimg,
                                    uint16_t* norm_out, hipStream_t s) {
  return launch_rmsnorm_mx_any<true>(hid, res, gamma, eps, T, H, Hu, res_out, img,
                                     reinterpret_cast<uint8_t*>(eimg), norm_out, s);
}

}  // namespace qkvmx
