// Pass 1 ([QKV-CTE] "Upstream behavior": O[S, I] = A[S, H] @ W[H, I] + bias; "Applies to /
// Pattern": every output tile accumulates over the whole contraction, then is dequantised,
// bias-added and stored; "Design 1)" step a: per-token sums of squares of the Q and K
// segments of the un-normalised output).
//
// gfx950 design
//  * Block tile 256 output channels x 256 tokens, 4 wavefronts (2 x 2), each 128 x 128 =
//    4 x 4 fragments of V_MFMA_SCALE_F32_32X32X64_F8F6F4 (fp32 accumulators, 256 per lane).
//  * Roles are swapped with respect to O = A W: the MFMA "A" operand is the weight (rows =
//    output channels, its E8M0 block exponents feed the MFMA's A-scale directly) and the "B"
//    operand is the ROW_MX activation (B-scale = 2^0; the fp32 row scale is applied in the
//    epilogue).  The accumulator then holds, per lane, 4-channel runs of one token, which the
//    epilogue stores as 8-byte bf16 vectors along the output row.
//  * K is staged through LDS 128 bytes at a time, double-buffered (2 x (32 + 32) KiB).  Rows are
//    stored as eight 16-byte chunks with chunk' = chunk ^ (row & 7), so the MFMA operand reads
//    (ds_read_b128, 8 lanes = 8 consecutive rows per phase) hit 8 distinct bank groups.
//  * Operand lane layout of the 32x32x64 MFMA (K = 64 bytes per row): lane group g = lane / 32
//    holds bytes [16g, 16g + 16) and [32 + 16g, 32 + 16g + 16) of row lane % 32; the exponent
//    of K-block b (32 bytes) of row m comes from lane m + 32 b, byte op_sel.
//  * Epilogue: x = acc * a_scale[token] * c[channel] + bias[channel] in fp32, sums of x^2 per
//    token over the Q and K columns (V excluded) written as one partial per 128 channels,
//    then bf16 round-to-nearest-even stores.  A second small kernel adds the partials in a
//    fixed order (deterministic, no atomics).
//  * Tile order: block ids are dealt round-robin to the 8 XCDs; they are remapped so that each
//    XCD owns a contiguous range of tiles, walked in groups of 8 token tiles x all channel tiles,
//    so the tiles resident on one XCD share activation rows and weight columns in its L2.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace qkvmx {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2_a8 __attribute__((ext_vector_type(2), aligned(8)));

constexpr int kThreads = 256;
constexpr int kRowBytes = kStageK;                 // 128 bytes of K per LDS row
constexpr int kOperandBytes = kTileM * kRowBytes;  // 32 KiB per operand per stage
constexpr int kGroupM = 8;                         // token tiles per raster group
constexpr int kXcds = 8;

struct ProjectArgs {
  const uint8_t* a_codes;
  int64_t a_stride;
  const uint8_t* a_scales;
  int64_t s_stride;
  const uint8_t* w_codes;      // [I][H]
  const uint32_t* w_scales;    // [I][S][2]
  const float* chan_scale;     // [I] or null
  const uint16_t* bias;        // [I] or null
  int64_t T, H, I, Iq, Ik;
  int64_t S;                   // supersteps of 256 K
  int tiles_m, tiles_n;
  uint16_t* out;
  float* ws;                   // [P][T][2] or null
};

__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ (row & 7)) << 4);
}

__global__ void __launch_bounds__(kThreads, 1) project_kernel(const ProjectArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kOperandBytes];  // [buf][W|X]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave & 1;        // channel half of the block tile
  const int wm = wave >> 1;       // token half

  // ---- tile id: XCD-contiguous ranges, grouped raster ----
  const int ntiles = a.tiles_m * a.tiles_n;
  const int b = blockIdx.x;
  const int xcd = b % kXcds, k_in = b / kXcds;
  const int per = ntiles / kXcds, rem = ntiles % kXcds;
  const int tile = xcd < rem ? xcd * (per + 1) + k_in : rem * (per + 1) + (xcd - rem) * per + k_in;
  const int group = tile / (kGroupM * a.tiles_n);
  const int first_m = group * kGroupM;
  const int gm = min(a.tiles_m - first_m, kGroupM);
  const int in_group = tile % (kGroupM * a.tiles_n);
  const int tm = first_m + in_group % gm;
  const int tn = in_group / gm;
  const int64_t m0 = (int64_t)tm * kTileM;
  const int64_t n0 = (int64_t)tn * kTileN;

  // ---- global -> LDS assignment: thread loads chunk c of rows r0 + 32 i (i = 0..7) ----
  // Row offsets are 32-bit (the host checks I * H and T * a_stride fit), rows past the end are
  // clamped to the last row (their results are never stored), K past H reads as zero.
  const int c_ld = tid & 7;
  const int r0 = tid >> 3;
  uint32_t woff[8], xoff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = r0 + 32 * i;
    const int64_t n = min(n0 + r, a.I - 1);
    const int64_t m = min(m0 + r, a.T - 1);
    woff[i] = (uint32_t)(n * a.H) + c_ld * 16;
    xoff[i] = (uint32_t)(m * a.a_stride) + c_ld * 16;
  }
  const int st_off = lds_off(r0, c_ld);   // + 4096 * i  (row + 32 keeps row & 7)

  uint4 wreg[8], xreg[8];
  auto gload = [&](int stage) {
    const uint32_t k0 = (uint32_t)stage * kStageK;
    const bool ok = (int64_t)k0 + c_ld * 16 < a.H;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (ok) {
        wreg[i] = *reinterpret_cast<const uint4*>(a.w_codes + (woff[i] + k0));
        const u32x4_a4 v = *reinterpret_cast<const u32x4_a4*>(a.a_codes + (xoff[i] + k0));
        xreg[i] = make_uint4(v.x, v.y, v.z, v.w);
      } else {
        wreg[i] = make_uint4(0, 0, 0, 0);
        xreg[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<uint4*>(&lds[buf][0][st_off + 4096 * i]) = wreg[i];
      *reinterpret_cast<uint4*>(&lds[buf][1][st_off + 4096 * i]) = xreg[i];
    }
  };

  // ---- per-lane exponent dwords for the 4 channel fragments ----
  const int g = lane >> 5;
  const uint32_t* scp[4];
#pragma unroll
  for (int cf = 0; cf < 4; ++cf) {
    int64_t n = n0 + wn * 128 + cf * 32 + (lane & 31);
    n = n < a.I ? n : a.I - 1;
    scp[cf] = a.w_scales + n * a.S * 2 + g;
  }
  uint32_t sc_cur[4], sc_nxt[4];
#pragma unroll
  for (int cf = 0; cf < 4; ++cf) sc_cur[cf] = scp[cf][0];

  v16f acc[4][4];
#pragma unroll
  for (int cf = 0; cf < 4; ++cf)
#pragma unroll
    for (int tf = 0; tf < 4; ++tf)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[cf][tf][r] = 0.0f;

  const int fr = lane & 31;           // fragment row of this lane
  const int w_row0 = wn * 128 + fr;   // + 32 cf
  const int x_row0 = wm * 128 + fr;   // + 32 tf

  // One LDS stage = 2 MFMA K-steps (kk); exponent byte = 2 * st + kk.
  auto compute = [&](auto st_c) {
    constexpr int st = decltype(st_c)::value;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      v8i wf[4], xf[4];
      const int c0 = 4 * kk + g, c1 = 4 * kk + 2 + g;
#pragma unroll
      for (int cf = 0; cf < 4; ++cf) {
        const int r = w_row0 + 32 * cf;
        const uint4 p0 = *reinterpret_cast<const uint4*>(&lds[st][0][lds_off(r, c0)]);
        const uint4 p1 = *reinterpret_cast<const uint4*>(&lds[st][0][lds_off(r, c1)]);
        wf[cf] = v8i{(int)p0.x, (int)p0.y, (int)p0.z, (int)p0.w,
                     (int)p1.x, (int)p1.y, (int)p1.z, (int)p1.w};
      }
#pragma unroll
      for (int tf = 0; tf < 4; ++tf) {
        const int r = x_row0 + 32 * tf;
        const uint4 p0 = *reinterpret_cast<const uint4*>(&lds[st][1][lds_off(r, c0)]);
        const uint4 p1 = *reinterpret_cast<const uint4*>(&lds[st][1][lds_off(r, c1)]);
        xf[tf] = v8i{(int)p0.x, (int)p0.y, (int)p0.z, (int)p0.w,
                     (int)p1.x, (int)p1.y, (int)p1.z, (int)p1.w};
      }
#pragma unroll
      for (int cf = 0; cf < 4; ++cf)
#pragma unroll
        for (int tf = 0; tf < 4; ++tf) {
          if (kk == 0)
            acc[cf][tf] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                wf[cf], xf[tf], acc[cf][tf], 0, 0, 2 * st, (int)sc_cur[cf], 0, 0x7F7F7F7F);
          else
            acc[cf][tf] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                wf[cf], xf[tf], acc[cf][tf], 0, 0, 2 * st + 1, (int)sc_cur[cf], 0, 0x7F7F7F7F);
        }
    }
  };

  // ---- main loop over 256-K supersteps (2 LDS stages each) ----
  const int nstages = (int)(2 * a.S);
  gload(0);
  lstore(0);
  __syncthreads();
  for (int64_t s = 0; s < a.S; ++s) {
    // stage 2s (buffer 0)
    if (2 * s + 1 < nstages) gload((int)(2 * s + 1));
    if (s + 1 < a.S) {
#pragma unroll
      for (int cf = 0; cf < 4; ++cf) sc_nxt[cf] = scp[cf][(s + 1) * 2];
    }
    compute(std::integral_constant<int, 0>{});
    if (2 * s + 1 < nstages) lstore(1);
    __syncthreads();
    // stage 2s + 1 (buffer 1)
    if (2 * s + 2 < nstages) gload((int)(2 * s + 2));
    compute(std::integral_constant<int, 1>{});
    if (2 * s + 2 < nstages) lstore(0);
    __syncthreads();
    if (s + 1 < a.S) {
#pragma unroll
      for (int cf = 0; cf < 4; ++cf) sc_cur[cf] = sc_nxt[cf];
    }
  }

  // ---- epilogue ----
  float sA[4];
  int64_t tok[4];
#pragma unroll
  for (int tf = 0; tf < 4; ++tf) {
    tok[tf] = m0 + wm * 128 + tf * 32 + fr;
    const int64_t t = tok[tf] < a.T ? tok[tf] : a.T - 1;
    sA[tf] = *reinterpret_cast<const float*>(a.a_scales + t * a.s_stride);
  }
  float sq_q[4] = {0.f, 0.f, 0.f, 0.f}, sq_k[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int cf = 0; cf < 4; ++cf) {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int64_t n = n0 + wn * 128 + cf * 32 + rq * 8 + g * 4;   // 4 consecutive channels
      if (n >= a.I) continue;
      float cs[4] = {1.f, 1.f, 1.f, 1.f}, bs[4] = {0.f, 0.f, 0.f, 0.f};
      if (a.chan_scale) {
        const float4 v = *reinterpret_cast<const float4*>(a.chan_scale + n);
        cs[0] = v.x; cs[1] = v.y; cs[2] = v.z; cs[3] = v.w;
      }
      if (a.bias) {
        const u32x2_a8 v = *reinterpret_cast<const u32x2_a8*>(a.bias + n);
        bs[0] = bf16_to_f32(v.x & 0xFFFFu); bs[1] = bf16_to_f32(v.x >> 16);
        bs[2] = bf16_to_f32(v.y & 0xFFFFu); bs[3] = bf16_to_f32(v.y >> 16);
      }
      const bool in_q = n < a.Iq;
      const bool in_k = !in_q && n < a.Iq + a.Ik;
#pragma unroll
      for (int tf = 0; tf < 4; ++tf) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[cf][tf][rq * 4 + e] * sA[tf] * cs[e] + bs[e];
        const float s2 = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
        if (in_q) sq_q[tf] += s2;
        if (in_k) sq_k[tf] += s2;
        if (tok[tf] < a.T) {
          u32x2_a8 o = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
          *reinterpret_cast<u32x2_a8*>(a.out + tok[tf] * a.I + n) = o;
        }
      }
    }
  }
  if (a.ws) {
    const int64_t p = (int64_t)tn * 2 + wn;
#pragma unroll
    for (int tf = 0; tf < 4; ++tf) {
      const float q = sq_q[tf] + __shfl_xor(sq_q[tf], 32);
      const float k = sq_k[tf] + __shfl_xor(sq_k[tf], 32);
      if (g == 0 && tok[tf] < a.T) {
        u32x2_a8 o = {__float_as_uint(q), __float_as_uint(k)};
        *reinterpret_cast<u32x2_a8*>(a.ws + (p * a.T + tok[tf]) * 2) = o;
      }
    }
  }
}

// ssq[t] = sum over partials p of ws[p][t] (fixed order).
__global__ void __launch_bounds__(256) ssq_reduce_kernel(const float* __restrict__ ws, int64_t P,
                                                         int64_t T, float* __restrict__ ssq) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  float q = 0.f, k = 0.f;
  for (int64_t p = 0; p < P; ++p) {
    const float2 v = reinterpret_cast<const float2*>(ws)[p * T + t];
    q += v.x;
    k += v.y;
  }
  reinterpret_cast<float2*>(ssq)[t] = make_float2(q, k);
}

}  // namespace

hipError_t launch_project(const uint8_t* a_codes, int64_t a_stride, const uint8_t* a_scales,
                          int64_t s_stride, const uint8_t* w_packed, const float* chan_scale,
                          const uint16_t* bias, int64_t T, int64_t H, int64_t I, int64_t Iq,
                          int64_t Ik, uint16_t* out, float* ssq, float* ws, hipStream_t s) {
  ProjectArgs a;
  a.a_codes = a_codes; a.a_stride = a_stride; a.a_scales = a_scales; a.s_stride = s_stride;
  a.w_codes = w_packed;
  a.w_scales = reinterpret_cast<const uint32_t*>(w_packed + packed_scales_offset(H, I));
  a.chan_scale = chan_scale; a.bias = bias;
  a.T = T; a.H = H; a.I = I; a.Iq = Iq; a.Ik = Ik;
  a.S = ceil_div(H, kSuperK);
  a.tiles_m = (int)ceil_div(T, kTileM);
  a.tiles_n = (int)ceil_div(I, kTileN);
  a.out = out;
  a.ws = ssq ? ws : nullptr;
  const unsigned nblocks = (unsigned)(a.tiles_m * a.tiles_n);
  hipLaunchKernelGGL(project_kernel, dim3(nblocks), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !ssq) return e;
  const int64_t P = ssq_partials(I);
  hipLaunchKernelGGL(ssq_reduce_kernel, dim3((unsigned)ceil_div(T, 256)), dim3(256), 0, s, ws, P,
                     T, ssq);
  return hipGetLastError();
}

}  // namespace qkvmx
