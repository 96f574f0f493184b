// Pass 2 ([QKV-CTE] "Design 1)" steps b-c, "Design 2)", "Design 5)"): across-heads RMSNorm and
// rotate-half RoPE applied in place to the Q and K columns of the bf16 [T, I] projection; V is
// never read or written.  HBM-bound: per token 4 * (Iq + Ik) bytes of Q/K plus the token's
// cos/sin rows (8 * d bytes) and its two sums; gamma is shared by all tokens and stays cached.
//
// Work unit = (segment, head, 8-lane chunk j0): the thread loads lanes j0..j0+7 and their
// rotate-half partners j0+d/2.. as two 16-byte vectors, so the 8 threads of a head read
// 2 x 128 contiguous bytes for d = 128.  The per-token inv_rms is computed once per thread
// from the token's sums and folded into the gamma multiply, as the pages fold it into cos/sin.
#include "device_common.h"
#include "internal.h"

namespace qkvmx {

namespace {

struct NormRopeArgs {
  uint16_t* qkv;
  const float* ssq;
  const uint16_t* gq;
  const uint16_t* gk;
  const float* cos_tab;
  const float* sin_tab;
  int64_t T;
  int64_t I;
  int nq, nkv, d;
  int units_q;       // active Q units per token (0 if the Q segment is untouched)
  int units;         // active units per token
  int blocks_per_token;
  float eps;
  bool norm_q, norm_k, rope;
};

__device__ __forceinline__ void unpack8(const uint4 v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = bf16_to_f32(w[e] & 0xFFFFu);
    f[2 * e + 1] = bf16_to_f32(w[e] >> 16);
  }
}

__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

__device__ __forceinline__ void load8f(const float* p, float (&f)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

__global__ void __launch_bounds__(1024) norm_rope_kernel(const NormRopeArgs a) {
  const int64_t token = blockIdx.x / a.blocks_per_token;
  const int u = (blockIdx.x % a.blocks_per_token) * blockDim.x + threadIdx.x;
  if (u >= a.units) return;
  const int cpd = a.d / 16;                 // chunks per head
  const bool is_k = u >= a.units_q;
  const int uu = is_k ? u - a.units_q : u;
  const int head = uu / cpd;
  const int j0 = (uu % cpd) * 8;
  const int half = a.d / 2;
  const int64_t seg_off = is_k ? (int64_t)a.nq * a.d : 0;
  uint16_t* base = a.qkv + token * a.I + seg_off + (int64_t)head * a.d;

  float lo[8], hi[8];
  unpack8(*reinterpret_cast<const uint4*>(base + j0), lo);
  unpack8(*reinterpret_cast<const uint4*>(base + half + j0), hi);

  const bool norm = is_k ? a.norm_k : a.norm_q;
  if (norm) {
    const int n = is_k ? a.nkv : a.nq;
    const float ss = a.ssq[token * 2 + (is_k ? 1 : 0)];
    const float r = 1.0f / sqrtf(ss / (float)(n * a.d) + a.eps);
    const uint16_t* g = (is_k ? a.gk : a.gq) + (int64_t)head * a.d;
    float glo[8], ghi[8];
    unpack8(*reinterpret_cast<const uint4*>(g + j0), glo);
    unpack8(*reinterpret_cast<const uint4*>(g + half + j0), ghi);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      lo[e] = lo[e] * (glo[e] * r);
      hi[e] = hi[e] * (ghi[e] * r);
    }
  }
  if (a.rope) {
    const float* cr = a.cos_tab + token * a.d;
    const float* sr = a.sin_tab + token * a.d;
    float clo[8], chi[8], slo[8], shi[8];
    load8f(cr + j0, clo);
    load8f(cr + half + j0, chi);
    load8f(sr + j0, slo);
    load8f(sr + half + j0, shi);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float ol = lo[e] * clo[e] - hi[e] * slo[e];
      const float oh = hi[e] * chi[e] + lo[e] * shi[e];
      lo[e] = ol;
      hi[e] = oh;
    }
  }
  *reinterpret_cast<uint4*>(base + j0) = pack8(lo);
  *reinterpret_cast<uint4*>(base + half + j0) = pack8(hi);
}

}  // namespace

hipError_t launch_norm_rope(uint16_t* qkv, const float* ssq, const uint16_t* q_gamma,
                            const uint16_t* k_gamma, const float* cos_tab, const float* sin_tab,
                            int64_t T, int nq, int nkv, int d, float eps, uint32_t flags,
                            hipStream_t s) {
  NormRopeArgs a;
  a.qkv = qkv; a.ssq = ssq; a.gq = q_gamma; a.gk = k_gamma; a.cos_tab = cos_tab;
  a.sin_tab = sin_tab; a.T = T; a.I = (int64_t)(nq + 2 * nkv) * d;
  a.nq = nq; a.nkv = nkv; a.d = d; a.eps = eps;
  a.norm_q = flags & 1u; a.norm_k = (flags & 2u) && nkv > 0; a.rope = flags & 4u;
  const int cpd = d / 16;
  const bool q_on = a.norm_q || a.rope;
  const bool k_on = nkv > 0 && (a.norm_k || a.rope);
  a.units_q = q_on ? nq * cpd : 0;
  a.units = a.units_q + (k_on ? nkv * cpd : 0);
  if (a.units == 0 || T == 0) return hipSuccess;       // nothing to do
  if (!q_on) {
    // only K is touched: shift the K segment to unit 0 by treating it as "K" from the start
    a.units_q = 0;
  }
  int bpt = (int)ceil_div(a.units, 512);
  int block = (int)ceil_div(ceil_div(a.units, bpt), 64) * 64;
  a.blocks_per_token = bpt;
  hipLaunchKernelGGL(norm_rope_kernel, dim3((unsigned)(T * bpt)), dim3(block), 0, s, a);
  return hipGetLastError();
}

}  // namespace qkvmx
